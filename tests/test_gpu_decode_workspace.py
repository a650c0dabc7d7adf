"""The decode workspace and the merge of the split partial results.

fa_decode writes each chunk's normalised partial output and log-sum-exp to
the caller's workspace, and a second kernel merges them per head.  The cases
here check that
- the workspace's contents on entry do not matter: zeros, all-ones bytes
  (NaN in fp32), random bytes, and the partials that earlier calls left, on
  the same shape or another, all give the oracle's result within tolerance
  and the same bits every time;
- split counts around the merge's unrolled loop (four rows in flight per
  group of threads, then a tail) merge every chunk exactly once;
- many heads merged at once stay independent and deterministic;
- with one split per head (chosen automatically once B*H fills the chip)
  the split kernel's own result is the oracle's.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import check, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu


def _case(seed, B, H, Nkv, d, dtype):
    rng = np.random.default_rng(seed)
    q = rand_bits(rng, (B, H, 1, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    return q, k, v


def _decode_into(tq, tk, tv, B, H, Nkv, d, dtype, splits, ws):
    o = torch.empty(B, H, d, dtype=torch.float32, device=tq.device)
    lse = torch.empty(B, H, dtype=torch.float32, device=tq.device)
    code = fa.FA_F16 if dtype == "f16" else fa.FA_BF16
    fa.fa_decode(tq[:, :, 0], tk, tv, o, lse, B, H, Nkv, d, 1 / np.sqrt(d), code | fa.FA_OUT_F32, splits, ws,
                 ws.numel(), torch.cuda.current_stream().cuda_stream)
    return o, lse


@pytest.mark.parametrize("splits", [5, 0])
def test_workspace_contents_ignored(splits):
    B, H, Nkv, d, dtype = 2, 3, 3000, 128, "f16"
    q, k, v = _case(7, B, H, Nkv, d, dtype)
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))), dtype=dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    need = fa.fa_decode_workspace_size(B, H, Nkv, d, splits)
    ws = torch.empty(need, dtype=torch.uint8, device=tq.device)
    gen = torch.Generator(device="cpu").manual_seed(3)
    fills = [("zeros", lambda: ws.zero_()), ("all-ones bytes", lambda: ws.fill_(255)),
             ("random bytes", lambda: ws.copy_(torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8))),
             ("an earlier call's partials", lambda: None), ("an earlier call's partials", lambda: None)]
    first = None
    for name, fill in fills:
        fill()
        say(f"fa_decode B{B}H{H}k{Nkv} splits={splits}, workspace holding {name}")
        o, lse = _decode_into(tq, tk, tv, B, H, Nkv, d, dtype, splits, ws)
        torch.cuda.synchronize()
        o, lse = to_np(o), to_np(lse)
        check(o[:, :, None], lse[..., None], o_ref, lse_ref, dtype, f"decode, workspace holding {name}")
        if first is None:
            first = (o, lse)
        assert np.array_equal(o, first[0]) and np.array_equal(lse, first[1]), name


def test_workspace_left_by_other_shapes():
    # one workspace, calls of different shapes: each call's partial LSEs sit
    # where an earlier call kept partial outputs, and the reverse
    d, dtype = 64, "bf16"
    shapes = [(1, 4, 2000, 9), (2, 2, 700, 3), (1, 4, 2000, 9), (1, 1, 4095, 64), (2, 2, 700, 3)]
    cap = max(fa.fa_decode_workspace_size(B, H, N, d, s) for B, H, N, s in shapes)
    ws = torch.full((cap,), 255, dtype=torch.uint8, device="cuda")
    results = {}
    for i, (B, H, Nkv, splits) in enumerate(shapes):
        q, k, v = _case(100 + Nkv, B, H, Nkv, d, dtype)
        tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
        say(f"fa_decode B{B}H{H}k{Nkv} splits={splits} in a shared workspace, call {i}")
        o, lse = _decode_into(tq, tk, tv, B, H, Nkv, d, dtype, splits, ws)
        torch.cuda.synchronize()
        o, lse = to_np(o), to_np(lse)
        o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))),
                                          dtype=dtype)
        check(o[:, :, None], lse[..., None], o_ref, lse_ref, dtype, f"decode {B, H, Nkv, splits}")
        key = (B, H, Nkv, splits)
        if key in results:
            assert np.array_equal(results[key][0], o) and np.array_equal(results[key][1], lse)
        results[key] = (o, lse)


# Nkv = 16 S - 5 keys in S requested splits gives chunks of 16 and exactly S
# splits, the last one ragged
@pytest.mark.parametrize("S", [2, 63, 64, 65, 255, 256, 257, 300])
def test_merge_split_counts(S):
    B, H, d, dtype = 1, 2, 64, "bf16"
    Nkv = 16 * S - 5
    assert fa.fa_decode_workspace_size(B, H, Nkv, d, S) == B * H * S * (d + 1) * 4
    q, k, v = _case(S, B, H, Nkv, d, dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, Nkv, d, S), dtype=torch.uint8, device=tq.device)
    say(f"fa_decode with {S} splits of 16 keys")
    o, lse = _decode_into(tq, tk, tv, B, H, Nkv, d, dtype, S, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))), dtype=dtype)
    check(to_np(o)[:, :, None], to_np(lse)[..., None], o_ref, lse_ref, dtype, f"decode S={S}")


def test_many_heads_merge_at_once():
    # 1024 heads of 4 short chunks, merged by 1024 workgroups at once
    B, H, Nkv, d, dtype = 16, 64, 256, 128, "f16"
    q, k, v = _case(11, B, H, Nkv, d, dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, Nkv, d, 4), dtype=torch.uint8, device=tq.device)
    say("fa_decode 16 x 64 heads x 256 keys, 4 splits, 3 calls")
    outs = []
    for _ in range(3):
        o, lse = _decode_into(tq, tk, tv, B, H, Nkv, d, dtype, 4, ws)
        outs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))), dtype=dtype)
    check(to_np(outs[0][0])[:, :, None], to_np(outs[0][1])[..., None], o_ref, lse_ref, dtype, "decode 1024 heads")
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    # the 16-bit output is the fp32 one rounded
    o16, _ = fa.decode(tq[:, :, 0].contiguous(), tk, tv, scale=1 / np.sqrt(d), num_splits=4)
    torch.cuda.synchronize()
    assert np.array_equal(fi.torch_to_bits(o16.cpu()), fi.f32_to_bits(to_np(outs[0][0]).astype(np.float32), dtype))


def test_automatic_single_split():
    # 2048 heads fill the chip with one workgroup each: the automatic split
    # count is 1, and the split kernel writes O and LSE itself
    B, H, Nkv, d, dtype = 32, 64, 300, 64, "f16"
    assert fa.fa_decode_num_splits(B, H, Nkv, d) == 1
    q, k, v = _case(12, B, H, Nkv, d, dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    say("fa_decode 32 x 64 heads x 300 keys, automatic split count (1)")
    o, lse = fa.decode(tq[:, :, 0].contiguous(), tk, tv, scale=1 / np.sqrt(d), out_dtype=torch.float32)
    o16, lse16 = fa.decode(tq[:, :, 0].contiguous(), tk, tv, scale=1 / np.sqrt(d))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))), dtype=dtype)
    check(to_np(o)[:, :, None], to_np(lse)[..., None], o_ref, lse_ref, dtype, "decode, one split per head")
    assert torch.equal(lse16, lse)
    assert np.array_equal(fi.torch_to_bits(o16.cpu()), fi.f32_to_bits(to_np(o).astype(np.float32), dtype))
