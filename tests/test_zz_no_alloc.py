"""fa_decode_noalloc: decode with the split partials in the library's device scratch.

The entry point is fa_decode for callers that cannot allocate device memory.
It runs the same kernels with the same split rule, so for the same arguments
its outputs must equal fa_decode's bit for bit (and so stay within the
oracle's tolerance).  Two calls in a row on one stream, the second with a
smaller input, check that the scratch left by a larger call does not leak
into a smaller one; a call with one split per head needs no scratch at all.
(Calls whose partials exceed the scratch are rejected on the host; the CPU
ABI tests cover that.)
"""
import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import oracle
from gpu_util import check, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, Nkv, d, dtype):
    rng = np.random.default_rng(seed)
    return (rand_bits(rng, (B, H, 1, d), dtype), rand_bits(rng, (B, H, Nkv, d), dtype),
            rand_bits(rng, (B, H, Nkv, d), dtype))


def _run(noalloc, tq, tk, tv, B, H, Nkv, d, dtype, splits, out_f32):
    code = (fa.FA_F16 if dtype == "f16" else fa.FA_BF16) | (fa.FA_OUT_F32 if out_f32 else 0)
    o = torch.full((B, H, d), float("nan"), dtype=torch.float32 if out_f32 else tq.dtype, device=tq.device)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=tq.device)
    stream = torch.cuda.current_stream().cuda_stream
    scale = 1 / np.sqrt(d)
    if noalloc:
        fa.fa_decode_noalloc(tq[:, :, 0], tk, tv, o, lse, B, H, Nkv, d, scale, code, splits, stream)
    else:
        need = fa.fa_decode_workspace_size(B, H, Nkv, d, splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=tq.device)
        fa.fa_decode(tq[:, :, 0], tk, tv, o, lse, B, H, Nkv, d, scale, code, splits, ws, need, stream)
    return o, lse


@pytest.mark.parametrize("dtype,d,splits", [("f16", 128, 0), ("bf16", 64, 7), ("f16", 64, 0)])
def test_noalloc_matches_decode_twice_then_smaller(dtype, d, splits):
    # the first call fills more of the scratch than the second reads
    shapes = [(4, 8, 5000), (4, 8, 5000), (2, 3, 1111)]
    for i, (B, H, Nkv) in enumerate(shapes):
        q, k, v = _inputs(40 + i, B, H, Nkv, d, dtype)
        tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
        say(f"fa_decode_noalloc call {i}: B{B} H{H} Nkv{Nkv} d{d} {dtype} splits={splits}")
        o_n, lse_n = _run(True, tq, tk, tv, B, H, Nkv, d, dtype, splits, out_f32=True)
        o_w, lse_w = _run(False, tq, tk, tv, B, H, Nkv, d, dtype, splits, out_f32=True)
        torch.cuda.synchronize()
        o_n, lse_n, o_w, lse_w = to_np(o_n), to_np(lse_n), to_np(o_w), to_np(lse_w)
        assert np.array_equal(o_n, o_w) and np.array_equal(lse_n, lse_w), f"call {i}: differs from fa_decode"
        o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=float(np.float32(1 / np.sqrt(d))),
                                          dtype=dtype)
        check(o_n[:, :, None], lse_n[..., None], o_ref, lse_ref, dtype, f"noalloc call {i}")


def test_noalloc_native_output_and_one_split():
    # 16-bit O, and a call with one split per head (no scratch used) between
    # two split calls
    dtype, d = "f16", 128
    for i, (B, H, Nkv, splits) in enumerate([(2, 4, 3000, 6), (3, 2, 900, 1), (1, 2, 700, 3)]):
        q, k, v = _inputs(60 + i, B, H, Nkv, d, dtype)
        tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
        say(f"fa_decode_noalloc native O: B{B} H{H} Nkv{Nkv} splits={splits}")
        o_n, lse_n = _run(True, tq, tk, tv, B, H, Nkv, d, dtype, splits, out_f32=False)
        o_w, lse_w = _run(False, tq, tk, tv, B, H, Nkv, d, dtype, splits, out_f32=False)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_w) and torch.equal(lse_n, lse_w)

