"""GPU parity: libfa355 against the fp64 oracle, through the C ABI.

Small and ragged shapes are compared element by element, and so are the
full-size workloads the benchmark times (in its launch configuration), with
the oracle run one head at a time; larger and rectangular shapes are compared
on sampled rows that the oracle computes one at a time, plus properties that
hold at any size.  Every case prints its name before it touches the GPU.
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import TOL_LSE, TOL_O, check, device, max_err, rand_bits, run_fwd, say, to_np, upload

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# small workloads, every element

@pytest.mark.parametrize("name", ["tiny_256_d64", "prefill_2k_d64"])
def test_small_workload_elementwise(name):
    w = fi.WORKLOADS[name]
    say(f"fa_fwd {name} B={w.B} H={w.H} N={w.Nq} d={w.d} {w.dtype} causal={w.causal} seed={w.seed}")
    x = fi.make_inputs(w)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, dtype=w.dtype)
    o, lse = run_fwd(x["q"], x["k"], x["v"], w.causal, w.scale, w.dtype, out_f32=True)
    check(o, lse, o_ref, lse_ref, w.dtype, name)


RAGGED = [
    # B, H, Nq, Nkv, d, causal, dtype
    (1, 1, 1, 1, 64, False, "f16"),
    (1, 1, 1, 1, 128, True, "bf16"),
    (1, 2, 37, 37, 64, True, "f16"),
    (2, 1, 130, 200, 128, True, "f16"),
    (1, 1, 129, 129, 128, True, "bf16"),
    (1, 1, 100, 1000, 64, False, "bf16"),
    (1, 3, 1, 300, 128, False, "f16"),
    (1, 1, 255, 257, 64, True, "f16"),
    (2, 2, 200, 64, 128, False, "f16"),
    (1, 1, 384, 384, 128, True, "f16"),
    (1, 1, 64, 65, 64, True, "bf16"),
    (1, 2, 513, 1100, 128, True, "bf16"),
    (3, 1, 96, 96, 64, False, "f16"),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_ragged_shapes(case):
    B, H, Nq, Nkv, d, causal, dtype = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q = rand_bits(rng, (B, H, Nq, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"fa_fwd ragged {case}")
    o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, scale=scale, dtype=dtype)
    o, lse = run_fwd(q, k, v, causal, scale, dtype, out_f32=True)
    check(o, lse, o_ref, lse_ref, dtype, f"ragged {case}")
    o16, lse16 = run_fwd(q, k, v, causal, scale, dtype, out_f32=False)
    # the native-type output is the fp32 result rounded to nearest even
    rounded = fi.f32_to_bits(o.astype(np.float32), dtype)
    assert np.array_equal(fi.f32_to_bits(o16.astype(np.float32), dtype), rounded)
    assert np.array_equal(lse16, lse)


# Grids large enough for the 8-wave launch shape (256 rows per workgroup):
# ragged query and key counts, waves wholly past Nq, Nq < Nkv.
WIDE = [
    # B, H, Nq, Nkv, d, causal, dtype
    (1, 256, 300, 300, 128, True, "f16"),
    (2, 128, 257, 500, 64, True, "bf16"),
    (4, 64, 130, 130, 128, False, "bf16"),
    (1, 256, 513, 513, 64, True, "f16"),
    (2, 128, 260, 333, 128, False, "f16"),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_wide_grid_shapes(case):
    test_ragged_shapes(case)


@pytest.mark.parametrize("scale", [0.0, -0.11, 0.7])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_scale_values(scale, dtype):
    # zero scale: uniform weights over the visible keys; negative scale: the
    # kernel negates Q and uses |scale|; both against the oracle, causal with Nq < Nkv
    rng = np.random.default_rng(6)
    B, H, Nq, Nkv, d = 1, 2, 150, 230, 128
    q = rand_bits(rng, (B, H, Nq, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    say(f"fa_fwd scale={scale} {dtype}")
    o_ref, lse_ref = oracle.attention(q, k, v, causal=True, scale=scale, dtype=dtype)
    o, lse = run_fwd(q, k, v, True, scale, dtype)
    check(o, lse, o_ref, lse_ref, dtype, f"scale={scale} {dtype}")


# ---------------------------------------------------------------------------
# invariants with exact answers

def _fwd_native(q, k, v, causal, scale, dtype):
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0_exactly(dtype, d):
    rng = np.random.default_rng(1)
    q, k, v = (rand_bits(rng, (1, 2, 300, d), dtype) for _ in range(3))
    say(f"fa_fwd causal row 0 d={d} {dtype}")
    o, lse = _fwd_native(q, k, v, True, 0.1, dtype)
    assert np.array_equal(fi.torch_to_bits(o[:, :, 0]), v[:, :, 0])
    s00 = 0.1 * np.einsum("bhd,bhd->bh", oracle.widen(q[:, :, 0], dtype), oracle.widen(k[:, :, 0], dtype))
    assert np.max(np.abs(lse[:, :, 0].numpy() - s00)) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dominant_key_selects_its_row_exactly(dtype):
    # every query equals 4 * e_0 and key 77 equals 32 * e_0: its score beats
    # the others (|q.k| <= 4 * 4) by more than 100, so O is V[77] bit for bit.
    rng = np.random.default_rng(2)
    d, N = 128, 200
    q = np.zeros((1, 1, N, d), np.float32)
    q[..., 0] = 4.0
    k = np.clip(rng.standard_normal((1, 1, N, d)), -4, 4).astype(np.float32)
    k[0, 0, 77] = 0.0
    k[0, 0, 77, 0] = 32.0
    v = rand_bits(rng, (1, 1, N, d), dtype)
    say(f"fa_fwd dominant key {dtype}")
    o, _ = _fwd_native(fi.f32_to_bits(q, dtype), fi.f32_to_bits(k, dtype), v, False, 1.0, dtype)
    assert np.array_equal(fi.torch_to_bits(o[0, 0]), np.broadcast_to(v[0, 0, 77], (N, d)))


def test_constant_v_and_zero_q():
    rng = np.random.default_rng(3)
    d, N = 128, 333
    q = rand_bits(rng, (1, 2, N, d), "f16", sigma=2.0)
    k = rand_bits(rng, (1, 2, N, d), "f16", sigma=2.0)
    c = rand_bits(rng, (d,), "f16")
    v = np.broadcast_to(c, (1, 2, N, d)).copy()
    say("fa_fwd constant V")
    o, _ = run_fwd(q, k, v, True, 0.125, "f16")
    assert max_err(o, np.broadcast_to(oracle.widen(c, "f16"), o.shape))[0] <= TOL_O["f16"]
    say("fa_fwd zero Q")
    z = np.zeros_like(q)
    v2 = rand_bits(rng, (1, 2, N, d), "f16")
    o, lse = run_fwd(z, k, v2, True, 0.125, "f16")
    vv = oracle.widen(v2, "f16")
    mean = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert max_err(o, mean)[0] <= TOL_O["f16"]
    assert max_err(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape))[0] <= TOL_LSE


def test_deterministic_and_heads_independent():
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 3, 300, 128
    q, k, v = (rand_bits(rng, (B, H, N, d), "bf16") for _ in range(3))
    say("fa_fwd determinism")
    o1, l1 = run_fwd(q, k, v, True, 0.09, "bf16")
    o2, l2 = run_fwd(q, k, v, True, 0.09, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    say("fa_fwd head independence")
    oh, lh = run_fwd(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], True, 0.09, "bf16")
    assert np.array_equal(oh[0, 0], o1[1, 2]) and np.array_equal(lh[0, 0], l1[1, 2])


def test_fwd_allocates_no_device_memory():
    rng = np.random.default_rng(5)
    q, k, v = (upload(rand_bits(rng, (1, 8, 2048, 128), "f16"), "f16") for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, 2048), dtype=torch.float32, device=q.device)
    say("fa_fwd memory footprint")
    fa.fa_fwd(q, k, v, o, lse, 1, 8, 2048, 2048, 128, 1, 0.088, fa.FA_F16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        fa.fa_fwd(q, k, v, o, lse, 1, 8, 2048, 2048, 128, 1, 0.088, fa.FA_F16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


# ---------------------------------------------------------------------------
# decode

DECODE = [
    # B, H, Nkv, d, dtype
    (2, 4, 5000, 128, "f16"),
    (1, 2, 777, 64, "bf16"),
    (3, 1, 1, 128, "bf16"),
    (1, 1, 33, 64, "f16"),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}H{}k{}d{}{}".format(*c))
def test_decode_every_split_count(case):
    B, H, Nkv, d, dtype = case
    rng = np.random.default_rng(Nkv)
    q = rand_bits(rng, (B, H, 1, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=scale, dtype=dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    outs = []
    for splits in (1, 2, 3, 7, 16, 0):
        say(f"fa_decode {case} splits={splits}")
        o, lse = fa.decode(tq, tk, tv, scale=scale, num_splits=splits, out_dtype=torch.float32)
        torch.cuda.synchronize()
        o, lse = to_np(o), to_np(lse)
        check(o, lse[..., None], o_ref, lse_ref, dtype, f"decode {case} splits={splits}")
        outs.append(o)
        o16, _ = fa.decode(tq, tk, tv, scale=scale, num_splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(fi.torch_to_bits(o16.cpu()), fi.f32_to_bits(o.astype(np.float32), dtype))
    for o in outs[1:]:
        assert max_err(o, outs[0])[0] <= TOL_O[dtype]


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows, in the benchmark's launch configuration

def _sample_rows(N, rng, extra=()):
    base = {0, 1, 31, 32, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 1, *extra}
    base |= set(int(i) for i in rng.integers(0, N, 24))
    return np.array(sorted(i for i in base if 0 <= i < N))


@pytest.mark.parametrize("name", ["prefill_8k_d128", "prefill_16k_d128_bf16"])
def test_full_size_prefill_every_element(name):
    # every element of O and LSE of every head, against the oracle run one
    # head at a time (one head's score matrix at a time in host memory)
    w = fi.WORKLOADS[name]
    say(f"generate {name}")
    x = fi.make_inputs(w)
    tq, tk, tv = upload(x["q"], w.dtype), upload(x["k"], w.dtype), upload(x["v"], w.dtype)
    say(f"fa_fwd {name} native O (benchmark configuration)")
    o16, lse16 = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    say(f"fa_fwd {name} fp32 O")
    o32, lse32 = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the native O is the rounded fp32 O, so its parity follows from the fp32 O's
    assert torch.equal(o16, o32.to(o16.dtype)) and torch.equal(lse16, lse32)
    worst_o = worst_l = (0.0, None)
    for bh in range(w.heads):
        b, h = divmod(bh, w.H)
        o_ref, lse_ref = oracle.attention(x["q"][b, h], x["k"][b, h], x["v"][b, h], causal=w.causal, scale=w.scale,
                                          dtype=w.dtype)
        eo, el = check(to_np(o32[b, h]), to_np(lse32[b, h]), o_ref, lse_ref, w.dtype,
                       f"{name} head {bh}: all {w.Nq} rows")
        worst_o, worst_l = max(worst_o, (eo, bh)), max(worst_l, (el, bh))
    say(f"{name}: every element of {w.heads} heads within tolerance; worst err_O {worst_o[0]:.3e} (head "
        f"{worst_o[1]}), worst err_LSE {worst_l[0]:.3e} (head {worst_l[1]})")


WIDE_RECT = [
    # B, H, Nq, Nkv, d, dtype: causal with Nq < Nkv (bottom-right) on grids that
    # select the 8-wave shape for 16-bit K and the 4-wave shape for E4M3 K
    (1, 64, 1500, 5000, 128, "f16"),
    (1, 128, 777, 3333, 64, "bf16"),
]


@pytest.mark.parametrize("case", WIDE_RECT, ids=lambda c: "B{}H{}q{}k{}d{}{}".format(*c))
def test_wide_causal_rectangular_sampled(case):
    B, H, Nq, Nkv, d, dtype = case
    rng = np.random.default_rng(Nq * Nkv)
    q = rand_bits(rng, (B, H, Nq, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    say(f"fa_fwd and fa_fwd_fp8 causal rectangular {case}")
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=scale, out_dtype=torch.float32)
    o8, lse8 = fa.fwd_fp8(tq, tk, tv, causal=True, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse, o8, lse8 = to_np(o), to_np(lse), to_np(o8), to_np(lse8)
    for bh in sorted({0, B * H // 2, B * H - 1}):
        b, h = divmod(bh, H)
        rows = _sample_rows(Nq, rng)
        o_ref, lse_ref = oracle.attention_rows(q[b, h], k[b, h], v[b, h], rows, causal=True, scale=scale, dtype=dtype)
        check(o[b, h][rows], lse[b, h][rows], o_ref, lse_ref, dtype, f"fwd {case} head {bh}")
        o_ref, lse_ref = oracle.attention_fp8qk_rows(q[b, h], k[b, h], v[b, h], rows, causal=True, scale=scale,
                                                     dtype=dtype)
        check(o8[b, h][rows], lse8[b, h][rows], o_ref, lse_ref, dtype, f"fwd_fp8 {case} head {bh}")


def test_full_size_decode_every_head():
    # all 512 heads, against the oracle run one head at a time
    w = fi.WORKLOADS["decode_32k_d128"]
    say("generate decode_32k_d128")
    x = fi.make_inputs(w)
    tq, tk, tv = upload(x["q"], w.dtype), upload(x["k"], w.dtype), upload(x["v"], w.dtype)
    say("fa_decode decode_32k_d128 native O (benchmark configuration)")
    o16, lse16 = fa.decode(tq, tk, tv, scale=w.scale)
    say("fa_decode decode_32k_d128 fp32 O")
    o32, lse32 = fa.decode(tq, tk, tv, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(o16.dtype)) and torch.equal(lse16, lse32)
    o_all, lse_all = to_np(o32), to_np(lse32)
    o_ref = np.empty_like(o_all)
    lse_ref = np.empty_like(lse_all)
    for bh in range(w.heads):
        b, h = divmod(bh, w.H)
        if bh % 64 == 0:
            say(f"oracle decode heads {bh}..{min(bh + 64, w.heads) - 1}")
        ro, rl = oracle.attention(x["q"][b, h], x["k"][b, h], x["v"][b, h], causal=False, scale=w.scale,
                                  dtype=w.dtype)
        o_ref[b, h], lse_ref[b, h] = ro[0], rl[0]
    check(o_all, lse_all, o_ref, lse_ref, w.dtype, f"decode, all {w.heads} heads")


def test_spike_on_query_reading():
    # the other reading of the spiked bf16 workload: one Q row per head x 20
    # (scores of std ~20 in that row: a nearly one-hot softmax); full heads at
    # a reduced length, the spiked rows and their neighbours sampled
    w = fi.WORKLOADS["prefill_16k_d128_bf16"].with_(H=4, Nq=4096, Nkv=4096, spike_on="query")
    say("generate spike-on-query workload")
    x = fi.make_inputs(w)
    say("fa_fwd spike-on-query")
    o32, lse32 = fa.fwd(upload(x["q"], w.dtype), upload(x["k"], w.dtype), upload(x["v"], w.dtype), causal=w.causal,
                        scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(o32).all() and torch.isfinite(lse32).all()
    rng = np.random.default_rng(5)
    for bh, i in enumerate(fi.spike_indices(w)):
        rows = _sample_rows(w.Nq, rng, (i - 1, i, i + 1))
        o_ref, lse_ref = oracle.attention_rows(x["q"][0, bh], x["k"][0, bh], x["v"][0, bh], rows, causal=w.causal,
                                               scale=w.scale, dtype=w.dtype)
        check(to_np(o32[0, bh])[rows], to_np(lse32[0, bh])[rows], o_ref, lse_ref, w.dtype,
              f"spike-on-query head {bh} row {i}")
