"""GPU parity of the backward (fa_bwd) against the fp64 oracle, through the C ABI.

The GPU forward supplies O (in the input type) and LSE, as a training step
would; fa_bwd then returns dQ, dK, dV, which are compared with the oracle's
chain-rule gradients evaluated in fp64 on the same 16-bit inputs.

Tolerance: max |err| <= TOL_REL * max |ref| per gradient.  The backward rounds
P and dS to the input type before the products that consume them (relative
error u = 2^-11 for fp16, 2^-8 for bf16, at most half an ulp) and forms
D = rowsum(dO * O) from the rounded forward output; a handful of such
roundings per gradient entry bounds the error by a few u of the gradient's
scale: TOL_REL = 10 u (fp16: 4.9e-3, bf16: 3.9e-2).
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TOL_REL = {k: 10 * u for k, u in U.items()}


def run_fwd_bwd(q, k, v, do, causal, scale, dtype, out_f32=True):
    tq, tk, tv, tdo = (upload(x, dtype) for x in (q, k, v, do))
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    g = fa.bwd(tq, tk, tv, o, tdo, lse, causal=causal, scale=scale,
               out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    return tuple(to_np(x) for x in g)


def check_grads(got, ref, dtype, what):
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert g.shape == r.shape, f"{what} {name}: shape {g.shape} vs {r.shape}"
        assert not np.isnan(g).any(), f"{what} {name}: NaN"
        if r.size == 0:
            continue
        err = float(np.max(np.abs(g - r)))
        mag = float(np.max(np.abs(r)))
        errs.append((name, err, mag))
        say(f"{what}: {name} max err {err:.3e} = {err / max(mag, 1e-300):.2e} of max|ref| {mag:.3e}")
        assert err <= TOL_REL[dtype] * mag + 1e-30, f"{what} {name}: error {err:.3e} > {TOL_REL[dtype]:.1e} x {mag:.3e}"
    return errs


SMALL = [
    # B, H, Nq, Nkv, d, causal, dtype
    (1, 2, 64, 64, 64, False, "f16"),
    (1, 2, 130, 130, 128, True, "f16"),
    (2, 1, 100, 257, 64, True, "bf16"),
    (1, 1, 1, 1, 128, False, "f16"),
    (1, 3, 77, 200, 128, False, "bf16"),
    (2, 2, 256, 256, 128, True, "f16"),
    (1, 1, 513, 600, 64, True, "f16"),
    (1, 2, 200, 64, 128, False, "bf16"),
    (1, 1, 1, 300, 64, True, "f16"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_bwd_small(case):
    B, H, Nq, Nkv, d, causal, dtype = case
    rng = np.random.default_rng(zlib.crc32(("bwd" + repr(case)).encode()))
    q, do = rand_bits(rng, (B, H, Nq, d), dtype), rand_bits(rng, (B, H, Nq, d), dtype)
    k, v = rand_bits(rng, (B, H, Nkv, d), dtype), rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"fa_bwd {case}")
    ref = oracle.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype=dtype)
    got = run_fwd_bwd(q, k, v, do, causal, scale, dtype)
    check_grads(got, ref, dtype, f"bwd {case}")
    # native-type gradients are the fp32 results rounded to nearest even
    g16 = run_fwd_bwd(q, k, v, do, causal, scale, dtype, out_f32=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, g16):
        assert np.array_equal(fi.f32_to_bits(a.astype(np.float32), dtype), fi.f32_to_bits(b.astype(np.float32), dtype)), name


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_bwd_scale_values(scale):
    rng = np.random.default_rng(31)
    B, H, Nq, Nkv, d, dtype = 1, 2, 96, 160, 128, "f16"
    q, do = rand_bits(rng, (B, H, Nq, d), dtype), rand_bits(rng, (B, H, Nq, d), dtype)
    k, v = rand_bits(rng, (B, H, Nkv, d), dtype), rand_bits(rng, (B, H, Nkv, d), dtype)
    say(f"fa_bwd scale={scale}")
    ref = oracle.attention_bwd(q, k, v, do, causal=True, scale=scale, dtype=dtype)
    got = run_fwd_bwd(q, k, v, do, True, scale, dtype)
    if scale == 0.0:
        # no score depends on q or k: the oracle's dQ = dK = 0 exactly (both
        # carry the factor scale); dV is the causal running mean of dO
        assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[1], np.zeros_like(got[1]))
        err = float(np.max(np.abs(got[2] - ref[2])))
        assert err <= TOL_REL[dtype] * float(np.max(np.abs(ref[2]))), err
    else:
        check_grads(got, ref, dtype, f"scale={scale}")


def test_bwd_invariants_and_determinism():
    rng = np.random.default_rng(32)
    B, H, Nq, Nkv, d, dtype = 1, 2, 192, 192, 64, "f16"
    q, do = rand_bits(rng, (B, H, Nq, d), dtype), rand_bits(rng, (B, H, Nq, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    # constant V: O does not depend on Q or K
    vc = np.broadcast_to(rand_bits(rng, (B, H, 1, d), dtype), (B, H, Nkv, d)).copy()
    say("fa_bwd constant V")
    dq, dk, dv = run_fwd_bwd(q, k, vc, do, True, 0.125, dtype)
    assert np.max(np.abs(dq)) <= 2e-3 and np.max(np.abs(dk)) <= 2e-3, (np.max(np.abs(dq)), np.max(np.abs(dk)))
    # key-sum of dK vanishes, key-sum of dV is the query-sum of dO
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    say("fa_bwd sums")
    g1 = run_fwd_bwd(q, k, v, do, True, 0.125, dtype)
    dof = oracle.widen(do, dtype)
    # exact zero / equality in exact arithmetic; per-entry errors of TOL_REL
    # of the largest entry, summed over Nkv keys with random signs
    bound = TOL_REL[dtype] * np.sqrt(Nkv)
    assert np.max(np.abs(g1[1].sum(axis=2))) <= bound * np.max(np.abs(g1[1]))
    assert np.max(np.abs(g1[2].sum(axis=2) - dof.sum(axis=2))) <= bound * np.max(np.abs(g1[2]))
    g2 = run_fwd_bwd(q, k, v, do, True, 0.125, dtype)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b), "backward not deterministic"


def _sampled_rows(rng, n, extra):
    return np.unique(np.concatenate([[0, 1, n // 2, n - 2, n - 1], rng.integers(0, n, extra)])).astype(np.int64)


@pytest.mark.parametrize("name,heads", [("prefill_8k_d128", [(0, 5), (0, 30)]),
                                        ("prefill_2k_d64", [(0, 0), (1, 7)])])
def test_bwd_full_size_sampled(name, heads):
    # the workload at full size in the shape the benchmark times; dO from the
    # seeded generator; sampled dQ rows and dK / dV rows of a few heads
    w = fi.WORKLOADS[name]
    say(f"fa_bwd {name} full size")
    x = fi.make_inputs(w)
    dob = fi.make_tensor(w, fi.DOUT)
    tq, tk, tv = (upload(x[t], w.dtype) for t in "qkv")
    tdo = upload(dob, w.dtype)
    o, lse = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not (torch.isnan(dq).any() or torch.isnan(dk).any() or torch.isnan(dv).any())
    rng = np.random.default_rng(7)
    for b, h in heads:
        qr = _sampled_rows(rng, w.Nq, 6)
        kc = _sampled_rows(rng, w.Nkv, 6)
        ref = oracle.attention_bwd_sampled(x["q"][b, h], x["k"][b, h], x["v"][b, h], dob[b, h], qr, kc,
                                           causal=w.causal, scale=w.scale, dtype=w.dtype)
        got = (to_np(dq[b, h])[qr], to_np(dk[b, h])[kc], to_np(dv[b, h])[kc])
        check_grads(got, ref, w.dtype, f"{name} head ({b},{h}) sampled")
