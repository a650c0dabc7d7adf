"""GPU parity of the backward (fa_bwd) against the fp64 oracle, through the C ABI.

The GPU forward supplies O (in the input type) and LSE, as a training step
would; fa_bwd then returns dQ, dK, dV, which are compared with the oracle's
chain-rule gradients evaluated in fp64 on the same 16-bit inputs.

Tolerance: max |err| <= TOL_REL * max |ref| per gradient.  The backward rounds
P and dS to the input type before the products that consume them (relative
error u = 2^-11 for fp16, 2^-8 for bf16, at most half an ulp); a handful of
such roundings per gradient entry bounds the error by a few u of the
gradient's scale: TOL_REL = 10 u (fp16: 4.9e-3, bf16: 3.9e-2).

dQ carries one more term.  D = rowsum(dO * O) is formed from the forward
output O in the input type, as the caller hands it over, so D_i is off by up
to u * A_i with A_i = sum_c |dO_ic O_ic|.  That error enters every
dS_ij = P_ij (dP_ij - D_i) of the row and reaches dQ_i = scale * sum_j dS_ij K_j
as at most |scale| u A_i sum_j P_ij |K_jc|, which is not bounded by the scale
of dQ itself: a key row much longer than the others (the spiked workload
multiplies one K row by 20) multiplies it while the cancellation in
dP - D keeps dQ small.  The dQ bound is therefore, element by element,
TOL_REL * max |dQ_ref| + 2 |scale| u A_i sum_j P_ij |K_jc|, with O, P and A from
the fp64 reference.  (dK = scale * dS^T Q sums the same D errors over queries
weighted by P; it stays within TOL_REL on every workload here.)
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


def d_term(q, k, v, dout, rows, causal, scale, dtype):
    """2 |scale| u A_i sum_j P_ij |K_jc| for the query rows `rows` of one head ([len(rows), d], fp64).

    q, k, v, dout are one head's 16-bit bit patterns ([N, d]); O, LSE come from
    the fp64 reference, P and A are recomputed from them here in numpy."""
    rows = np.asarray(rows, dtype=np.int64)
    o, lse = oracle.attention_rows(q, k, v, rows, causal=causal, scale=scale, dtype=dtype)
    qf = oracle.widen(q, dtype)[rows]
    kf = oracle.widen(k, dtype)
    dof = oracle.widen(dout, dtype)[rows]
    Nq, Nkv = q.shape[0], k.shape[0]
    s = scale * (qf @ kf.T)
    if causal:
        s = np.where(np.arange(Nkv)[None, :] <= rows[:, None] + (Nkv - Nq), s, -np.inf)
    p = np.exp(s - lse[:, None])
    a = np.sum(np.abs(dof * o), axis=1)
    return 2.0 * abs(scale) * U[dtype] * a[:, None] * (p @ np.abs(kf))


def check_grads(got, ref, dtype, what, dq_extra=None):
    errs, bad = [], []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert g.shape == r.shape, f"{what} {name}: shape {g.shape} vs {r.shape}"
        assert not np.isnan(g).any(), f"{what} {name}: NaN"
        if r.size == 0:
            continue
        err = float(np.max(np.abs(g - r)))
        mag = float(np.max(np.abs(r)))
        errs.append((name, err, mag))
        say(f"{what}: {name} max err {err:.3e} = {err / max(mag, 1e-300):.2e} of max|ref| {mag:.3e}")
        bound = TOL_REL[dtype] * mag + 1e-30
        if name == "dQ" and dq_extra is not None:
            excess = np.abs(g - r) - (bound + dq_extra)
            worst = np.unravel_index(int(np.argmax(excess)), excess.shape)
            say(f"{what}: dQ with the D term: worst margin {float(excess[worst]):.3e} at {worst}")
            if excess[worst] > 0:
                bad.append(f"dQ: error {float(np.abs(g - r)[worst]):.3e} at {worst} > {bound:.3e} + D term "
                           f"{float(dq_extra[worst]):.3e}")
        elif err > bound:
            bad.append(f"{name}: error {err:.3e} > {TOL_REL[dtype]:.1e} x {mag:.3e}")
    assert not bad, f"{what}: " + "; ".join(bad)
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
    extra = np.stack([np.stack([d_term(q[b, h], k[b, h], v[b, h], do[b, h], np.arange(Nq), causal, scale, dtype)
                                for h in range(H)]) for b in range(B)])
    check_grads(got, ref, dtype, f"bwd {case}", dq_extra=extra)
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
                                        ("prefill_2k_d64", [(0, 0), (1, 7)]),
                                        ("prefill_16k_d128_bf16", [(0, 3), (0, 12)])])
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
        if w.spike:  # the spiked key and its neighbours
            j = fi.spike_indices(w)[b * w.H + h]
            kc = np.unique(np.concatenate([kc, [max(j - 1, 0), j, min(j + 1, w.Nkv - 1)]])).astype(np.int64)
        ref = oracle.attention_bwd_sampled(x["q"][b, h], x["k"][b, h], x["v"][b, h], dob[b, h], qr, kc,
                                           causal=w.causal, scale=w.scale, dtype=w.dtype)
        got = (to_np(dq[b, h])[qr], to_np(dk[b, h])[kc], to_np(dv[b, h])[kc])
        extra = d_term(x["q"][b, h], x["k"][b, h], x["v"][b, h], dob[b, h], qr, w.causal, w.scale, w.dtype)
        check_grads(got, ref, w.dtype, f"{name} head ({b},{h}) sampled", dq_extra=extra)
