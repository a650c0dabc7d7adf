"""GPU parity of the backward (fa_bwd) against the fp64 oracle, through the C ABI.

fa_bwd is handed the forward's output O in the input type and its LSE, as a
training step would.  Here both come from the oracle: its O rounded to the
input type and its LSE in fp32 (so no GPU result feeds the comparison).
fa_bwd returns dQ, dK, dV, which are compared with the oracle's chain-rule
gradients evaluated in fp64 on the same 16-bit inputs, with D formed from the
same 16-bit O that fa_bwd is given (D_i = sum_c dO_ic O_ic: the reading that
the backward works from the O it is handed).

Tolerance: max |err| <= TOL_REL * max |ref| per gradient.  The backward rounds
P and dS to the input type before the products that consume them (relative
error u = 2^-11 for fp16, 2^-8 for bf16, at most half an ulp); a handful of
such roundings per gradient entry bounds the error by a few u of the
gradient's scale: TOL_REL = 10 u (fp16: 4.9e-3, bf16: 3.9e-2).

Diagnostic only: against the oracle's D from the exact O, the rounding of O
to 16 bits would move dQ_i by up to |scale| u A_i sum_j P_ij |K_jc| with
A_i = sum_c |dO_ic O_ic| -- a term not bounded by dQ's own scale (a key row 20x
longer than the rest multiplies it).  The tests print how many rows that term
would push beyond a tenth of the plain bar; with D from the handed-over O it
plays no part in the comparison.
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import device, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TOL_REL = {k: 10 * u for k, u in U.items()}


def oracle_forward(q, k, v, causal, scale, dtype):
    """The forward result fa_bwd is handed, from the oracle: O (fp64, rounded
    through fp32 to the input type's bits) and LSE as fp32."""
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale, dtype=dtype)
    return fi.f32_to_bits(o.astype(np.float32), dtype), lse.astype(np.float32)


def run_bwd(q, k, v, do, o16, lse32, causal, scale, dtype, out_f32=True):
    tq, tk, tv, tdo, to = (upload(x, dtype) for x in (q, k, v, do, o16))
    tl = torch.from_numpy(np.ascontiguousarray(lse32)).to(device())
    g = fa.bwd(tq, tk, tv, to, tdo, tl, causal=causal, scale=scale, out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    return tuple(to_np(x) for x in g)


def d_term(q, k, v, dout, rows, causal, scale, dtype):
    """|scale| u A_i sum_j P_ij |K_jc| for the query rows `rows` of one head
    ([len(rows), d], fp64): the most that rounding O to the input type could
    move dQ through D.  O, LSE from the fp64 reference, P and A recomputed
    from them here in numpy."""
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
    return abs(scale) * U[dtype] * a[:, None] * (p @ np.abs(kf))


def check_grads(got, ref, dtype, what, dq_term=None):
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
        if name == "dQ" and dq_term is not None:
            rows_big = int(np.sum(np.max(dq_term, axis=-1) > 0.1 * bound))
            say(f"{what}: rows whose O-rounding term would exceed a tenth of the dQ bar: {rows_big} of "
                f"{dq_term.reshape(-1, dq_term.shape[-1]).shape[0]} (not used: D comes from the same O)")
        if err > bound:
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
    o16, lse32 = oracle_forward(q, k, v, causal, scale, dtype)
    ref = oracle.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype=dtype, o_for_d=o16)
    got = run_bwd(q, k, v, do, o16, lse32, causal, scale, dtype)
    term = np.stack([np.stack([d_term(q[b, h], k[b, h], v[b, h], do[b, h], np.arange(Nq), causal, scale, dtype)
                               for h in range(H)]) for b in range(B)])
    check_grads(got, ref, dtype, f"bwd {case}", dq_term=term)
    # native-type gradients are the fp32 results rounded to nearest even
    g16 = run_bwd(q, k, v, do, o16, lse32, causal, scale, dtype, out_f32=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, g16):
        assert np.array_equal(fi.f32_to_bits(a.astype(np.float32), dtype), fi.f32_to_bits(b.astype(np.float32), dtype)), name


# d = 64 grids wide enough (at least two workgroups per CU in a pass) for the
# 16x16x32 passes, which d = 64 uses only there; ragged lengths, causal and
# rectangular.  The last case takes the key-block pass on the 16x16x32 kernel
# (64 heads x 9 key blocks) and the query-block pass on the 32x32 one (64 x 4
# query blocks).  Every head is compared in full.
WIDE64 = [
    (2, 32, 1000, 1000, 64, True, "f16"),
    (1, 96, 700, 1100, 64, False, "bf16"),
    (1, 64, 1024, 1030, 64, True, "bf16"),
    (1, 64, 500, 1100, 64, True, "f16"),
]


@pytest.mark.parametrize("case", WIDE64, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_bwd_wide_grid_d64(case):
    B, H, Nq, Nkv, d, causal, dtype = case
    assert B * H * -(-Nq // 128) >= 512 or B * H * -(-Nkv // 128) >= 512
    rng = np.random.default_rng(zlib.crc32(("bwd-wide" + repr(case)).encode()))
    q, do = rand_bits(rng, (B, H, Nq, d), dtype), rand_bits(rng, (B, H, Nq, d), dtype)
    k, v = rand_bits(rng, (B, H, Nkv, d), dtype), rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"fa_bwd wide d=64 {case}")
    o16, lse32 = oracle_forward(q, k, v, causal, scale, dtype)
    ref = oracle.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype=dtype, o_for_d=o16)
    got = run_bwd(q, k, v, do, o16, lse32, causal, scale, dtype)
    check_grads(got, ref, dtype, f"bwd wide {case}")
    g16 = run_bwd(q, k, v, do, o16, lse32, causal, scale, dtype, out_f32=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, g16):
        assert np.array_equal(fi.f32_to_bits(a.astype(np.float32), dtype), fi.f32_to_bits(b.astype(np.float32), dtype)), name


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_bwd_scale_values(scale):
    rng = np.random.default_rng(31)
    B, H, Nq, Nkv, d, dtype = 1, 2, 96, 160, 128, "f16"
    q, do = rand_bits(rng, (B, H, Nq, d), dtype), rand_bits(rng, (B, H, Nq, d), dtype)
    k, v = rand_bits(rng, (B, H, Nkv, d), dtype), rand_bits(rng, (B, H, Nkv, d), dtype)
    say(f"fa_bwd scale={scale}")
    o16, lse32 = oracle_forward(q, k, v, True, scale, dtype)
    ref = oracle.attention_bwd(q, k, v, do, causal=True, scale=scale, dtype=dtype, o_for_d=o16)
    got = run_bwd(q, k, v, do, o16, lse32, True, scale, dtype)
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
    dq, dk, dv = run_bwd(q, k, vc, do, *oracle_forward(q, k, vc, True, 0.125, dtype), True, 0.125, dtype)
    assert np.max(np.abs(dq)) <= 2e-3 and np.max(np.abs(dk)) <= 2e-3, (np.max(np.abs(dq)), np.max(np.abs(dk)))
    # key-sum of dK vanishes, key-sum of dV is the query-sum of dO
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    say("fa_bwd sums")
    fwd_out = oracle_forward(q, k, v, True, 0.125, dtype)
    g1 = run_bwd(q, k, v, do, *fwd_out, True, 0.125, dtype)
    dof = oracle.widen(do, dtype)
    # exact zero / equality in exact arithmetic; per-entry errors of TOL_REL
    # of the largest entry, summed over Nkv keys with random signs
    bound = TOL_REL[dtype] * np.sqrt(Nkv)
    assert np.max(np.abs(g1[1].sum(axis=2))) <= bound * np.max(np.abs(g1[1]))
    assert np.max(np.abs(g1[2].sum(axis=2) - dof.sum(axis=2))) <= bound * np.max(np.abs(g1[2]))
    g2 = run_bwd(q, k, v, do, *fwd_out, True, 0.125, dtype)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b), "backward not deterministic"


def _sampled_rows(rng, n, extra):
    return np.unique(np.concatenate([[0, 1, n // 2, n - 2, n - 1], rng.integers(0, n, extra)])).astype(np.int64)


@pytest.mark.parametrize("name,heads", [("prefill_8k_d128", [(0, 5), (0, 30)]),
                                        ("prefill_2k_d64", [(0, 0), (1, 7)]),
                                        ("prefill_16k_d128_bf16", [(0, 3), (0, 12)])])
def test_bwd_full_size_sampled(name, heads):
    # the workload at full size in the shape the benchmark times; dO from the
    # seeded generator; sampled dQ rows and dK / dV rows of a few heads.  The
    # sampled heads get the oracle's O and LSE; the others keep the GPU
    # forward's (their gradients are not compared)
    w = fi.WORKLOADS[name]
    say(f"fa_bwd {name} full size")
    x = fi.make_inputs(w)
    dob = fi.make_tensor(w, fi.DOUT)
    tq, tk, tv = (upload(x[t], w.dtype) for t in "qkv")
    tdo = upload(dob, w.dtype)
    o, lse = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    fwd_ref = {}
    for b, h in heads:
        o16, lse32 = oracle_forward(x["q"][b, h], x["k"][b, h], x["v"][b, h], w.causal, w.scale, w.dtype)
        o[b, h] = upload(o16, w.dtype)
        lse[b, h] = torch.from_numpy(lse32).to(lse.device)
        fwd_ref[(b, h)] = o16
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
                                           causal=w.causal, scale=w.scale, dtype=w.dtype, o_for_d=fwd_ref[(b, h)])
        got = (to_np(dq[b, h])[qr], to_np(dk[b, h])[kc], to_np(dv[b, h])[kc])
        term = d_term(x["q"][b, h], x["k"][b, h], x["v"][b, h], dob[b, h], qr, w.causal, w.scale, w.dtype)
        check_grads(got, ref, w.dtype, f"{name} head ({b},{h}) sampled", dq_term=term)
