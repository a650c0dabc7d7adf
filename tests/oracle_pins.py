"""Checks that pin the fp64 attention reference to things other than itself.

Every function takes an ``oracle.Oracle`` handle and raises AssertionError when
the reference disagrees with the pin.  tests/test_oracle_pins.py runs them on
the real build; tests/test_oracle_mutants.py runs them on builds with planted
mistakes and requires each mistake to be caught.

What the pins rest on:
  * the definition softmax(scale * Q K^T) V evaluated independently: a
    50-digit decimal brute force without the max shift, and torch's float64
    scaled_dot_product_attention / logsumexp (library special cases);
  * closed forms and invariants of the definition: constant V, Q = 0,
    causal row 0, a dominant score, a single key, the worked two-key example,
    convex-combination bounds, exact power-of-two linearity in V, joint
    permutation of K and V, invariance under a uniform shift of the scores;
  * the two-block merge of partial softmax results ("FlashAttention 1-2-3:
    The IO-Aware Revolution in LLM Inference", section "The Math Behind the
    Online Softmax Trick"): attention over all keys equals the merge of
    attention over two disjoint key sets, for any split point;
  * exact decoding of the 16-bit storage formats, against numpy (binary16)
    and torch (bfloat16);
  * for the backward (dQ, dK, dV given dL/dO): torch float64 autograd through
    an independently written masked softmax attention, central finite
    differences of the (separately pinned) forward, and exact invariants:
    the key-sum of dK vanishes (each softmax row sums to one), the key-sum of
    dV equals the query-sum of dO, a constant V gives dQ = dK = 0, and the
    gradients are linear in dO.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _visible_count(i, Nq, Nkv, causal):
    return Nkv if not causal else min(Nkv, i + Nkv - Nq + 1)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# storage formats

def pin_widen_f16(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 decode differs from numpy"


def pin_widen_bf16(orc):
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decode differs from torch"
    # a few closed forms: 1.0, -2.0, smallest subnormal, largest finite
    assert orc.widen(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], np.uint16), "bf16").tolist() == [
        1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]


# ---------------------------------------------------------------------------
# independent evaluations of the definition

def _decimal_attention(q, k, v, causal, scale):
    """softmax(scale q k^T) v at 50 significant digits, straight from the definition."""
    Nq, d = q.shape
    Nkv = k.shape[0]
    o = np.zeros((Nq, d))
    lse = np.zeros(Nq)
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(scale)
        for i in range(Nq):
            weights = []
            for j in range(Nkv):
                if causal and j > i + (Nkv - Nq):
                    continue
                dot = sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c])) for c in range(d))
                weights.append((j, (sc * dot).exp()))
            z = sum(w for _, w in weights)
            for c in range(d):
                num = sum(w * Decimal(float(v[j, c])) for j, w in weights)
                o[i, c] = float(num / z)
            lse[i] = float(z.ln())
    return o, lse


def pin_decimal_bruteforce(orc):
    rng = _rng(11)
    cases = [(1, 1, 1, False, 0.5), (5, 5, 3, True, 0.7), (4, 7, 4, True, 0.5),
             (6, 6, 2, False, -0.9), (3, 8, 5, False, 0.45), (2, 2, 1, True, 1.0)]
    for Nq, Nkv, d, causal, scale in cases:
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nkv, d))
        v = rng.standard_normal((Nkv, d))
        o, lse = orc.attention(q, k, v, causal=causal, scale=scale)
        o_ref, lse_ref = _decimal_attention(q, k, v, causal, scale)
        _close(o, o_ref, what=f"O vs decimal {Nq}x{Nkv}x{d} causal={causal}")
        _close(lse, lse_ref, what=f"LSE vs decimal {Nq}x{Nkv}x{d} causal={causal}")


def pin_torch_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = _rng(12)
    for B, H, Nq, Nkv, d, causal in [(2, 3, 17, 17, 8, True), (1, 2, 33, 64, 16, True),
                                      (2, 1, 40, 23, 32, False), (1, 1, 64, 64, 64, True)]:
        scale = 1.0 / math.sqrt(d)
        q = rng.standard_normal((B, H, Nq, d))
        k = rng.standard_normal((B, H, Nkv, d))
        v = rng.standard_normal((B, H, Nkv, d))
        o, lse = orc.attention(q, k, v, causal=causal, scale=scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        mask = torch.ones(Nq, Nkv, dtype=torch.bool)
        if causal:
            mask = mask.tril(diagonal=Nkv - Nq)
        o_ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        s = (tq @ tk.transpose(-1, -2)) * scale
        lse_ref = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        _close(o, o_ref.numpy(), what=f"O vs torch sdpa {B}x{H}x{Nq}x{Nkv}x{d}")
        _close(lse, lse_ref.numpy(), what=f"LSE vs torch logsumexp {B}x{H}x{Nq}x{Nkv}x{d}")
        if causal and Nq == Nkv:
            o_ref2 = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
            _close(o, o_ref2.numpy(), what="O vs torch sdpa is_causal")


# ---------------------------------------------------------------------------
# closed forms and invariants

def pin_two_key_worked(orc):
    # scale 1, query (1, 0) against keys (0, 0) and (1, 0) -- scores 0 and 1 --
    # with values e_0 and e_1: weights 1/(1+e) and e/(1+e), LSE ln(1+e).
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [1.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = orc.attention(q, k, v, causal=False, scale=1.0)
    e = math.e
    _close(o, [[1 / (1 + e), e / (1 + e)]], 1e-15, "two-key weights")
    _close(lse, [math.log1p(e)], 1e-15, "two-key LSE")
    # causal, two queries: row 0 sees key 0 only, row 1 both keys
    q2 = np.array([[1.0, 0.0], [1.0, 0.0]])
    o2, lse2 = orc.attention(q2, k, v, causal=True, scale=1.0)
    _close(o2, [[1.0, 0.0], [1 / (1 + e), e / (1 + e)]], 1e-15, "two-key causal weights")
    _close(lse2, [0.0, math.log1p(e)], 1e-15, "two-key causal LSE")


def pin_constant_v(orc):
    rng = _rng(13)
    for causal in (False, True):
        q = rng.standard_normal((2, 2, 24, 8)) * 3
        k = rng.standard_normal((2, 2, 24, 8)) * 3
        c = rng.standard_normal(8)
        v = np.broadcast_to(c, (2, 2, 24, 8)).copy()
        o, _ = orc.attention(q, k, v, causal=causal, scale=0.4)
        _close(o, np.broadcast_to(c, o.shape), 1e-14, f"constant V causal={causal}")


def pin_q_zero(orc):
    rng = _rng(14)
    for Nq, Nkv, causal in [(9, 9, True), (5, 12, True), (7, 11, False)]:
        d = 6
        q = np.zeros((Nq, d))
        k = rng.standard_normal((Nkv, d))
        v = rng.standard_normal((Nkv, d))
        o, lse = orc.attention(q, k, v, causal=causal, scale=0.3)
        for i in range(Nq):
            n = _visible_count(i, Nq, Nkv, causal)
            _close(o[i], v[:n].mean(axis=0), 1e-14, f"Q=0 mean row {i}")
            _close(lse[i], math.log(n), 1e-14, f"Q=0 LSE row {i}")


def pin_causal_row0(orc):
    rng = _rng(15)
    q = rng.standard_normal((16, 8))
    k = rng.standard_normal((16, 8))
    v = rng.standard_normal((16, 8))
    o, lse = orc.attention(q, k, v, causal=True, scale=0.35)
    assert np.array_equal(o[0], v[0]), "causal row 0 must equal V[0]"
    _close(lse[0], 0.35 * float(np.dot(q[0], k[0])), 1e-14, "causal row 0 LSE")


def pin_dominant_score(orc):
    rng = _rng(16)
    Nq, Nkv, d, js = 4, 10, 4, 6
    q = np.zeros((Nq, d))
    q[:, 0] = 1.0
    q[:, 1:] = rng.standard_normal((Nq, d - 1)) * 0.1
    k = rng.standard_normal((Nkv, d)) * 0.1
    k[js] = [45.0, 0.0, 0.0, 0.0]
    v = rng.standard_normal((Nkv, d))
    o, lse = orc.attention(q, k, v, causal=False, scale=1.0)
    _close(o, np.broadcast_to(v[js], o.shape), 1e-14, "dominant key selects its V row")
    _close(lse, np.full(Nq, 45.0), 1e-12, "dominant key LSE")
    # scores spread far beyond exp's range (key 0 at -400, the dominant key at
    # +400): a softmax that does not subtract the true row max overflows.
    k[0] = [-400.0, 0.0, 0.0, 0.0]
    k[js] = [400.0, 0.0, 0.0, 0.0]
    o, lse = orc.attention(q, k, v, causal=False, scale=1.0)
    _close(o, np.broadcast_to(v[js], o.shape), 1e-14, "wide spread: dominant key selects its V row")
    _close(lse, np.full(Nq, 400.0), 1e-12, "wide spread: LSE equals the dominant score")


def pin_single_key(orc):
    rng = _rng(17)
    q = rng.standard_normal((3, 5))
    k = rng.standard_normal((1, 5))
    v = rng.standard_normal((1, 5))
    o, lse = orc.attention(q, k, v, causal=False, scale=0.8)
    assert np.array_equal(o, np.broadcast_to(v[0], o.shape)), "one key: O = V[0]"
    _close(lse, 0.8 * (q @ k[0]), 1e-14, "one key: LSE = score")


def pin_bounds(orc):
    rng = _rng(18)
    Nq, Nkv, d = 12, 20, 7
    q = rng.standard_normal((Nq, d)) * 2
    k = rng.standard_normal((Nkv, d)) * 2
    v = rng.standard_normal((Nkv, d))
    o, lse = orc.attention(q, k, v, causal=True, scale=0.5)
    s = 0.5 * (q @ k.T)
    for i in range(Nq):
        n = _visible_count(i, Nq, Nkv, True)
        vis = v[:n]
        assert np.all(o[i] >= vis.min(axis=0) - 1e-14) and np.all(o[i] <= vis.max(axis=0) + 1e-14)
        smax = s[i, :n].max()
        assert smax - 1e-14 <= lse[i] <= smax + math.log(n) + 1e-14, f"LSE bounds row {i}"


def pin_linearity(orc):
    rng = _rng(19)
    q = rng.standard_normal((2, 1, 15, 6))
    k = rng.standard_normal((2, 1, 18, 6))
    v = rng.standard_normal((2, 1, 18, 6))
    o, lse = orc.attention(q, k, v, causal=True, scale=0.6)
    o8, lse8 = orc.attention(q, k, v * 8.0, causal=True, scale=0.6)
    assert np.array_equal(o8, o * 8.0), "O(8V) must equal 8 O(V) exactly"
    assert np.array_equal(lse8, lse), "LSE must not depend on V"


def pin_permutation(orc):
    rng = _rng(20)
    q = rng.standard_normal((9, 5))
    k = rng.standard_normal((14, 5))
    v = rng.standard_normal((14, 5))
    perm = rng.permutation(14)
    o, lse = orc.attention(q, k, v, causal=False, scale=0.7)
    op, lsep = orc.attention(q, k[perm], v[perm], causal=False, scale=0.7)
    _close(op, o, 1e-14, "joint permutation of K, V")
    _close(lsep, lse, 1e-14, "joint permutation LSE")


def pin_shift_invariance(orc):
    # Appending a column (c to every query, 1 to every key) adds scale*c to
    # every score: O is unchanged, LSE moves by scale*c.  With c large the
    # exponentials overflow unless the row max is subtracted first.
    rng = _rng(21)
    Nq, Nkv, d, scale, c = 6, 9, 4, 0.5, 2000.0
    q = rng.standard_normal((Nq, d))
    k = rng.standard_normal((Nkv, d))
    v = rng.standard_normal((Nkv, d))
    o, lse = orc.attention(q, k, v, causal=True, scale=scale)
    q2 = np.concatenate([q, np.full((Nq, 1), c)], axis=1)
    k2 = np.concatenate([k, np.ones((Nkv, 1))], axis=1)
    v2 = np.concatenate([v, np.zeros((Nkv, 1))], axis=1)  # one head dimension for q, k and v
    o2, lse2 = orc.attention(q2, k2, v2, causal=True, scale=scale)
    _close(o2[:, :d], o, 1e-12, "uniform score shift leaves O unchanged")
    _close(lse2 - scale * c, lse, 1e-10, "uniform score shift moves LSE by the shift")


def pin_merge_identity(orc):
    rng = _rng(22)
    Nq, Nkv, d = 7, 30, 8
    q = rng.standard_normal((Nq, d)) * 1.5
    k = rng.standard_normal((Nkv, d)) * 1.5
    v = rng.standard_normal((Nkv, d))
    o, lse = orc.attention(q, k, v, causal=False, scale=0.4)
    for a in (1, 7, 15, 29):
        o1, l1 = orc.attention(q, k[:a], v[:a], causal=False, scale=0.4)
        o2, l2 = orc.attention(q, k[a:], v[a:], causal=False, scale=0.4)
        lm = np.logaddexp(l1, l2)
        om = np.exp(l1 - lm)[:, None] * o1 + np.exp(l2 - lm)[:, None] * o2
        _close(om, o, what=f"merged O, split at {a}")
        _close(lm, lse, what=f"merged LSE, split at {a}")


def pin_rows_match_full(orc):
    rng = _rng(23)
    for causal, Nq, Nkv in [(True, 21, 30), (False, 13, 8)]:
        d = 9
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nkv, d))
        v = rng.standard_normal((Nkv, d))
        o, lse = orc.attention(q, k, v, causal=causal, scale=0.3)
        rows = np.array([0, Nq - 1, Nq // 2, 3])
        orow, lrow = orc.attention_rows(q, k, v, rows, causal=causal, scale=0.3)
        assert np.array_equal(orow, o[rows]) and np.array_equal(lrow, lse[rows]), "rows vs full"


def pin_head_independence(orc):
    rng = _rng(24)
    q = rng.standard_normal((2, 3, 10, 4))
    k = rng.standard_normal((2, 3, 12, 4))
    v = rng.standard_normal((2, 3, 12, 4))
    o, lse = orc.attention(q, k, v, causal=True, scale=0.5)
    for b in range(2):
        for h in range(3):
            oh, lh = orc.attention(q[b, h], k[b, h], v[b, h], causal=True, scale=0.5)
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h]), "head offsets"


def pin_widened_inputs(orc):
    # the 16-bit entry point equals the fp64 entry point on the decoded values
    rng = _rng(25)
    for dtype in ("f16", "bf16"):
        raw = rng.standard_normal((3, 6, 5)).astype(np.float32)
        if dtype == "f16":
            bits = raw.astype(np.float16).view(np.uint16)
            vals = bits.view(np.float16).astype(np.float64)
        else:
            import torch
            t = torch.from_numpy(raw).to(torch.bfloat16)
            bits = t.view(torch.int16).numpy().view(np.uint16)
            vals = t.to(torch.float64).numpy()
        o_b, l_b = orc.attention(bits[0], bits[1], bits[2], causal=True, scale=0.5, dtype=dtype)
        o_v, l_v = orc.attention(vals[0], vals[1], vals[2], causal=True, scale=0.5)
        assert np.array_equal(o_b, o_v) and np.array_equal(l_b, l_v), f"{dtype} inputs"


# ---------------------------------------------------------------------------
# backward

def _torch_attention_grads(q, k, v, do, causal, scale):
    """dQ, dK, dV of sum(O * do) by torch float64 autograd on the CPU."""
    import torch
    tq, tk, tv = (torch.from_numpy(np.array(x)).requires_grad_(True) for x in (q, k, v))
    Nq, Nkv = q.shape[-2], k.shape[-2]
    mask = torch.ones(Nq, Nkv, dtype=torch.bool)
    if causal:
        mask = mask.tril(diagonal=Nkv - Nq)
    s = (tq @ tk.transpose(-1, -2)) * scale
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
    o = p @ tv
    (o * torch.from_numpy(np.array(do))).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_bwd_torch_autograd(orc):
    rng = _rng(21)
    for B, H, Nq, Nkv, d, causal, scale in [(2, 2, 9, 9, 4, True, 0.5), (1, 2, 13, 30, 8, True, 0.35),
                                            (2, 1, 20, 11, 16, False, 0.25), (1, 1, 7, 7, 3, False, -0.8)]:
        q = rng.standard_normal((B, H, Nq, d))
        k = rng.standard_normal((B, H, Nkv, d))
        v = rng.standard_normal((B, H, Nkv, d))
        do = rng.standard_normal((B, H, Nq, d))
        got = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale)
        ref = _torch_attention_grads(q, k, v, do, causal, scale)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            _close(a, b, tol=1e-11, what=f"{name} vs torch autograd {B}x{H}x{Nq}x{Nkv}x{d} causal={causal}")


def pin_bwd_finite_difference(orc):
    # central differences of L = sum(O * dO) through the forward reference
    rng = _rng(22)
    Nq, Nkv, d, scale = 6, 9, 5, 0.6
    for causal in (False, True):
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nkv, d))
        v = rng.standard_normal((Nkv, d))
        do = rng.standard_normal((Nq, d))
        grads = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale)
        h = 1e-5
        for which, x in enumerate((q, k, v)):
            for _ in range(6):
                idx = tuple(int(rng.integers(0, n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                lp = float(np.sum(orc.attention(*args_p, causal=causal, scale=scale)[0] * do))
                lm = float(np.sum(orc.attention(*args_m, causal=causal, scale=scale)[0] * do))
                fd = (lp - lm) / (2 * h)
                g = float(grads[which][idx])
                assert abs(fd - g) <= 1e-7 * max(1.0, abs(g)), \
                    f"d{'QKV'[which]}{idx} = {g:.12f}, finite difference {fd:.12f} (causal={causal})"


def pin_bwd_invariants(orc):
    rng = _rng(23)
    B, H, Nq, Nkv, d = 2, 2, 11, 17, 6
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, H, Nkv, d))
    v = rng.standard_normal((B, H, Nkv, d))
    do = rng.standard_normal((B, H, Nq, d))
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal, scale=0.4)
        # each softmax row sums to one, so its dS row sums to zero
        _close(dk.sum(axis=2), np.zeros((B, H, d)), tol=1e-12, what="key-sum of dK")
        _close(dv.sum(axis=2), do.sum(axis=2), tol=1e-12, what="key-sum of dV vs query-sum of dO")
        # constant V: O does not depend on Q or K
        vc = np.broadcast_to(rng.standard_normal((B, H, 1, d)), v.shape).copy()
        dq0, dk0, _ = orc.attention_bwd(q, k, vc, do, causal=causal, scale=0.4)
        _close(dq0, np.zeros_like(dq0), tol=1e-12, what="dQ with constant V")
        _close(dk0, np.zeros_like(dk0), tol=1e-12, what="dK with constant V")
        # linear in dO: doubling it doubles every gradient exactly
        dq2, dk2, dv2 = orc.attention_bwd(q, k, v, 2.0 * do, causal=causal, scale=0.4)
        assert np.array_equal(dq2, 2.0 * dq) and np.array_equal(dk2, 2.0 * dk) and \
            np.array_equal(dv2, 2.0 * dv), "gradients not linear in dO"


def pin_bwd_sampled_matches_full(orc):
    # the row/column sampling entry against the whole-head backward
    rng = _rng(24)
    for Nq, Nkv, d, causal in [(13, 29, 8, True), (20, 20, 16, True), (9, 5, 4, False)]:
        q, do = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
        k, v = rng.standard_normal((Nkv, d)), rng.standard_normal((Nkv, d))
        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal, scale=0.3)
        qr = np.array([0, Nq - 1, Nq // 2], dtype=np.int64)
        kc = np.array([Nkv - 1, 0, Nkv // 3], dtype=np.int64)
        sq, sk, sv = orc.attention_bwd_sampled(q, k, v, do, qr, kc, causal=causal, scale=0.3)
        _close(sq, dq[qr], tol=1e-12, what="sampled dQ rows")
        _close(sk, dk[kc], tol=1e-12, what="sampled dK rows")
        _close(sv, dv[kc], tol=1e-12, what="sampled dV rows")


def pin_bwd_d_from_given_o(orc):
    # D formed from a given forward output O: with the exact O the gradients
    # are torch's autograd ones (D = rowsum(P dP) = rowsum(dO O)); with O + E
    # the closed form of the shift dD_i = sum_c dO_ic E_ic holds:
    #   dQ_i changes by -scale dD_i (P K)_i,  dK_j by -scale sum_i P_ij dD_i q_i,  dV not at all
    # (P from torch's float64 softmax); the row/column sampling entry agrees
    import torch
    rng = _rng(25)
    for Nq, Nkv, d, causal, scale in [(11, 11, 6, True, 0.45), (7, 19, 5, True, -0.3), (9, 6, 8, False, 0.7)]:
        q, do = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
        k, v = rng.standard_normal((Nkv, d)), rng.standard_normal((Nkv, d))
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        s_ = scale * (tq @ tk.T)
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nkv)[None, :]
            s_ = s_.masked_fill(j > i + (Nkv - Nq), float("-inf"))
        p = torch.softmax(s_, -1)
        o = (p @ tv).numpy()
        ref = _torch_attention_grads(q[None, None], k[None, None], v[None, None], do[None, None], causal, scale)
        got = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale, o_for_d=o)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            _close(a, b[0, 0], tol=1e-11, what=f"{name} with D from the exact O")
        e = rng.standard_normal((Nq, d)) * 1e-2
        dd = np.sum(do * e, axis=1)
        pn = p.numpy()
        shifted = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale, o_for_d=o + e)
        _close(shifted[0] - got[0], -scale * dd[:, None] * (pn @ k), tol=1e-12, what="dQ shift from D")
        _close(shifted[1] - got[1], -scale * (pn * dd[:, None]).T @ q, tol=1e-12, what="dK shift from D")
        _close(shifted[2], got[2], tol=1e-13, what="dV independent of D")
        qr = np.array([0, Nq - 1, Nq // 2], dtype=np.int64)
        kc = np.array([Nkv - 1, 0, Nkv // 2], dtype=np.int64)
        sq, sk, sv = orc.attention_bwd_sampled(q, k, v, do, qr, kc, causal=causal, scale=scale, o_for_d=o + e)
        _close(sq, shifted[0][qr], tol=1e-12, what="sampled dQ rows, D from O")
        _close(sk, shifted[1][kc], tol=1e-12, what="sampled dK rows, D from O")
        _close(sv, shifted[2][kc], tol=1e-12, what="sampled dV rows, D from O")


# ---------------------------------------------------------------------------
# decode over a paged cache

def scatter_pages(rng, kd, vd, lens, page_size, layout, extra_pages=3, garbage=1e3):
    """Scatter dense caches kd, vd [B,H,Nmax,d] into a shuffled page pool.

    Written independently of the reference's gather: pages are drawn from a
    random permutation of the pool, the unused pool rows hold V = garbage (and
    K = 0, so that a wrongly read row gets a weight comparable to the real
    ones), and table entries past a sequence's last page are -1.  Returns
    (k_pages, v_pages, block_table)."""
    B, H, _, d = kd.shape
    need = [-(-int(n) // page_size) for n in lens]
    max_pages = max(need + [0]) + 1
    P = sum(need) + extra_pages
    perm = rng.permutation(P)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    shape = (P, H, page_size, d) if layout == "hnd" else (P, page_size, H, d)
    kp = np.zeros(shape, dtype=kd.dtype)
    vp = np.full(shape, garbage, dtype=vd.dtype)
    used = 0
    for b in range(B):
        for t in range(need[b]):
            page = perm[used]
            used += 1
            table[b, t] = page
            n_here = min(page_size, int(lens[b]) - t * page_size)
            rows = slice(t * page_size, t * page_size + n_here)
            if layout == "hnd":
                kp[page, :, :n_here] = kd[b, :, rows]
                vp[page, :, :n_here] = vd[b, :, rows]
            else:
                kp[page, :n_here] = kd[b, :, rows].transpose(1, 0, 2)
                vp[page, :n_here] = vd[b, :, rows].transpose(1, 0, 2)
    return kp, vp, table


def pin_paged_matches_dense(orc):
    # paging only changes where the keys live: the result is the dense
    # attention (pinned above) over each sequence's first lens[b] keys
    for layout in ("hnd", "nhd"):
        for page_size, lens in ((4, [1, 4, 9, 13]), (1, [3, 1, 2]), (5, [11, 5, 24, 6, 1])):
            rng = _rng(97 + page_size)
            B, H, d = len(lens), 3, 8
            Nmax = max(lens)
            q = rng.standard_normal((B, H, d))
            kd = rng.standard_normal((B, H, Nmax, d))
            vd = rng.standard_normal((B, H, Nmax, d))
            kp, vp, table = scatter_pages(rng, kd, vd, lens, page_size, layout)
            scale = 1 / math.sqrt(d)
            o, lse = orc.paged_decode(q, kp, vp, table, np.array(lens, dtype=np.int32), scale=scale, layout=layout)
            for b in range(B):
                for h in range(H):
                    n = lens[b]
                    ro, rl = orc.attention(q[b, h][None], kd[b, h, :n], vd[b, h, :n], causal=False, scale=scale)
                    _close(o[b, h], ro[0], what=f"paged {layout} ps={page_size} O ({b},{h})")
                    _close(lse[b, h], rl[0], what=f"paged {layout} ps={page_size} LSE ({b},{h})")


def pin_paged_empty_and_single(orc):
    # a sequence with one key returns that key's value row and LSE = its
    # score; a sequence with no key returns O = 0, LSE = -inf
    rng = _rng(101)
    B, H, d, page_size = 3, 2, 4, 2
    lens = [1, 0, 3]
    q = rng.standard_normal((B, H, d))
    kd = rng.standard_normal((B, H, 3, d))
    vd = rng.standard_normal((B, H, 3, d))
    for layout in ("hnd", "nhd"):
        kp, vp, table = scatter_pages(rng, kd, vd, lens, page_size, layout)
        o, lse = orc.paged_decode(q, kp, vp, table, np.array(lens, dtype=np.int32), scale=0.7, layout=layout)
        for h in range(H):
            _close(o[0, h], vd[0, h, 0], what="single key O")
            _close(lse[0, h], 0.7 * float(q[0, h] @ kd[0, h, 0]), what="single key LSE")
            assert np.all(o[1, h] == 0.0) and lse[1, h] == -np.inf, (o[1, h], lse[1, h])


# ---------------------------------------------------------------------------
# FP8 (E4M3) Q and K

def _torch_e4m3_codes(x):
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_torch(orc):
    # every one of the 256 codes decodes to torch's float8_e4m3fn value
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def pin_e4m3_quantize_torch(orc):
    # in range, the rounding is torch's float8_e4m3fn cast (nearest, ties to
    # even): all finite binary16 values and a spread of bfloat16 values
    h = np.arange(65536, dtype=np.uint16)
    x = h.view(np.float16).astype(np.float64)
    keep = np.isfinite(x) & (np.abs(x) <= 448)
    ours = orc.quantize_e4m3(h[keep], "f16")
    ref = _torch_e4m3_codes(x[keep])
    assert np.array_equal(ours, ref), int(np.sum(ours != ref))
    rng = _rng(111)
    b = rng.integers(0, 65536, 20000).astype(np.uint16)
    xb = orc.widen(b, "bf16")
    kb = np.isfinite(xb) & (np.abs(xb) <= 448)
    assert np.array_equal(orc.quantize_e4m3(b[kb], "bf16"), _torch_e4m3_codes(xb[kb]))


def pin_e4m3_grid_and_saturation(orc):
    # closed forms: every E4M3 value is a fixed point, the midpoint of two
    # neighbours goes to the one with the even code, magnitudes above 448
    # (infinity included) saturate, NaN stays NaN
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = orc.e4m3_to_f64(codes)
    assert np.array_equal(orc.quantize_e4m3(vals), codes)
    pos = np.sort(orc.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    got = orc.quantize_e4m3(mids)
    lo = np.arange(0, 0x7E, dtype=np.uint8)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    big = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 479.0, 1e6, np.inf, -500.0, -np.inf])
    assert np.array_equal(orc.quantize_e4m3(big), np.array([0x7E] * 8 + [0xFE] * 2, dtype=np.uint8))
    assert (orc.quantize_e4m3(np.array([np.nan])) & 0x7F) == 0x7F


def pin_fp8_attention_identity(orc):
    # Q and K already on the E4M3 grid: quantising changes nothing, so the
    # FP8 attention equals the ordinary attention exactly
    rng = _rng(113)
    codes = rng.integers(0, 0x7E, (2, 2, 2, 24, 16)).astype(np.uint8) | (rng.integers(0, 2, (2, 2, 2, 24, 16)) << 7).astype(np.uint8)
    codes = np.where((codes >> 3) & 15 > 9, codes & 0x87, codes)  # keep magnitudes moderate
    q, k = orc.e4m3_to_f64(codes[0]), orc.e4m3_to_f64(codes[1])
    v = rng.standard_normal((2, 2, 24, 16))
    for causal in (False, True):
        o8, l8 = orc.attention_fp8qk(q, k, v, causal=causal, scale=0.3)
        o, l = orc.attention(q, k, v, causal=causal, scale=0.3)
        assert np.array_equal(o8, o) and np.array_equal(l8, l)


def pin_fp8_attention_torch(orc):
    # off the grid: torch float64 attention on torch-quantised Q and K
    import torch
    rng = _rng(117)
    B, H, Nq, Nkv, d = 1, 2, 20, 33, 32
    q = (rng.standard_normal((B, H, Nq, d)) * 1.5).astype(np.float16)
    k = (rng.standard_normal((B, H, Nkv, d)) * 1.5).astype(np.float16)
    v = rng.standard_normal((B, H, Nkv, d)).astype(np.float16)
    for causal in (False, True):
        o8, l8 = orc.attention_fp8qk(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), causal=causal,
                                     scale=0.2, dtype="f16")
        tq = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
        tk = torch.from_numpy(k.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
        tv = torch.from_numpy(v.astype(np.float64))
        s = 0.2 * tq @ tk.transpose(-1, -2)
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nkv)[None, :]
            s = s.masked_fill(j > i + (Nkv - Nq), float("-inf"))
        _close(o8, (torch.softmax(s, -1) @ tv).numpy(), tol=1e-12, what="fp8 attention O")
        _close(l8, torch.logsumexp(s, -1).numpy(), tol=1e-12, what="fp8 attention LSE")
        # and the quantisation matters: the 16-bit attention differs
        o16, _ = orc.attention(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), causal=causal, scale=0.2,
                               dtype="f16")
        assert np.max(np.abs(o16 - o8)) > 1e-4


def pin_fp8_rows_match_full(orc):
    rng = _rng(119)
    q = (rng.standard_normal((40, 16)) * 2).astype(np.float16).view(np.uint16)
    k = (rng.standard_normal((50, 16)) * 2).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((50, 16)).astype(np.float16).view(np.uint16)
    rows = np.array([0, 7, 39], dtype=np.int64)
    o, lse = orc.attention_fp8qk(q, k, v, causal=True, scale=0.25, dtype="f16")
    ro, rl = orc.attention_fp8qk_rows(q, k, v, rows, causal=True, scale=0.25, dtype="f16")
    _close(ro, o[rows], tol=1e-12, what="fp8 rows O")
    _close(rl, lse[rows], tol=1e-12, what="fp8 rows LSE")
    kc = orc.quantize_e4m3(k, "f16")
    ko, kl = orc.attention_fp8qk(q, kc, v, causal=True, scale=0.25, dtype="f16", k_codes=True)
    assert np.array_equal(ko, o) and np.array_equal(kl, lse)


PINS = [
    pin_widen_f16, pin_widen_bf16, pin_decimal_bruteforce, pin_torch_sdpa, pin_two_key_worked,
    pin_constant_v, pin_q_zero, pin_causal_row0, pin_dominant_score, pin_single_key, pin_bounds,
    pin_linearity, pin_permutation, pin_shift_invariance, pin_merge_identity, pin_rows_match_full,
    pin_head_independence, pin_widened_inputs, pin_bwd_torch_autograd, pin_bwd_finite_difference,
    pin_bwd_invariants, pin_bwd_sampled_matches_full, pin_bwd_d_from_given_o, pin_paged_matches_dense, pin_paged_empty_and_single,
    pin_e4m3_decode_torch, pin_e4m3_quantize_torch, pin_e4m3_grid_and_saturation, pin_fp8_attention_identity,
    pin_fp8_attention_torch, pin_fp8_rows_match_full,
]
