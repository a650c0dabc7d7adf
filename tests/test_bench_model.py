"""The benchmark's byte and FLOP models, and the parity comparator itself (CPU only).

The score-matrix sizes and the unfused traffic figure are the numbers the
pages print (tests/golden/score_matrix_bytes.json, each with its source); the
FLOP and byte counts of the benchmark workloads are their closed forms.
"""
import json
import os

import numpy as np
import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "score_matrix_bytes.json")


def test_score_matrix_bytes_match_the_pages():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        assert bench.score_matrix_bytes(case["n"], case["bytes_per_element"]) == case["bytes"], case["source"]
    u = g["unfused_traffic"]
    # S written once and read once: printed as 268 MB (decimal, three figures)
    s_bytes = 2 * bench.score_matrix_bytes(u["N"], u["bytes_per_element"])
    assert round(s_bytes / 1e6) == u["s_write_read_mb"]


def test_workload_flops_and_bytes():
    # prefill 1 x 32 x 8192 x 128 causal: 4 B H N^2 d / 2
    assert bench.metric_flops(1, 32, 8192, 8192, 128, True) == 549_755_813_888
    assert bench.metric_flops(1, 32, 8192, 8192, 128, False) == 2 * 549_755_813_888
    # read Q, K, V once, write O (fp16) and LSE (fp32) once
    assert bench.algorithmic_bytes(1, 32, 8192, 8192, 128) == 32 * (2 * 3 * 8192 * 128 + 2 * 8192 * 128 + 4 * 8192)
    assert bench.algorithmic_bytes(1, 32, 8192, 8192, 128) == 269_484_032
    # decode 16 x 32 heads x 32768 keys: the 8 GiB cache dominates
    assert bench.algorithmic_bytes(16, 32, 1, 32768, 128) == 8_590_198_784
    # backward: Q, K, V, O, dO, LSE read; dQ, dK, dV written
    assert bench.backward_bytes(1, 32, 8192, 8192, 128) == 32 * (2 * 8 * 8192 * 128 + 4 * 8192)
    assert bench.backward_flops(1, 32, 8192, 8192, 128, True) == 549_755_813_888 * 5 // 2


def test_comparator_fails_on_one_bad_element():
    # the parity check must notice a single element off by ten tolerances, an
    # LSE off by as much, and a NaN; and pass the unperturbed arrays
    from gpu_util import TOL_LSE, TOL_O, check
    rng = np.random.default_rng(5)
    o_ref = rng.standard_normal((2, 3, 17, 8))
    lse_ref = rng.standard_normal((2, 3, 17))
    for dtype in ("f16", "bf16"):
        check(o_ref.copy(), lse_ref.copy(), o_ref, lse_ref, dtype, "unperturbed")
        o = o_ref.copy()
        o[1, 2, 16, 7] += 10 * TOL_O[dtype]
        with pytest.raises(AssertionError):
            check(o, lse_ref, o_ref, lse_ref, dtype, "one O element")
        lse = lse_ref.copy()
        lse[0, 1, 3] -= 10 * TOL_LSE
        with pytest.raises(AssertionError):
            check(o_ref, lse, o_ref, lse_ref, dtype, "one LSE element")
        o = o_ref.copy()
        o[0, 0, 0, 0] = np.nan
        with pytest.raises(AssertionError):
            check(o, lse_ref, o_ref, lse_ref, dtype, "NaN")


def test_bench_comparator_names_the_worst_element():
    # the bench's record of the timed outputs: the worst element's index across
    # heads added one at a time, pass/fail at the stated tolerance, NaN fails,
    # and the relative form used for the backward's gradients
    rng = np.random.default_rng(6)
    ref = rng.standard_normal((4, 5, 3))
    w = bench.Worst()
    for h in range(4):
        got = ref[h].copy()
        if h == 2:
            got[3, 1] += 0.5
        w.add(got, ref[h], (0, h))
    rec, ok = w.record("O", tol=0.1)
    assert rec["err_O"] == pytest.approx(0.5) and rec["worst_O"] == [0, 2, 3, 1] and not ok
    assert w.record("O", tol=1.0)[1]
    rec, ok = w.record("O", rel=0.5 / np.max(np.abs(ref)) * 1.01)
    assert ok and rec["err_O_rel"] == pytest.approx(0.5 / np.max(np.abs(ref)))
    w.add(np.array([np.nan]), np.array([0.0]), (9,))
    assert not w.record("O", tol=1e9)[1]


def test_bench_paged_oracle_leg_compares_each_sequence():
    # the paged decode leg's oracle comparison on host tensors: each sequence
    # through the oracle over the pool pages its table names (renumbered), the
    # timed O taken as [B, H, 1, d]; a planted error is found at its index
    import types

    import torch

    import fa_inputs as fi
    import oracle
    w = types.SimpleNamespace(B=3, H=2, d=64, dtype="f16", scale=0.125, name="paged_tiny")
    plan = fi.paged_plan(5, w.B, 40, 16, ragged=True)
    g = torch.Generator().manual_seed(8)
    kp = torch.randn((plan.num_pages, w.H, plan.page_size, w.d), generator=g).half()
    vp = torch.randn((plan.num_pages, w.H, plan.page_size, w.d), generator=g).half()
    q = torch.randn((w.B, w.H, 1, w.d), generator=g).half()
    o_ref, lse_ref = oracle.paged_decode(fi.torch_to_bits(q.reshape(w.B, w.H, w.d)), fi.torch_to_bits(kp),
                                         fi.torch_to_bits(vp), plan.block_table, plan.seq_lens, scale=w.scale,
                                         layout="hnd", dtype="f16")
    o = torch.from_numpy(o_ref).half().reshape(w.B, w.H, 1, w.d)
    lse = torch.from_numpy(lse_ref).float()
    rec = bench.oracle_paged_leg(w, plan, q, kp, vp, o, lse, 100.0)
    assert rec["parity"]["pass"] and rec["parity"]["err_O"] <= 2.0 ** -11
    assert rec["cpu_baseline"]["kind"] == "oracle" and "3 of 3 sequences" in rec["cpu_baseline"]["sample"]
    o[1, 1, 0, 5] += 0.5
    rec = bench.oracle_paged_leg(w, plan, q, kp, vp, o, lse, 100.0)
    assert not rec["parity"]["pass"] and rec["parity"]["worst_O"] == [1, 1, 5]
