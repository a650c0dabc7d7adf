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
