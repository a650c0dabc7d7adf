"""The unfused baseline of the speed-vs-length sweep computes the same attention.

bench.unfused_attention / unfused_decode (library GEMMs and softmax, S and P
materialised in 16 bits) are compared with the fp64 oracle.  Their 16-bit S
and P make them less accurate than the fused kernels, so the bar is looser:
max |O error| <= 1e-2 (fp16 inputs); the fused kernels keep theirs.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from gpu_util import rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", [(1, 2, 300, 300, 128, True), (2, 1, 100, 257, 64, True),
                                  (1, 3, 64, 200, 128, False)])
def test_unfused_attention_matches_oracle(case):
    B, H, Nq, Nkv, d, causal = case
    rng = np.random.default_rng(71)
    q = rand_bits(rng, (B, H, Nq, d), "f16", sigma=1.5)
    k = rand_bits(rng, (B, H, Nkv, d), "f16", sigma=1.5)
    v = rand_bits(rng, (B, H, Nkv, d), "f16")
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"unfused attention {case}")
    o = bench.unfused_attention(upload(q, "f16"), upload(k, "f16"), upload(v, "f16"), causal, scale)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention(q, k, v, causal=causal, scale=scale, dtype="f16")
    err = float(np.max(np.abs(to_np(o) - o_ref)))
    say(f"unfused attention {case}: max err {err:.2e}")
    assert err <= 1e-2, err


def test_unfused_decode_matches_oracle():
    rng = np.random.default_rng(73)
    B, H, N, d = 3, 2, 700, 128
    q = rand_bits(rng, (B, H, d), "f16")
    k = rand_bits(rng, (B, H, N, d), "f16")
    v = rand_bits(rng, (B, H, N, d), "f16")
    say("unfused decode")
    o = bench.unfused_decode(upload(q, "f16"), upload(k, "f16"), upload(v, "f16"), 0.09)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention(q[:, :, None], k, v, causal=False, scale=0.09, dtype="f16")
    err = float(np.max(np.abs(to_np(o) - o_ref[:, :, 0])))
    assert err <= 1e-2, err
