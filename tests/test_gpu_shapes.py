"""Parity at the boundaries where the forward changes launch shape.

The host picks a workgroup geometry from the grid size:
- 8 waves (256 query rows) once B*H*ceil(Nq/256) >= 256, 16-bit K only, and
  causal at d = 64 only from B*H*ceil(Nq/256) >= 512 (4 waves below that);
- two 4-wave key groups on 128 rows once B*H*ceil(Nq/128) <= 256 and Nkv > 192,
  or, causal at d = 64 with 16-bit K, two 2-wave key groups on 64 rows;
- 4 waves (128 rows) otherwise, and always for E4M3 K when the grid is large.

Each case below sits on one side of one of those thresholds (the shape each
selects is noted), for fa_fwd and fa_fwd_fp8, against the fp64 oracle at the
usual tolerances.  A wrong threshold would send these shapes to a geometry
the other tests never reach at that size.
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import oracle
from gpu_util import check, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, Nq, Nkv, d, causal, dtype    16-bit K shape / E4M3 K shape
    (1, 128, 512, 512, 128, True, "f16"),   # 8 waves: exactly 256 wide blocks / 4 waves
    (1, 255, 256, 256, 64, False, "bf16"),  # 4 waves: 255 wide blocks, 510 tiles / 4 waves
    (1, 256, 128, 193, 64, True, "f16"),    # 4 waves: 256 wide blocks, causal d = 64 / key groups: 256 tiles, 193 keys
    (1, 256, 128, 192, 64, True, "bf16"),   # 4 waves: 256 wide blocks, causal d = 64 / 4 waves: 192 keys
    (1, 256, 512, 512, 64, True, "f16"),    # 8 waves: 512 wide blocks, causal d = 64 / 4 waves
    (1, 255, 512, 600, 64, True, "bf16"),   # 4 waves: 510 wide blocks, causal d = 64, Nq < Nkv (both)
    (1, 256, 128, 193, 64, False, "f16"),   # 8 waves: 256 wide blocks, no mask / key groups
    (1, 128, 256, 193, 128, False, "bf16"),  # key groups: 256 tiles, 193 keys (both)
    (1, 128, 256, 192, 128, False, "f16"),  # 4 waves: 192 keys (both)
    (1, 129, 256, 400, 64, True, "bf16"),   # 4 waves: 258 tiles (both)
    (2, 64, 200, 1000, 128, True, "f16"),   # key groups, causal with Nq < Nkv (both)
    # causal d = 64 small grids: 64-row tiles of two 2-wave key groups (16-bit K)
    (1, 128, 256, 256, 64, True, "bf16"),   # 64-row key groups: 256 tiles / key groups
    (1, 129, 256, 256, 64, True, "f16"),    # 4 waves: 258 tiles (both)
    (1, 3, 300, 1000, 64, True, "f16"),     # 64-row key groups, ragged last tile, Nq < Nkv / key groups
    (2, 5, 40, 193, 64, True, "bf16"),      # 64-row key groups, one tile whose second wave has 8 rows
    (1, 8, 130, 192, 64, True, "f16"),      # 4 waves: 192 keys (both)
]


def _ids(c):
    return "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6])


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_launch_shape_boundaries(case):
    B, H, Nq, Nkv, d, causal, dtype = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q = rand_bits(rng, (B, H, Nq, d), dtype)
    k = rand_bits(rng, (B, H, Nkv, d), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    say(f"fa_fwd and fa_fwd_fp8 at a launch-shape boundary {case}")
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale, out_dtype=torch.float32)
    o8, lse8 = fa.fwd_fp8(tq, tk, tv, causal=causal, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, scale=scale, dtype=dtype)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"fwd {case}")
    o_ref, lse_ref = oracle.attention_fp8qk(q, k, v, causal=causal, scale=scale, dtype=dtype)
    check(to_np(o8), to_np(lse8), o_ref, lse_ref, dtype, f"fwd_fp8 {case}")
