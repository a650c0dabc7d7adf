"""Helpers for the GPU parity tests: upload seeded bits, run the library, compare with the oracle.

Tolerances (max absolute error against the fp64 reference): O within 2e-3 for
fp16 inputs and 1.5e-2 for bf16 inputs, LSE within 1e-3; any NaN fails.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi

TOL_O = {"f16": 2e-3, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def say(msg: str):
    """Name the GPU step about to run, unbuffered, so a crash report shows it."""
    print(f"[gpu] {msg}", file=sys.__stderr__, flush=True)


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def upload(bits: np.ndarray, dtype: str):
    return fi.bits_to_torch(bits, dtype).to(device())


def rand_bits(rng, shape, dtype, sigma=1.0):
    return fi.f32_to_bits((rng.standard_normal(shape) * sigma).astype(np.float32), dtype)


def max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert not np.isnan(got).any(), "NaN in GPU output"
    if got.size == 0:
        return 0.0, None
    diff = np.abs(got - ref)
    worst = np.unravel_index(int(np.argmax(diff)), diff.shape)
    return float(diff[worst]), tuple(int(i) for i in worst)


def mean_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return float(np.mean(np.abs(got - np.asarray(ref, dtype=np.float64)))) if got.size else 0.0


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what):
    eo, wo = max_err(o_gpu, o_ref)
    el, wl = max_err(lse_gpu, lse_ref)
    say(f"{what}: err_O={eo:.3e} at {wo} (mean {mean_err(o_gpu, o_ref):.2e}), "
        f"err_LSE={el:.3e} at {wl} (mean {mean_err(lse_gpu, lse_ref):.2e})")
    assert eo <= TOL_O[dtype], f"{what}: O error {eo:.3e} at {wo} exceeds {TOL_O[dtype]}"
    assert el <= TOL_LSE, f"{what}: LSE error {el:.3e} at {wl} exceeds {TOL_LSE}"
    return eo, el


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_fwd(q, k, v, causal, scale, dtype, out_f32=True):
    """q, k, v: uint16 bits [B,H,N,d].  Returns (o, lse) as float64 numpy arrays."""
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale,
                    out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)
