"""A sweep of random small shapes for the forward and decode entry points.

hypothesis draws the shapes (derandomized: the same cases on every run) --
ragged lengths that are not tile multiples, Nq != Nkv, Nq = 1, both head
dimensions and both types, causal and not, 16-bit and E4M3 K, and decode
split counts -- and each case is compared with the fp64 oracle at the usual
tolerances.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import exact_io_aware_65_amd as fa
import oracle
from gpu_util import check, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


@st.composite
def fwd_cases(draw):
    causal = draw(st.booleans())
    Nq = draw(st.integers(1, 400))
    Nkv = Nq + draw(st.integers(0, 300)) if causal else draw(st.integers(1, 700))
    return dict(B=draw(st.integers(1, 3)), H=draw(st.integers(1, 3)), Nq=Nq, Nkv=Nkv,
                d=draw(st.sampled_from([64, 128])), causal=causal, dtype=draw(st.sampled_from(["f16", "bf16"])),
                fp8=draw(st.booleans()), scale=draw(st.sampled_from([None, 0.05, -0.2])),
                seed=draw(st.integers(0, 2 ** 31 - 1)))


@SETTINGS
@given(fwd_cases())
def test_fwd_random_shapes(c):
    rng = np.random.default_rng(c["seed"])
    B, H, Nq, Nkv, d, dtype = c["B"], c["H"], c["Nq"], c["Nkv"], c["d"], c["dtype"]
    q, k, v = (rand_bits(rng, (B, H, n, d), dtype) for n in (Nq, Nkv, Nkv))
    scale = float(np.float32(1 / np.sqrt(d) if c["scale"] is None else c["scale"]))
    say(f"random fwd {c}")
    run = fa.fwd_fp8 if c["fp8"] else fa.fwd
    o, lse = run(upload(q, dtype), upload(k, dtype), upload(v, dtype), causal=c["causal"], scale=scale,
                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attention_fp8qk if c["fp8"] else oracle.attention
    o_ref, lse_ref = ref(q, k, v, causal=c["causal"], scale=scale, dtype=dtype)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"random fwd {c}")


@st.composite
def decode_cases(draw):
    return dict(B=draw(st.integers(1, 4)), H=draw(st.integers(1, 4)), Nkv=draw(st.integers(1, 5000)),
                d=draw(st.sampled_from([64, 128])), dtype=draw(st.sampled_from(["f16", "bf16"])),
                splits=draw(st.sampled_from([0, 1, 2, 5, 33])), seed=draw(st.integers(0, 2 ** 31 - 1)))


@SETTINGS
@given(decode_cases())
def test_decode_random_shapes(c):
    rng = np.random.default_rng(c["seed"])
    B, H, Nkv, d, dtype = c["B"], c["H"], c["Nkv"], c["d"], c["dtype"]
    q = rand_bits(rng, (B, H, 1, d), dtype)
    k, v = (rand_bits(rng, (B, H, Nkv, d), dtype) for _ in range(2))
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"random decode {c}")
    o, lse = fa.decode(upload(q[:, :, 0], dtype), upload(k, dtype), upload(v, dtype), scale=scale,
                       num_splits=c["splits"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=scale, dtype=dtype)
    check(to_np(o), to_np(lse), o_ref[:, :, 0], lse_ref[:, :, 0], dtype, f"random decode {c}")
