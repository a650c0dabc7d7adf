"""The seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

import fa_inputs as fi


def test_workload_table():
    w = fi.WORKLOADS
    assert (w["tiny_256_d64"].B, w["tiny_256_d64"].H, w["tiny_256_d64"].Nq, w["tiny_256_d64"].d) == (1, 2, 256, 64)
    assert w["tiny_256_d64"].out_f32 and not w["tiny_256_d64"].causal and w["tiny_256_d64"].seed == 0
    assert (w["prefill_8k_d128"].H, w["prefill_8k_d128"].Nq, w["prefill_8k_d128"].sigma_qk) == (32, 8192, 1.5)
    assert w["prefill_16k_d128_bf16"].dtype == "bf16" and w["prefill_16k_d128_bf16"].spike
    assert w["decode_32k_d128"].Nq == 1 and w["decode_32k_d128"].Nkv == 32768 and w["decode_32k_d128"].decode
    assert [x.seed for x in w.values()] == [0, 1, 2, 3, 4]
    assert w["prefill_8k_d128"].scale == float(np.float32(1 / np.sqrt(128)))


def test_deterministic_and_head_order_free():
    w = fi.WORKLOADS["tiny_256_d64"].with_(H=3, B=2, Nq=40, Nkv=50)
    a = fi.make_inputs(w)
    b = fi.make_inputs(w)
    for t in "qkv":
        assert np.array_equal(a[t], b[t])
    q, k, v = fi.head_inputs(w, 1, 2)
    assert np.array_equal(q, a["q"][1, 2]) and np.array_equal(k, a["k"][1, 2]) and np.array_equal(v, a["v"][1, 2])
    assert a["q"].shape == (2, 3, 40, 64) and a["k"].shape == (2, 3, 50, 64)


def test_moments_and_sigma():
    w = fi.WORKLOADS["prefill_8k_d128"].with_(H=2, Nq=2048, Nkv=2048)
    x = fi.make_tensor(w, fi.Q).view(np.float16).astype(np.float64)
    y = fi.make_tensor(w, fi.V).view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.5) < 0.01
    assert abs(y.mean()) < 0.01 and abs(y.std() - 1.0) < 0.01


def test_bf16_cast_is_round_to_nearest_even():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 3).astype(np.float32)
    # include exact ties: values half-way between two bf16 numbers
    ties = (np.arange(1, 1001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = fi.f32_to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(fi.f32_to_bits(x, "f16"), x.astype(np.float16).view(np.uint16))


def test_spike_row():
    w = fi.WORKLOADS["prefill_16k_d128_bf16"].with_(H=2, Nq=300, Nkv=300)
    k = fi.make_tensor(w, fi.K)
    idx = fi.spike_indices(w)
    assert len(idx) == 2 and all(0 <= j < 300 for j in idx)
    for h, j in enumerate(idx):
        raw = fi.normals(w.seed, fi.K, 0, h, 300, 128)
        assert np.array_equal(k[0, h, j], fi.f32_to_bits(raw[j] * np.float32(20.0), "bf16"))
        other = (j + 1) % 300
        assert np.array_equal(k[0, h, other], fi.f32_to_bits(raw[other], "bf16"))


def test_bits_roundtrip_torch():
    bits = np.array([0x3C00, 0xC000, 0x0001], dtype=np.uint16)
    t = fi.bits_to_torch(bits, "f16")
    assert t.tolist() == [1.0, -2.0, 2.0 ** -24]
    assert np.array_equal(fi.torch_to_bits(t), bits)
