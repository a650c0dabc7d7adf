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
    assert [x.seed for x in w.values()] == [0, 1, 2, 3, 4, 4]
    assert w["decode_32k_d128_paged16"].page_size == 16 and w["decode_32k_d128_paged16"].with_(
        name="decode_32k_d128", page_size=0) == w["decode_32k_d128"]
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


def test_spike_on_query():
    # the other reading of the spike workload: one Q row per head x 20, K untouched
    w = fi.WORKLOADS["prefill_16k_d128_bf16"].with_(H=2, Nq=300, Nkv=320, spike_on="query")
    q, k = fi.make_tensor(w, fi.Q), fi.make_tensor(w, fi.K)
    idx = fi.spike_indices(w)
    assert len(idx) == 2 and all(0 <= i < 300 for i in idx)
    for h, i in enumerate(idx):
        raw = fi.normals(w.seed, fi.Q, 0, h, 300, 128)
        assert np.array_equal(q[0, h, i], fi.f32_to_bits(raw[i] * np.float32(20.0), "bf16"))
        assert np.array_equal(q[0, h, (i + 1) % 300], fi.f32_to_bits(raw[(i + 1) % 300], "bf16"))
    plain = fi.make_tensor(w.with_(spike=False), fi.K)
    assert np.array_equal(k, plain)
    with pytest.raises(ValueError):
        fi.make_tensor(w.with_(spike_on="value"), fi.Q)


def test_bits_roundtrip_torch():
    bits = np.array([0x3C00, 0xC000, 0x0001], dtype=np.uint16)
    t = fi.bits_to_torch(bits, "f16")
    assert t.tolist() == [1.0, -2.0, 2.0 ** -24]
    assert np.array_equal(fi.torch_to_bits(t), bits)


def test_paged_plan_and_scatter():
    plan = fi.paged_plan(9, 5, 50, 8, ragged=True, spare_pages=4)
    assert plan.block_table.shape == (5, 7) and plan.seq_lens.dtype == np.int32
    assert ((1 <= plan.seq_lens) & (plan.seq_lens <= 50)).all()
    need = -(-plan.seq_lens // 8)
    used = np.concatenate([plan.block_table[b, :need[b]] for b in range(5)])
    # every page is used at most once, the rest of the table is -1
    assert len(set(used.tolist())) == used.size and plan.num_pages == used.size + 4
    assert all((plan.block_table[b, need[b]:] == -1).all() for b in range(5))
    assert np.array_equal(fi.paged_plan(9, 5, 50, 8, ragged=True, spare_pages=4).block_table, plan.block_table)
    rng = np.random.default_rng(0)
    x = rng.integers(0, 60000, (5, 3, 50, 4)).astype(np.uint16)
    for layout in ("hnd", "nhd"):
        pool = fi.scatter_to_pages(x, plan, layout, fill=0xFFFF)
        for b in range(5):
            for j in range(int(plan.seq_lens[b])):
                page, slot = plan.block_table[b, j // 8], j % 8
                row = pool[page, :, slot] if layout == "hnd" else pool[page, slot]
                assert np.array_equal(row, x[b, :, j])
        assert (pool == 0xFFFF).sum() == 3 * 4 * (plan.num_pages * 8 - int(plan.seq_lens.sum()))


def test_scatter_to_pages_torch_matches_numpy():
    plan = fi.paged_plan(3, 2, 32, 4, spare_pages=2)
    x = np.random.default_rng(1).integers(0, 60000, (2, 3, 32, 8)).astype(np.uint16)
    for layout in ("hnd", "nhd"):
        ref = fi.scatter_to_pages(x, plan, layout)
        got = fi.scatter_to_pages_torch(torch.from_numpy(x.view(np.int16)), plan, layout).numpy().view(np.uint16)
        used = np.unique(plan.block_table[plan.block_table >= 0])
        assert np.array_equal(got[used], ref[used])
