"""GPU parity of decode over a paged cache (fa_decode_paged) against the fp64 oracle.

Pools come from the seeded page plans of fa_inputs (shuffled page order,
ragged lengths, unused slots filled with loud values); the oracle gathers the
same pool through the same table.  Tolerances as for dense decode: O within
2e-3 (fp16) / 1.5e-2 (bf16), LSE within 1e-3.  Where the paged call sees the
same keys in the same order as a dense fa_decode call with the same split
count (full-length sequences, max_seq_len = Nkv), the kernels perform the same
arithmetic, so the outputs must match bit for bit.
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import check, device, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu

LOUD = {"f16": 0x5E00, "bf16": 0x4580}  # 384 / 4096: a wrongly read slot shows at once


def _ints(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device())


def _pools(rng, B, H, Nmax, d, dtype, plan, layout):
    q = rand_bits(rng, (B, H, d), dtype)
    k = rand_bits(rng, (B, H, Nmax, d), dtype)
    v = rand_bits(rng, (B, H, Nmax, d), dtype)
    kp = fi.scatter_to_pages(k, plan, layout, fill=0)
    vp = fi.scatter_to_pages(v, plan, layout, fill=LOUD[dtype])
    return q, k, v, kp, vp


CASES = [
    # B, H, d, max_len, page_size, lens (None: drawn ragged), layout, dtype
    (4, 2, 128, 300, 16, None, "hnd", "f16"),
    (3, 3, 64, 257, 1, None, "nhd", "f16"),
    (5, 2, 128, 500, 7, [1, 500, 0, 64, 333], "hnd", "bf16"),
    (2, 4, 64, 1024, 64, [1024, 999], "nhd", "bf16"),
    (6, 1, 128, 90, 3, None, "nhd", "f16"),
    (1, 2, 128, 4096, 16, [4096], "hnd", "f16"),
    (8, 2, 64, 2000, 48, None, "hnd", "f16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}d{}n{}ps{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[6], c[7]))
def test_paged_decode_small(case):
    B, H, d, max_len, ps, lens, layout, dtype = case
    seed = zlib.crc32(repr(case).encode())
    plan = fi.paged_plan(seed, B, max_len, ps, ragged=lens is None, spare_pages=3, lens=lens)
    rng = np.random.default_rng(seed)
    q, _, _, kp, vp = _pools(rng, B, H, max_len, d, dtype, plan, layout)
    scale = float(np.float32(1 / np.sqrt(d)))
    o_ref, lse_ref = oracle.paged_decode(q, kp, vp, plan.block_table, plan.seq_lens, scale=scale, layout=layout,
                                         dtype=dtype)
    tq, tkp, tvp = upload(q, dtype), upload(kp, dtype), upload(vp, dtype)
    table, lens_t = _ints(plan.block_table), _ints(plan.seq_lens)
    empty = plan.seq_lens == 0
    for splits in (0, 1, 5):
        for bound in (max_len, int(plan.seq_lens.max()) or 1):
            say(f"fa_decode_paged {case} splits={splits} max_seq_len={bound}")
            o, lse = fa.decode_paged(tq, tkp, tvp, table, lens_t, layout=layout, max_seq_len=bound, scale=scale,
                                     num_splits=splits, out_dtype=torch.float32)
            torch.cuda.synchronize()
            o, lse = to_np(o), to_np(lse)
            assert (o[empty] == 0).all() and (lse[empty] == -np.inf).all()
            live = ~empty
            check(o[live], lse[live], o_ref[live], lse_ref[live], dtype, f"paged {case} splits={splits} bound={bound}")
    # native output = the fp32 result rounded to nearest even
    o16, _ = fa.decode_paged(tq, tkp, tvp, table, lens_t, layout=layout, scale=scale)
    o32, _ = fa.decode_paged(tq, tkp, tvp, table, lens_t, layout=layout, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o16.float(), o32.to(o16.dtype).float())


def test_paged_equals_dense_bitwise():
    # full-length sequences through a shuffled table: the same keys in the same
    # order and the same splits as the dense call, hence the same bits
    rng = np.random.default_rng(41)
    B, H, N, d, dtype = 3, 4, 1000, 128, "f16"
    plan = fi.paged_plan(41, B, N, 16, spare_pages=5)
    q, k, v, kp, vp = _pools(rng, B, H, N, d, dtype, plan, "nhd")
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    tkp, tvp = upload(kp, dtype), upload(vp, dtype)
    table, lens = _ints(plan.block_table), _ints(plan.seq_lens)
    for splits in (0, 3):
        say(f"paged vs dense splits={splits}")
        od, ld = fa.decode(tq, tk, tv, scale=0.09, num_splits=splits)
        op, lp = fa.decode_paged(tq, tkp, tvp, table, lens, layout="nhd", max_seq_len=N, scale=0.09,
                                 num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(od, op) and torch.equal(ld, lp)


def test_paged_clamps_device_values():
    # lengths and page indices live on the device, so the kernel clamps them:
    # a length above max_seq_len counts as max_seq_len, a negative one as 0,
    # and a page index outside the pool reads the nearest pool page
    rng = np.random.default_rng(43)
    B, H, N, d, ps, dtype = 4, 2, 64, 64, 8, "f16"
    plan = fi.paged_plan(43, B, N, ps, lens=[64, 40, 10, 64])
    q, _, _, kp, vp = _pools(rng, B, H, N, d, dtype, plan, "hnd")
    table = plan.block_table.copy()
    table[0, 2] = plan.num_pages + 7     # used entry beyond the pool
    table[2, 1] = -5                     # used entry below it
    lens = np.array([64 + 100, 40, 10, -3], dtype=np.int32)
    # what the clamped call must equal
    table_c = table.copy()
    table_c[0, 2] = plan.num_pages - 1
    table_c[2, 1] = 0
    lens_c = np.array([64, 40, 10, 0], dtype=np.int32)
    o_ref, lse_ref = oracle.paged_decode(q, kp, vp, table_c, lens_c, scale=0.125, layout="hnd", dtype=dtype)
    say("fa_decode_paged clamped lengths and pages")
    o, lse = fa.decode_paged(upload(q, dtype), upload(kp, dtype), upload(vp, dtype), _ints(table), _ints(lens),
                             max_seq_len=N, scale=0.125, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    assert (o[3] == 0).all() and (lse[3] == -np.inf).all()
    check(o[:3], lse[:3], o_ref[:3], lse_ref[:3], dtype, "clamped")


def test_full_size_paged_decode():
    # the benchmark's paged workload at full size: bitwise equal to the dense
    # decode of the same cache, and sampled heads against the oracle
    w = fi.WORKLOADS["decode_32k_d128_paged16"]
    plan = fi.workload_plan(w)
    say("generate decode_32k_d128_paged16")
    x = fi.make_inputs(w)
    tq = upload(x["q"][:, :, 0], w.dtype)
    tk, tv = upload(x["k"], w.dtype), upload(x["v"], w.dtype)
    tkp, tvp = fi.scatter_to_pages_torch(tk, plan), fi.scatter_to_pages_torch(tv, plan)
    table, lens = _ints(plan.block_table), _ints(plan.seq_lens)
    say("fa_decode_paged decode_32k_d128_paged16 (benchmark configuration)")
    op, lp = fa.decode_paged(tq, tkp, tvp, table, lens, max_seq_len=w.Nkv, scale=w.scale)
    od, ld = fa.decode(tq, tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(op, od) and torch.equal(lp, ld)
    o32, l32 = fa.decode_paged(tq, tkp, tvp, table, lens, max_seq_len=w.Nkv, scale=w.scale,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    o32, l32 = to_np(o32), to_np(l32)
    for b, h in ((0, 0), (7, 19), (15, 31)):
        o_ref, lse_ref = oracle.attention(x["q"][b, h], x["k"][b, h], x["v"][b, h], causal=False, scale=w.scale,
                                          dtype=w.dtype)
        check(o32[b, h], l32[b, h][None], o_ref[0], lse_ref, w.dtype, f"paged full size head ({b},{h})")


def test_full_size_ragged_paged_decode():
    # ragged lengths up to 32K, page size 16, a shuffled pool; sampled heads
    # against the oracle over each sequence's prefix
    w = fi.WORKLOADS["decode_32k_d128_paged16"].with_(B=8, H=8, ragged=True)
    plan = fi.workload_plan(w)
    say(f"generate ragged paged decode lens={plan.seq_lens.tolist()}")
    x = fi.make_inputs(w)
    kp, vp = fi.scatter_to_pages(x["k"], plan), fi.scatter_to_pages(x["v"], plan)
    say("fa_decode_paged ragged 32K")
    o, lse = fa.decode_paged(upload(x["q"][:, :, 0], w.dtype), upload(kp, w.dtype), upload(vp, w.dtype),
                             _ints(plan.block_table), _ints(plan.seq_lens), max_seq_len=w.Nkv, scale=w.scale,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    for b, h in ((0, 3), (3, 0), (5, 7), (7, 5)):
        n = int(plan.seq_lens[b])
        o_ref, lse_ref = oracle.attention(x["q"][b, h], x["k"][b, h, :n], x["v"][b, h, :n], causal=False,
                                          scale=w.scale, dtype=w.dtype)
        check(o[b, h], lse[b, h][None], o_ref[0], lse_ref, w.dtype, f"ragged head ({b},{h}) n={n}")
