"""Maximum sizes: heads just under the library's 4 GiB-per-head limit.

One head of K and V (or of Q and O) may span up to 4 GiB, while whole tensors
may be larger, with head bases past 2^32 bytes.  Two heads of 2^24 - 48 keys
(d = 128, fp16: 4 GiB - 12 KiB each) put the second head's base past 4 GiB
and make the key offsets inside each head reach the top of the 32-bit range;
the second case does the same with 2^24 - 37 query rows.  Both lengths are
ragged against the kernels' tiles.

Inputs come from the seeded generator at full size.  The oracle computes
sampled rows over every key of a head (the rows past 2^23, whose byte offsets
pass 2^31, are among them).  Tolerances are those of every other parity
test.  Over 16M unit-normal keys at scale 1/sqrt(d), |O| is about 3e-4, below
the O tolerance, so a key read from a wrong address would go unseen; the key
case therefore uses scale 0.5 (score std ~5.7), where a few dozen keys
scattered over the whole head carry the softmax and |O| is of order 0.1-1.
Each case draws and widens 2^31-element tensors on the host, so together
they take a minute or two.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import check, device, say, to_np, upload

pytestmark = pytest.mark.gpu

NKV_MAX = (1 << 24) - 48   # a whole number of 16-key pages, 16 keys into a 64-key tile
NQ_MAX = (1 << 24) - 37    # 27 rows into a 64-row tile
D = 128
PEAKED = 0.5


def _ints(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device())


def test_keys_at_the_per_head_limit():
    w = fi.Workload("max_keys_d128", B=1, H=2, Nq=64, Nkv=NKV_MAX, d=D, dtype="f16", causal=False, seed=23)
    head_bytes = w.Nkv * w.d * 2
    assert (1 << 32) - (1 << 14) < head_bytes < (1 << 32)
    say(f"generate {w.name}: K and V of {w.H} heads x {w.Nkv} keys ({head_bytes} bytes per head)")
    x = fi.make_inputs(w)
    tq, tk, tv = (upload(x[t], w.dtype) for t in "qkv")
    say("fa_fwd at the per-head key limit, non-causal and causal")
    o_n, l_n = fa.fwd(tq, tk, tv, causal=False, scale=PEAKED, out_dtype=torch.float32)
    o_c, l_c = fa.fwd(tq, tk, tv, causal=True, scale=PEAKED, out_dtype=torch.float32)
    # the last query row sees every key, causal or not: it is also the decode query
    qd = tq[:, :, -1].contiguous()
    say("fa_decode at the per-head key limit")
    o_d, l_d = fa.decode(qd, tk, tv, scale=PEAKED, out_dtype=torch.float32)
    plan = fi.paged_plan(w.seed, w.B, w.Nkv, 16)
    kp, vp = fi.scatter_to_pages_torch(tk, plan), fi.scatter_to_pages_torch(tv, plan)
    say(f"fa_decode_paged at the per-head key limit: {plan.num_pages} pages of 16 keys, pools past 8 GiB")
    o_p, l_p = fa.decode_paged(qd, kp, vp, _ints(plan.block_table), _ints(plan.seq_lens), max_seq_len=w.Nkv,
                               scale=PEAKED, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the same keys in the same order with the same split count: the same bits
    assert torch.equal(o_p, o_d) and torch.equal(l_p, l_d)
    del kp, vp, tk, tv
    o_n, l_n, o_c, l_c, o_d, l_d = (to_np(t) for t in (o_n, l_n, o_c, l_c, o_d, l_d))
    last = w.Nq - 1
    for h in range(w.H):
        say(f"oracle: head {h}, widen {w.Nkv} keys")
        qh, kh, vh = (oracle.widen(x[t][0, h], w.dtype) for t in "qkv")
        rows = np.array([0, 31, last], dtype=np.int64)
        ro, rl = oracle.attention_rows(qh, kh, vh, rows, causal=False, scale=PEAKED)
        assert np.abs(ro).max(axis=1).min() > 0.1, "the check no longer tells key sets apart"
        check(o_n[0, h, rows], l_n[0, h, rows], ro, rl, w.dtype, f"fwd, max keys, head {h}")
        check(o_c[0, h, last:], l_c[0, h, last:], ro[-1:], rl[-1:], w.dtype, f"causal fwd last row, head {h}")
        check(o_d[0, h:h + 1], l_d[0, h:h + 1], ro[-1:], rl[-1:], w.dtype, f"decode, max keys, head {h}")
        if h == w.H - 1:
            # causal rows: row i sees the first Nkv - Nq + 1 + i keys
            rc = np.array([0, 32], dtype=np.int64)
            co, cl = oracle.attention_rows(qh, kh, vh, rc, causal=True, scale=PEAKED)
            check(o_c[0, h, rc], l_c[0, h, rc], co, cl, w.dtype, f"causal fwd, max keys, head {h}")
        del qh, kh, vh


def test_queries_at_the_per_head_limit():
    w = fi.Workload("max_queries_d128", B=1, H=2, Nq=NQ_MAX, Nkv=200, d=D, dtype="f16", causal=False, seed=24)
    head_bytes = w.Nq * w.d * 2
    assert (1 << 32) - (1 << 14) < head_bytes < (1 << 32)
    say(f"generate {w.name}: Q of {w.H} heads x {w.Nq} rows ({head_bytes} bytes per head)")
    x = fi.make_inputs(w)
    tq, tk, tv = (upload(x[t], w.dtype) for t in "qkv")
    say("fa_fwd at the per-head query limit (fp16 O)")
    o, lse = fa.fwd(tq, tk, tv, causal=False, scale=w.scale)
    say("fa_fwd_fp8 at the per-head query limit (fp16 O)")
    o8, lse8 = fa.fwd_fp8(tq, tk, tv, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    for t in (o, lse, o8, lse8):
        assert torch.isfinite(t).all()
    rng = np.random.default_rng(w.seed)
    n, half = w.Nq, 1 << 23
    rows = np.unique(np.concatenate([[0, 1, half - 1, half, half + 1, n - 28, n - 2, n - 1],
                                     rng.integers(0, n, 6)])).astype(np.int64)
    idx = torch.from_numpy(rows).to(device())
    for h in range(w.H):
        say(f"oracle: head {h}, {rows.size} sampled rows")
        qs = x["q"][0, h][rows]  # without a mask the rows are independent
        ro, rl = oracle.attention(qs, x["k"][0, h], x["v"][0, h], causal=False, scale=w.scale, dtype=w.dtype)
        check(to_np(o[0, h][idx]), to_np(lse[0, h][idx]), ro, rl, w.dtype, f"fwd, max queries, head {h}")
        codes = oracle.quantize_e4m3(x["k"][0, h], w.dtype)
        fo, fl = oracle.attention_fp8qk(qs, codes, x["v"][0, h], causal=False, scale=w.scale, dtype=w.dtype,
                                        k_codes=True)
        check(to_np(o8[0, h][idx]), to_np(lse8[0, h][idx]), fo, fl, w.dtype, f"fwd_fp8, max queries, head {h}")
