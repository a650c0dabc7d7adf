"""API paths of the C ABI on the GPU: optional LSE, caller streams, shared workspaces.

Each check compares one call path with another whose parity against the
oracle is covered elsewhere, bit for bit: the kernels are deterministic, so a
path that only changes plumbing must not change a single output bit.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
from gpu_util import device, rand_bits, say, upload

pytestmark = pytest.mark.gpu


def _qkv(seed, B, H, Nq, Nkv, d, dtype="f16"):
    rng = np.random.default_rng(seed)
    return (upload(rand_bits(rng, (B, H, Nq, d), dtype), dtype), upload(rand_bits(rng, (B, H, Nkv, d), dtype), dtype),
            upload(rand_bits(rng, (B, H, Nkv, d), dtype), dtype))


def test_fwd_without_lse():
    for case in ((1, 4, 300, 300, 128, True), (2, 2, 77, 500, 64, False), (1, 64, 512, 512, 128, True)):
        B, H, Nq, Nkv, d, causal = case
        q, k, v = _qkv(11, B, H, Nq, Nkv, d)
        say(f"fa_fwd lse=NULL {case}")
        o1, lse = fa.fwd(q, k, v, causal=causal)
        o2, none = fa.fwd(q, k, v, causal=causal, with_lse=False)
        o3, _ = fa.fwd_fp8(q, k, v, causal=causal)
        o4, _ = fa.fwd_fp8(q, k, v, causal=causal, with_lse=False)
        torch.cuda.synchronize()
        assert none is None and torch.equal(o1, o2) and torch.equal(o3, o4)


def test_decode_without_lse_and_shared_workspace():
    B, H, d = 3, 4, 128
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, 4000, d, 0), dtype=torch.uint8, device=device())
    for Nkv in (4000, 1000, 37):
        q, k, v = _qkv(12 + Nkv, B, H, 1, Nkv, d)
        q = q[:, :, 0].contiguous()
        say(f"fa_decode lse=NULL, workspace sized for 4000 keys, Nkv={Nkv}")
        o_ref, _ = fa.decode(q, k, v)
        o = torch.empty_like(q)
        need = fa.fa_decode_workspace_size(B, H, Nkv, d, 0)
        assert need <= ws.numel()
        fa.fa_decode(q, k, v, o, None, B, H, Nkv, d, 1 / np.sqrt(d), fa.FA_F16, 0, ws, ws.numel(),
                     torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)


def test_paged_decode_without_lse():
    B, H, d, N = 3, 2, 64, 500
    plan = fi.paged_plan(13, B, N, 16, ragged=True)
    rng = np.random.default_rng(13)
    q = upload(rand_bits(rng, (B, H, d), "f16"), "f16")
    kp = upload(fi.scatter_to_pages(rand_bits(rng, (B, H, N, d), "f16"), plan), "f16")
    vp = upload(fi.scatter_to_pages(rand_bits(rng, (B, H, N, d), "f16"), plan), "f16")
    table = torch.from_numpy(plan.block_table).to(device())
    lens = torch.from_numpy(plan.seq_lens).to(device())
    say("fa_decode_paged lse=NULL")
    o_ref, _ = fa.decode_paged(q, kp, vp, table, lens, max_seq_len=N)
    o = torch.empty_like(q)
    nbytes = fa.fa_decode_workspace_size(B, H, N, d, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device())
    fa.fa_decode_paged(q, kp, vp, table, lens, o, None, B, H, d, plan.num_pages, 16, plan.block_table.shape[1],
                       fa.FA_PAGED_HND, N, 1 / np.sqrt(d), fa.FA_F16, 0, ws, nbytes,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_caller_stream():
    # every entry point runs on the stream it is given (a second stream of
    # default priority), ordered after work queued there before it
    q, k, v = _qkv(14, 1, 4, 256, 256, 128)
    ref_o, ref_lse = fa.fwd(q, k, v, causal=True)
    ref_g = fa.bwd(q, k, v, ref_o, q, ref_lse, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("entry points on a caller stream")
    with torch.cuda.stream(s):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()  # queued on s before the library calls
        o, lse = fa.fwd(q2, k2, v2, causal=True)
        g = fa.bwd(q2, k2, v2, o, q2, lse, causal=True)
        od, _ = fa.decode(q2[:, :, :1].contiguous(), k2, v2)
    s.synchronize()
    od_ref, _ = fa.decode(q[:, :, :1].contiguous(), k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    assert all(torch.equal(a, b) for a, b in zip(g, ref_g))
    assert torch.equal(od, od_ref)


def test_binding_rejects_misplaced_tensors():
    # the binding refuses, before any launch, tensors the kernels could not
    # address: a host LSE for the backward, tensors of the wrong rank
    q, k, v = _qkv(15, 1, 2, 128, 128, 64)
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    say("binding argument checks (no launch)")
    with pytest.raises(ValueError, match="lse"):
        fa.bwd(q, k, v, o, q, lse.cpu(), causal=True)
    with pytest.raises(ValueError, match="dimensions"):
        fa.fwd(q[0], k[0], v[0])
    with pytest.raises(ValueError, match="dimensions"):
        fa.decode(q[:, :, 0].contiguous(), k[0], v[0])
    # a torch stream object is accepted where the C call takes a stream
    s = torch.cuda.Stream()
    o2 = torch.empty_like(o)
    fa.fa_fwd(q, k, v, o2, None, 1, 2, 128, 128, 64, 1, 1 / np.sqrt(64), fa.FA_F16, s)
    s.synchronize()
    assert torch.equal(o2, o)


def test_graph_capture_replays():
    # the entry points enqueue kernels only (no allocation, no memset, no
    # synchronisation), so a caller can capture them into a HIP graph; every
    # replay, with eager work of the program between replays, gives the bits
    # of the eager calls
    B, H, N, d = 1, 4, 300, 64
    q, k, v = _qkv(16, B, H, N, N, d)
    dev = q.device
    code = fa.FA_F16
    scale = 1 / np.sqrt(d)
    o, lse = torch.empty_like(q), torch.empty(B, H, N, dtype=torch.float32, device=dev)
    qd = q[:, :, -1].contiguous()
    od, lsed = torch.empty_like(qd), torch.empty(B, H, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, N, d, 0), dtype=torch.uint8, device=dev)
    g3 = [torch.empty_like(q) for _ in range(3)]
    bws = torch.empty(fa.fa_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)

    def calls(s):
        fa.fa_fwd(q, k, v, o, lse, B, H, N, N, d, 1, scale, code, s)
        fa.fa_decode(qd, k, v, od, lsed, B, H, N, d, scale, code, 0, ws, ws.numel(), s)
        fa.fa_bwd(q, k, v, o, q, lse, g3[0], g3[1], g3[2], B, H, N, N, d, 1, scale, code, bws, bws.numel(), s)

    outs = (o, lse, od, lsed, *g3)
    say("eager calls, then capture into a graph")
    calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        other, _ = fa.fwd(q, k, v, causal=False)  # eager work between replays
        torch.cuda.synchronize()
        say(f"graph replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), f"replay {r}"
        assert not torch.isnan(other).any()


def test_empty_inputs():
    # zero-size tensors (whose data pointers are NULL) through every entry point
    dev = device()
    q0 = torch.zeros(1, 2, 0, 64, dtype=torch.float16, device=dev)
    k, v = (torch.randn(1, 2, 300, 64, device=dev).half() for _ in range(2))
    say("empty inputs: fwd, fwd_fp8, decode, quantize")
    o, lse = fa.fwd(q0, k, v, causal=True)
    o8, lse8 = fa.fwd_fp8(q0, k, v)
    assert o.shape == q0.shape and lse.shape == (1, 2, 0) and o8.shape == q0.shape
    e = torch.zeros(0, 2, 9, 64, dtype=torch.bfloat16, device=dev)
    assert fa.fwd(e, e, e)[0].shape == e.shape
    od, ld = fa.decode(torch.zeros(0, 2, 64, dtype=torch.float16, device=dev), e.half(), e.half())
    assert od.shape == (0, 2, 64) and ld.shape == (0, 2)
    assert fa.quantize_e4m3(q0).shape == q0.shape
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,causal,out_f32", [(64, False, False), (128, True, True)])
def test_bwd_without_query_rows(d, causal, out_f32):
    # no query reaches any key: dK = dV = 0 is written, and the query-side
    # pointers (here NULL) are never touched
    dev = device()
    k, v = (torch.randn(2, 3, 300, d, device=dev).half() for _ in range(2))
    gdt = torch.float32 if out_f32 else torch.float16
    dk = torch.full(k.shape, float("nan"), dtype=gdt, device=dev)
    dv = torch.full(v.shape, float("nan"), dtype=gdt, device=dev)
    code = fa.FA_F16 | (fa.FA_OUT_F32 if out_f32 else 0)
    say(f"fa_bwd Nq=0 d={d} causal={causal} out_f32={out_f32}")
    fa.fa_bwd(None, k, v, None, None, None, None, dk, dv, 2, 3, 0, 300, d, causal, 0.1, code, None, 0,
              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()
    q0 = torch.zeros(2, 3, 0, d, dtype=torch.float16, device=dev)
    lse0 = torch.zeros(2, 3, 0, dtype=torch.float32, device=dev)
    dq, dk2, dv2 = fa.bwd(q0, k, v, q0, q0, lse0, causal=causal, out_dtype=gdt)
    torch.cuda.synchronize()
    assert dq.shape == q0.shape and (dk2 == 0).all() and (dv2 == 0).all()


def test_concurrent_callers():
    # the library keeps no shared mutable state (the last-error text is per
    # thread): four host threads, each on its own stream, calling the forward,
    # decode and backward at once give the bits of the same calls made one by one
    import threading
    cases = []
    for i in range(4):
        q, k, v = _qkv(100 + i, 1, 4, 200 + 37 * i, 300 + 41 * i, 64 if i % 2 else 128)
        cases.append((q, k, v))

    def run(case):
        q, k, v = case
        o, lse = fa.fwd(q, k, v, causal=True)
        od, ld = fa.decode(q[:, :, -1].contiguous(), k, v)
        g = fa.bwd(q, k, v, o, q, lse, causal=True)
        return (o, lse, od, ld) + tuple(g)

    say("four threads on four streams")
    ref = [run(c) for c in cases]
    torch.cuda.synchronize()
    out = [None] * len(cases)
    streams = [torch.cuda.Stream() for _ in cases]
    start = threading.Barrier(len(cases))

    def worker(i):
        with torch.cuda.stream(streams[i]):
            start.wait()
            for _ in range(3):
                out[i] = run(cases[i])
        streams[i].synchronize()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for r, o in zip(ref, out):
        assert all(torch.equal(a, b) for a, b in zip(r, o))
