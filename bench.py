#!/usr/bin/env python3
"""Benchmark of libfa355 on one MI355X.

One step is one pass of the whole hot path on synthetic inputs already
resident in HBM:
  1. fa_fwd   on the long-context prefill: B=1, H=32, Nq=Nkv=8192, d=128,
              fp16, causal, scale 1/sqrt(128), Q and K ~ 1.5 N(0,1), V ~ N(0,1);
  2. fa_decode on the decode workload: B=16, H=32, one query against
              Nkv=32768 cached keys, d=128, fp16, split-KV.
Each call is bracketed by HIP events on the stream it is launched on.  The
headline value is prefill TFLOP/s (4*B*H*N^2*d FLOPs halved for causal, over
the mean kernel time); decode is reported in HBM GB/s over its algorithmic
bytes (K and V once, q, o and lse).  rank 0 prints one JSON line.

Separately from the step, the backward (fa_bwd: dQ, dK, dV from O and LSE,
with dO from the seeded generator) is timed on the prefill workload and
reported in its own "backward" object, the other two prefill workloads
(2K d64 fp16 and 16K d128 bf16 causal) in "other_prefill" (also timed as one HIP graph of
back-to-back calls, since a 2K call is shorter than the host's time to issue it), the FP8 variant (fa_fwd_fp8: Q and K
rounded to E4M3 for the first product) on the prefill workload in an
"fp8_forward" object, and decode over a paged cache (fa_decode_paged: the
decode cache scattered into a shuffled pool of 16-key pages) in a
"paged_decode" object; none of them is part of `value`.  A plain
streaming-read kernel (libfa355_probe) timed over the decode K cache gives
the measured HBM read rate decode is also compared against ("read_probe").

The CPU baseline is the fp64 oracle (plain standard attention that
materialises the score matrix) timed on a sample of the prefill heads on the
host's cores; it is a reference point, not the target.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bwd] [--no-other] [--no-fp8] [--no-paged]
    python bench.py --sweep [--steps K] [--warmup W]   # fused vs unfused over sequence length
    python bench.py --map [--steps K] [--warmup W]     # fused kernels over N, d, mask, type
    python bench.py --data-probe [--steps K] [--warmup W]  # fa_fwd on workload, zero and constant inputs
    python bench.py --lds-probe                        # LDS access patterns, one launch each (for rocprofv3)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s & % MFMA peak, N=8192 d=128 causal; decode HBM GB/s"
PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak (published)
PEAK_MFMA_F8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak (published)
PREFILL = "prefill_8k_d128"
DECODE = "decode_32k_d128"
PAGED = "decode_32k_d128_paged16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = {
    "prefill": ["exact_io_aware_65_amd/csrc/fa_fwd.hip", "exact_io_aware_65_amd/csrc/fa_device.hpp"],
    "decode": ["exact_io_aware_65_amd/csrc/fa_decode.hip", "exact_io_aware_65_amd/csrc/fa_device.hpp"],
    "backward": ["exact_io_aware_65_amd/csrc/fa_bwd.hip", "exact_io_aware_65_amd/csrc/fa_device.hpp"],
}


# ---------------------------------------------------------------------------
# FLOP and byte models

def metric_flops(B, H, Nq, Nkv, d, causal):
    """The method's contraction FLOPs, 2 * (QK^T + PV); halved for a causal mask."""
    f = 4 * B * H * Nq * Nkv * d
    return f // 2 if causal else f


def algorithmic_bytes(B, H, Nq, Nkv, d, elt=2, out_elt=2, lse=True):
    """Compulsory HBM traffic: read q, k, v once; write o (and lse) once."""
    return elt * B * H * (Nq + 2 * Nkv) * d + out_elt * B * H * Nq * d + (4 * B * H * Nq if lse else 0)


def score_matrix_bytes(n, elt=2):
    """Bytes of one head's n x n score matrix: what the fused kernel never writes."""
    return n * n * elt


def _code_only(text: str) -> str:
    """Source text without comments and with runs of blank space folded, so that
    editing a comment does not count as changing the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, key=None):
    """HBM bytes per launch from rocprofv3 counters, if they were taken on the current kernel sources.

    kernel names the source group whose digest must match ("prefill" or
    "decode"); key the record entry (default: that group's own launch)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.loads(f.read().split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get(f"{kernel}_digest") != kernel_source_digest(kernel):
        return None
    return rec.get(f"{key or kernel}_bytes")


def calibrate_copy():
    """A plain device copy of 1 GiB, three times: the reference FETCH_SIZE / WRITE_SIZE are read on it."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copied_bytes": n, "times": 3}))


# ---------------------------------------------------------------------------

ORACLE_BUDGET_S = 30.0   # CPU seconds of oracle work per leg (whole heads, at least one)
TOL_O = {"f16": 2e-3, "bf16": 1.5e-2}  # max |O - O_oracle|, per input type
TOL_LSE = 1e-3                         # max |LSE - LSE_oracle|
TOL_GRAD_REL = {"f16": 10 * 2.0 ** -11, "bf16": 10 * 2.0 ** -8}  # backward: of max |grad_oracle|


def host_info():
    """The host CPU the oracle runs on: model name and logical cores."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cores": os.cpu_count()}


class Worst:
    """Largest |got - ref| over the elements added so far, with its index; any NaN fails."""

    def __init__(self):
        self.err, self.at, self.nan, self.n, self.abs_sum, self.ref_max = 0.0, None, False, 0, 0.0, 0.0

    def add(self, got, ref, prefix=()):
        import numpy as np
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if got.size == 0:
            return
        self.nan |= bool(np.isnan(got).any())
        diff = np.abs(got - ref)
        k = int(np.nanargmax(diff)) if not np.isnan(diff).all() else 0
        if diff.flat[k] > self.err or self.at is None:
            self.err, self.at = float(diff.flat[k]), [*prefix, *(int(i) for i in np.unravel_index(k, diff.shape))]
        self.n += got.size
        self.abs_sum += float(np.nansum(diff))
        self.ref_max = max(self.ref_max, float(np.max(np.abs(ref))))

    def record(self, name, tol=None, rel=None):
        out = {f"err_{name}": self.err, f"worst_{name}": self.at, f"mean_abs_err_{name}": self.abs_sum / max(self.n, 1)}
        if rel is not None:
            out[f"err_{name}_rel"] = self.err / self.ref_max if self.ref_max else 0.0
        ok = not self.nan and (tol is None or self.err <= tol) and (rel is None or self.err <= rel * self.ref_max)
        return out, ok


def oracle_forward_leg(w, head_inputs, o_dev, lse_dev, budget_s=ORACLE_BUDGET_S, fp8=False, keep_ref=False):
    """The oracle beside one forward leg.

    Whole heads of workload w, one at a time (head_inputs(b, h) -> the head's
    q, k, v bits), until budget_s of oracle time has passed: the time gives
    the leg's cpu_baseline, and the results are compared with every element
    of the same heads of the outputs the timed calls produced (o_dev, lse_dev,
    as timed: O in the input type).  keep_ref also returns the oracle's O
    rounded to the input type and its LSE for every head it ran."""
    import numpy as np

    import fa_inputs as fi
    import oracle
    o_all = o_dev.float().cpu().numpy()
    lse_all = lse_dev.float().cpu().numpy().reshape(o_all.shape[:3])
    wo, wl = Worst(), Worst()
    spent, heads, kept = 0.0, 0, {}
    for bh in range(w.heads):
        b, h = divmod(bh, w.H)
        q, k, v = head_inputs(b, h)
        t0 = time.perf_counter()
        if fp8:
            o_ref, lse_ref = oracle.attention_fp8qk(q, k, v, causal=w.causal, scale=w.scale, dtype=w.dtype)
        else:
            o_ref, lse_ref = oracle.attention(q, k, v, causal=w.causal, scale=w.scale, dtype=w.dtype)
        spent += time.perf_counter() - t0
        heads += 1
        wo.add(o_all[b, h], o_ref, (b, h))
        wl.add(lse_all[b, h], lse_ref, (b, h))
        if keep_ref:
            kept[(b, h)] = (fi.f32_to_bits(o_ref.astype(np.float32), w.dtype), lse_ref.astype(np.float32))
        if spent >= budget_s:
            break
    flops = metric_flops(1, heads, w.Nq, w.Nkv, w.d, w.causal)
    ro, ok_o = wo.record("O", TOL_O[w.dtype])
    rl, ok_l = wl.record("LSE", TOL_LSE)
    cpu = {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
           "seconds": round(spent, 2),
           "sample": f"{heads} of {w.heads} heads of {w.name} ({'E4M3 Q and K, ' if fp8 else ''}fp64, score "
                     f"matrix materialised), {spent:.1f} s"}
    parity = {**ro, **rl, "tol_O": TOL_O[w.dtype], "tol_LSE": TOL_LSE, "pass": ok_o and ok_l,
              "compared": f"every element of O ({w.dtype}, as timed) and LSE of {heads} of {w.heads} heads",
              "index": "worst_O = [b, h, row, dim], worst_LSE = [b, h, row]"}
    return (cpu, parity, kept) if keep_ref else (cpu, parity)


def oracle_decode_leg(w, head_inputs, o_dev, lse_dev, budget_s=ORACLE_BUDGET_S):
    """The oracle beside decode: heads of workload w, one at a time
    (head_inputs(b, h) -> the head's q [1, d], k, v bits), until budget_s of
    oracle time has passed; compared with the timed calls' O (input type) and
    LSE."""
    import oracle
    o_all = o_dev.float().cpu().numpy().reshape(w.B, w.H, w.d)
    lse_all = lse_dev.float().cpu().numpy().reshape(w.B, w.H)
    wo, wl = Worst(), Worst()
    spent, heads = 0.0, 0
    for bh in range(w.heads):
        b, h = divmod(bh, w.H)
        q, k, v = head_inputs(b, h)
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(q, k, v, causal=False, scale=w.scale, dtype=w.dtype)
        spent += time.perf_counter() - t0
        heads += 1
        wo.add(o_all[b, h], o_ref[0], (b, h))
        wl.add(lse_all[b, h], lse_ref[0], (b, h))
        if spent >= budget_s:
            break
    nbytes = algorithmic_bytes(1, heads, 1, w.Nkv, w.d)
    ro, ok_o = wo.record("O", TOL_O[w.dtype])
    rl, ok_l = wl.record("LSE", TOL_LSE)
    cpu = {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": oracle.threads(), "kind": "oracle",
           "seconds": round(spent, 2),
           "sample": f"{heads} of {w.heads} heads of {w.name} (fp64), {spent:.1f} s; rate over the same "
                     f"algorithmic bytes as the GPU figure"}
    parity = {**ro, **rl, "tol_O": TOL_O[w.dtype], "tol_LSE": TOL_LSE, "pass": ok_o and ok_l,
              "compared": f"O ({w.dtype}, as timed) and LSE of {heads} of {w.heads} heads",
              "index": "worst_O = [b, h, dim], worst_LSE = [b, h]"}
    return cpu, parity


def backward_flops(B, H, Nq, Nkv, d, causal):
    """The usual count for the attention backward: five products (2.5 x the forward)."""
    return metric_flops(B, H, Nq, Nkv, d, causal) * 5 // 2


def backward_bytes(B, H, Nq, Nkv, d, elt=2):
    """Compulsory HBM traffic of the backward: read q, k, v, o, dO and LSE once; write dQ, dK, dV once."""
    return B * H * (elt * (3 * Nq + 2 * Nkv) * d + 4 * Nq + elt * (Nq + 2 * Nkv) * d)


def time_backward(fa, fi, w, q, k, v, stream, warmup, steps, fwd_ref=None, oracle_budget=None):
    """fa_bwd on workload w (dO from the seeded generator), each call bracketed by HIP events.

    fa_bwd is handed O (input type) and LSE: the oracle's for the heads in
    fwd_ref ({(b, h): (O bits, LSE fp32)}), the GPU forward's for the rest.
    With oracle_budget, the oracle's gradients (D from the same O) of the
    fwd_ref heads, in order, until that many seconds have passed, are compared
    with every element of those heads of the timed calls' dQ, dK, dV, and
    the oracle's time is this leg's cpu_baseline."""
    import statistics

    import torch
    dout_bits = fi.make_tensor(w, fi.DOUT)
    dout = fi.bits_to_torch(dout_bits, w.dtype).to(q.device)
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    for (b, h), (o16, l32) in (fwd_ref or {}).items():
        o[b, h] = fi.bits_to_torch(o16, w.dtype).to(q.device)
        lse[b, h] = torch.from_numpy(l32).to(q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa.fa_bwd_workspace_size(w.B, w.H, w.Nq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    sp = stream.cuda_stream

    def call():
        fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal, w.scale, fa.FA_F16
                  if w.dtype == "f16" else fa.FA_BF16, ws, nbytes, sp)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    mean = statistics.fmean(ms)
    flops = backward_flops(w.B, w.H, w.Nq, w.Nkv, w.d, w.causal)
    res = {
        "workload": w.name,
        "ms_mean": round(mean, 4),
        "ms_min": round(min(ms), 4),
        "flops": flops,
        "TFLOP/s": round(flops / (mean * 1e-3) / 1e12, 2),
        "frac_of_mfma_peak": round(flops / (mean * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
        "algorithmic_bytes": backward_bytes(w.B, w.H, w.Nq, w.Nkv, w.d),
        "workspace_bytes": nbytes,
        "traffic": measured_traffic("backward"),
        "note": "FLOPs counted as 2.5 x the forward (five products); the kernels do seven "
                "(S and dP are formed in both the key-block and the query-block pass)",
    }
    if oracle_budget and fwd_ref:
        import oracle
        got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
        worst = {n: Worst() for n in ("dQ", "dK", "dV")}
        spent, heads = 0.0, 0
        x = {t: fi.make_tensor(w, i) for t, i in (("q", fi.Q), ("k", fi.K), ("v", fi.V))}
        for (b, h), (o16, _) in sorted(fwd_ref.items()):
            t0 = time.perf_counter()
            ref = oracle.attention_bwd(x["q"][b, h], x["k"][b, h], x["v"][b, h], dout_bits[b, h], causal=w.causal,
                                       scale=w.scale, dtype=w.dtype, o_for_d=o16)
            spent += time.perf_counter() - t0
            heads += 1
            for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
                worst[n].add(g[b, h], r, (b, h))
            if spent >= oracle_budget:
                break
        parity, ok = {}, True
        for n, wst in worst.items():
            rec, good = wst.record(n, rel=TOL_GRAD_REL[w.dtype])
            parity.update(rec)
            ok &= good
        parity.update({"tol_rel": TOL_GRAD_REL[w.dtype], "pass": ok,
                       "compared": f"every element of dQ, dK, dV ({w.dtype}, as timed) of {heads} of {w.heads} "
                                   "heads; fa_bwd handed the oracle's O (rounded to the input type) and LSE for "
                                   "them, and the oracle forms D from the same O",
                       "index": "worst_* = [b, h, row, dim]"})
        res["parity"] = parity
        res["cpu_baseline"] = {"value": flops / w.heads * heads / spent / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.threads(), "kind": "oracle", "seconds": round(spent, 2),
                               "sample": f"{heads} of {w.heads} heads of {w.name}, the backward (fp64, P and dS "
                                         f"materialised), {spent:.1f} s"}
    return res


def time_fp8_forward(fa, fi, w, q, k, v, stream, warmup, steps, head_inputs=None, oracle_budget=ORACLE_BUDGET_S):
    """fa_fwd_fp8 on workload w: K rounded to E4M3 once (timed on its own), then
    the forward with Q rounded in the kernel, each call bracketed by HIP events.
    With head_inputs (b, h -> the head's 16-bit q, k, v bits) the oracle of
    the FP8 variant (its own E4M3 codec on q and k) runs beside it."""
    import statistics

    import torch
    sp = stream.cuda_stream
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=k.device)
    code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=q.device)

    def quant():
        fa.fa_quantize_e4m3(k, k8, k.numel(), code, sp)

    def call():
        fa.fa_fwd_fp8(q, k8, v, o, lse, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal, w.scale, code, sp)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    qms = timed(quant)
    ms = timed(call)
    mean = statistics.fmean(ms)
    oracle_leg = None
    if head_inputs is not None:
        oracle_leg = oracle_forward_leg(w, head_inputs, o, lse, budget_s=oracle_budget, fp8=True)
    flops = metric_flops(w.B, w.H, w.Nq, w.Nkv, w.d, w.causal)
    tflops = flops / (mean * 1e-3) / 1e12
    # half the FLOPs (Q K^T) at the E4M3 rate, half (P V) at the 16-bit rate
    mixed_peak = 1.0 / (0.5 / PEAK_MFMA_F8_TFLOPS + 0.5 / PEAK_MFMA_F16_TFLOPS)
    return {
        "workload": w.name,
        "ms_mean": round(mean, 4),
        "ms_min": round(min(ms), 4),
        "flops": flops,
        "TFLOP/s": round(tflops, 2),
        "frac_of_mixed_peak": round(tflops / mixed_peak, 4),
        "mixed_peak_TFLOP/s": round(mixed_peak, 1),
        "quantize_k_ms": round(statistics.fmean(qms), 4),
        "traffic": measured_traffic("prefill", "fp8"),
        "note": "Q K^T on the E4M3 MFMA (5.0 PFLOP/s peak), P V in 16 bits (2.5 PFLOP/s); K rounded to E4M3 once "
                "before the timed calls (quantize_k_ms), Q inside the kernel",
        **({"cpu_baseline": oracle_leg[0], "parity": oracle_leg[1]} if oracle_leg else {}),
    }


# ---------------------------------------------------------------------------
# the unfused baseline and the speed-vs-length sweep

def unfused_attention(q, k, v, causal, scale, mask=None):
    """Standard attention with every intermediate in device memory ("FlashAttention",
    section "The problem: the n x n score matrix"): S = (scale q) k^T in q's type,
    masked, P = softmax(S) in q's type, O = P v -- three kernels and two n x n
    tensors per head, the shape of PyTorch's math path.  A comparison point
    only, built from torch's library GEMMs and softmax; mask, if given, is the
    [Nq, Nkv] boolean of hidden keys."""
    import torch
    s = torch.matmul(q * scale, k.transpose(-1, -2).contiguous())
    if causal:
        if mask is None:
            mask = causal_mask(q.shape[-2], k.shape[-2], q.device)
        s.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v)


def causal_mask(n_q, n_k, device):
    """Keys hidden from each query row: j > i + (n_k - n_q)."""
    import torch
    return torch.ones(n_q, n_k, dtype=torch.bool, device=device).triu_(n_k - n_q + 1)


def unfused_decode(q, k, v, scale):
    """One query per head against the cache, unfused: s = K (scale q) in q's type
    ([B, H, N, 1] in memory), p = softmax(s), o = p^T V."""
    import torch
    s = torch.matmul(k, (q * scale).unsqueeze(-1))
    p = torch.softmax(s, dim=-2)
    return torch.matmul(p.transpose(-1, -2).contiguous(), v).squeeze(-2)


def measure_read_bandwidth(buf, stream, warmup, steps):
    """HBM read rate of a plain streaming-read kernel over the device tensor buf.

    The probe (libfa355_probe.so, built beside the library) reads every byte
    once with 16-byte non-temporal loads, one contiguous chunk per workgroup:
    the same access pattern as the decode kernels, without their arithmetic.
    Decode is reported against it as well as against the published peak."""
    import ctypes

    import torch
    from exact_io_aware_65_amd import build as libbuild
    if not os.path.exists(libbuild.PROBE_LIBRARY):
        raise RuntimeError(f"{libbuild.PROBE_LIBRARY} is missing: run python -m exact_io_aware_65_amd.build")
    lib = ctypes.CDLL(libbuild.PROBE_LIBRARY)
    lib.fa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_read.restype = ctypes.c_int
    sink = torch.empty(lib.fa_probe_read_blocks() * 256, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()

    def call():
        rc = lib.fa_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
        if rc:
            raise RuntimeError(f"fa_probe_read failed ({rc})")

    mean = _event_ms(call, stream, warmup, steps)
    return {"bytes": nbytes, "ms_mean": round(mean, 4), "GB/s": round(nbytes / (mean * 1e-3) / 1e9, 1),
            "kernel": "read_chunks (16-byte non-temporal loads, one chunk per workgroup)"}


def device_name(props):
    """The product name the driver reports in sysfs, else torch's device name."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/product_name")):
        try:
            with open(path) as f:
                name = f.read().strip()
            if name:
                return name
        except OSError:
            pass
    return props.name or getattr(props, "gcnArchName", "")


def build_info():
    """What build.py recorded beside the libraries (git commit of the sources)."""
    from exact_io_aware_65_amd import build as libbuild
    try:
        with open(libbuild.BUILD_INFO) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def _event_ms(fn, stream, warmup, steps):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return statistics.fmean(a.elapsed_time(b) for a, b in evs)


def _graph_ms(launch, warmup, steps):
    """Mean time per call when `steps` calls, captured once into a HIP graph,
    replay back to back: the kernels' own rate, without the host's launch gap
    between calls (which per-call events include once a call is shorter than
    the host's time to issue it).  launch(stream_handle) enqueues one call."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            launch(cs)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


SWEEP_PREFILL = (512, 1024, 2048, 4096, 8192, 16384, 32768)
SWEEP_DECODE = (1024, 4096, 16384, 32768)


def run_sweep(warmup, steps):
    """fa_fwd against the unfused baseline over sequence lengths (B=1, H=32, d=128,
    causal, fp16 -- the pages' benchmark shape), and fa_decode against unfused
    decode over cache lengths (B=16, H=32, d=128).  Each length also reports the
    largest |O_fused - O_unfused| and the device memory each path needs beyond
    its inputs and outputs."""
    import torch

    import exact_io_aware_65_amd as fa
    import fa_inputs as fi
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    out = {"prefill": [], "decode": []}
    base = fi.WORKLOADS[PREFILL]
    for n in SWEEP_PREFILL:
        w = base.with_(name=f"sweep_prefill_{n}", Nq=n, Nkv=n)
        x = fi.make_inputs(w)
        q, k, v = (fi.bits_to_torch(x[t], w.dtype).to(dev) for t in "qkv")
        x = None
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, n), dtype=torch.float32, device=dev)
        mask = causal_mask(n, n, dev)
        torch.cuda.synchronize()
        fused = _event_ms(lambda: fa.fa_fwd(q, k, v, o, lse, w.B, w.H, n, n, w.d, True, w.scale, fa.FA_F16, sp),
                          stream, warmup, steps)
        base_mem = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        ou = unfused_attention(q, k, v, True, w.scale, mask)
        torch.cuda.synchronize()
        extra = torch.cuda.max_memory_allocated(dev) - base_mem - ou.numel() * ou.element_size()
        diff = float((ou.float() - o.float()).abs().max())
        ou = None
        unf = _event_ms(lambda: unfused_attention(q, k, v, True, w.scale, mask), stream, warmup, steps)
        flops = metric_flops(w.B, w.H, n, n, w.d, True)
        out["prefill"].append({
            "N": n, "fused_ms": round(fused, 4), "unfused_ms": round(unf, 4), "speedup": round(unf / fused, 2),
            "fused_TFLOP/s": round(flops / (fused * 1e-3) / 1e12, 1),
            "unfused_TFLOP/s": round(flops / (unf * 1e-3) / 1e12, 1),
            "unfused_extra_bytes": int(extra), "fused_extra_bytes": 0, "max_abs_diff_O": diff})
        print(f"[sweep] prefill N={n}: fused {fused:.3f} ms, unfused {unf:.3f} ms, x{unf / fused:.2f}",
              file=sys.stderr, flush=True)
        q = k = v = o = lse = mask = None
        torch.cuda.empty_cache()
    dbase = fi.WORKLOADS[DECODE]
    for n in SWEEP_DECODE:
        w = dbase.with_(name=f"sweep_decode_{n}", Nkv=n)
        x = fi.make_inputs(w)
        q = fi.bits_to_torch(x["q"][:, :, 0], w.dtype).to(dev)
        k, v = (fi.bits_to_torch(x[t], w.dtype).to(dev) for t in "kv")
        x = None
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        nbytes = fa.fa_decode_workspace_size(w.B, w.H, n, w.d, 0)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        fused = _event_ms(lambda: fa.fa_decode(q, k, v, o, lse, w.B, w.H, n, w.d, w.scale, fa.FA_F16, 0, ws, nbytes, sp),
                          stream, warmup, steps)
        ou = unfused_decode(q, k, v, w.scale)
        torch.cuda.synchronize()
        diff = float((ou.float() - o.float()).abs().max())
        unf = _event_ms(lambda: unfused_decode(q, k, v, w.scale), stream, warmup, steps)
        nb = algorithmic_bytes(w.B, w.H, 1, n, w.d)
        out["decode"].append({
            "Nkv": n, "fused_ms": round(fused, 4), "unfused_ms": round(unf, 4), "speedup": round(unf / fused, 2),
            "fused_GB/s": round(nb / (fused * 1e-3) / 1e9, 1), "unfused_GB/s": round(nb / (unf * 1e-3) / 1e9, 1),
            "fused_workspace_bytes": nbytes, "max_abs_diff_O": diff})
        print(f"[sweep] decode Nkv={n}: fused {fused:.3f} ms, unfused {unf:.3f} ms, x{unf / fused:.2f}",
              file=sys.stderr, flush=True)
        q = k = v = o = lse = ws = None
        torch.cuda.empty_cache()
    return out


MAP_TOKENS = 1 << 18                     # B*H*N of every forward point (heads scale with 1/N)
MAP_PREFILL = (1024, 2048, 4096, 8192, 16384, 32768)
MAP_DECODE = ((16, 32, 4096), (16, 32, 16384), (16, 32, 65536), (16, 32, 131072),  # (B, H, cache length)
              (4, 8, 131072), (1, 8, 32768), (1, 1, 1 << 20))


def run_map(warmup, steps):
    """Fused kernels only, over shapes: fa_fwd, fa_fwd_fp8 and fa_bwd for N in
    MAP_PREFILL, d in {64, 128}, causal or not, fp16 and bf16, with B = 1 and
    H = MAP_TOKENS / N; fa_decode for the (B, H, cache length) points of
    MAP_DECODE, d in {64, 128}, fp16.  Inputs are drawn on the device (timing
    only)."""
    import torch

    import exact_io_aware_65_amd as fa
    import fa_inputs as fi
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    out = {"prefill": [], "decode": []}
    for n in MAP_PREFILL:
        H = MAP_TOKENS // n
        for d in (64, 128):
            for dtype in ("f16", "bf16"):
                q, k, v, do = (fi.device_normals((1, H, n, d), dtype, 100 + t, dev) for t in range(4))
                k8 = fa.quantize_e4m3(k)
                o = torch.empty_like(q)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                bws = torch.empty(max(fa.fa_bwd_workspace_size(1, H, n), 16), dtype=torch.uint8, device=dev)
                lse = torch.empty((1, H, n), dtype=torch.float32, device=dev)
                code = fa.FA_F16 if dtype == "f16" else fa.FA_BF16
                scale = 1.0 / math.sqrt(d)
                for causal in (True, False):
                    t16 = _event_ms(lambda: fa.fa_fwd(q, k, v, o, lse, 1, H, n, n, d, causal, scale, code, sp),
                                    stream, warmup, steps)
                    t8 = _event_ms(lambda: fa.fa_fwd_fp8(q, k8, v, o, lse, 1, H, n, n, d, causal, scale, code, sp),
                                   stream, warmup, steps)
                    fa.fa_fwd(q, k, v, o, lse, 1, H, n, n, d, causal, scale, code, sp)  # O and LSE of this mask
                    tb = _event_ms(lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, 1, H, n, n, d, causal, scale,
                                                     code, bws, bws.numel(), sp), stream, warmup, steps)
                    flops = metric_flops(1, H, n, n, d, causal)
                    bflops = backward_flops(1, H, n, n, d, causal)
                    out["prefill"].append({"N": n, "H": H, "d": d, "dtype": dtype, "causal": causal,
                                           "ms": round(t16, 4), "TFLOP/s": round(flops / (t16 * 1e-3) / 1e12, 1),
                                           "fp8_ms": round(t8, 4),
                                           "fp8_TFLOP/s": round(flops / (t8 * 1e-3) / 1e12, 1),
                                           "bwd_ms": round(tb, 4),
                                           "bwd_TFLOP/s": round(bflops / (tb * 1e-3) / 1e12, 1)})
                    print(f"[map] fwd N={n} H={H} d={d} {dtype} {'causal' if causal else 'full'}: "
                          f"{flops / (t16 * 1e-3) / 1e12:.0f} / fp8 {flops / (t8 * 1e-3) / 1e12:.0f} / "
                          f"bwd {bflops / (tb * 1e-3) / 1e12:.0f} TFLOP/s", file=sys.stderr, flush=True)
                q = k = v = do = k8 = o = lse = dq = dk = dv = bws = None
                torch.cuda.empty_cache()
    for B, H, n in MAP_DECODE:
        for d in (64, 128):
            q = fi.device_normals((B, H, d), "f16", 200, dev)
            k, v = (fi.device_normals((B, H, n, d), "f16", 201 + t, dev) for t in range(2))
            o = torch.empty_like(q)
            lse = torch.empty((B, H), dtype=torch.float32, device=dev)
            nbytes = fa.fa_decode_workspace_size(B, H, n, d, 0)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            scale = 1.0 / math.sqrt(d)
            t = _event_ms(lambda: fa.fa_decode(q, k, v, o, lse, B, H, n, d, scale, fa.FA_F16, 0, ws, nbytes, sp),
                          stream, warmup, steps)
            nb = algorithmic_bytes(B, H, 1, n, d)
            out["decode"].append({"Nkv": n, "B": B, "H": H, "d": d, "splits": fa.fa_decode_num_splits(B, H, n, d),
                                  "ms": round(t, 4), "GB/s": round(nb / (t * 1e-3) / 1e9, 1)})
            print(f"[map] decode B={B} H={H} Nkv={n} d={d}: {nb / (t * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr,
                  flush=True)
            q = k = v = o = lse = ws = None
            torch.cuda.empty_cache()
    return out


DATA_PROBE = ("prefill_8k_d128", "prefill_16k_d128_bf16")


LDS_SKIP = 0xFFFFFFFF


def _swap23(x):
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1)


def lds_probe_patterns():
    """LDS access patterns for the bank probe (libfa355_probe fa_probe_lds):
    (name, kind, 64 lane byte offsets), kind 0 = ds_read_b128, 1 =
    ds_read_b64_tr_b16; LDS_SKIP marks a lane that does not read.

    First, pairs: lane 0 at byte 0 and lane b at byte 256 (the same banks, a
    different address), the other lanes idle; a conflict means the hardware
    serves lanes 0 and b in the same cycle.  Then the row reads and
    transposed reads of the kernels' LDS tiles, as the kernels address them
    (lane l = 16 g + i of the 16x16x32 fragment layout; rows of 256 bytes,
    128 for E4M3 K), under their chunk permutations and under the first
    versions they replaced, and two controls."""
    pats = []
    for b in range(1, 64):
        offs = [LDS_SKIP] * 64
        offs[0], offs[b] = 0, 256
        pats.append((f"pair: lane 0 and lane {b}", 0, offs))

    def rows16(chunk_of, rowb=256):
        return [(l & 15) * rowb + (chunk_of(l >> 4, l & 15) << 4) for l in range(64)]

    def dual_old(r):
        return ((r & 7) << 1) | ((r >> 3) & 1)

    def dual(r):
        return (((r & 7) ^ ((r >> 1) & 4)) << 1) | ((r >> 3) & 1)

    pats += [
        ("b128 16-bit K rows (16x16x32 forward): chunk g ^ (row & 15)", 0, rows16(lambda g, i: g ^ (i & 15))),
        ("b128 dual-read tiles, first version: chunk g ^ ((row & 7) << 1 | row >> 3)", 0,
         rows16(lambda g, i: g ^ dual_old(i))),
        ("b128 dual-read tiles (backward Q, dO, K): chunk g ^ (((row & 7) ^ (row >> 1 & 4)) << 1 | row >> 3)", 0,
         rows16(lambda g, i: g ^ dual(i))),
        ("b128 E4M3 K rows of 128 bytes, first version: chunk 2g ^ (row >> 1 & 7)", 0,
         rows16(lambda g, i: (2 * g) ^ ((i >> 1) & 7), 128)),
        ("b128 E4M3 K rows of 128 bytes (16x16x128 forward): chunk 2g ^ (row & 6 | row >> 3)", 0,
         rows16(lambda g, i: (2 * g) ^ ((i & 6) | ((i >> 3) & 1)), 128)),
        ("b128 16-bit K rows (32x32x16 kernels): lane l reads row swap23(l % 32) at chunk l / 32 ^ (row & 15)", 0,
         [_swap23(l & 31) * 256 + (((l >> 5) ^ (_swap23(l & 31) & 15)) << 4) for l in range(64)]),
        ("b128 control: rows 0-15 at chunk g (16 rows in one bank group)", 0, rows16(lambda g, i: g)),
    ]

    def tr(perm):
        out = []
        for l in range(64):
            g, i = l >> 4, l & 15
            row = 4 * g + (i >> 2)
            out.append(row * 256 + ((((i & 3) >> 1) ^ perm(row)) << 4) + ((i & 1) << 3))
        return out

    pats += [
        ("tr V^T (16x16x32 forward): 8 rows x 32 bytes per half-wave, chunk pair 2 (row & 7)", 1, tr(lambda r: 2 * (r & 7))),
        ("tr dual-read tiles (backward Q, dO, K)", 1, tr(dual)),
        ("tr control: 8 rows at one chunk pair", 1, tr(lambda r: 0)),
    ]
    return pats


def lds_model_conflict_degree(kind, offsets):
    """Bank-conflict degree of one pattern under the bank model the kernels'
    permutations are built for: 64 banks of 4 bytes (address bits 2-7); a
    ds_read_b128 served in four groups of 16 lanes (in each half-wave, the
    lane quads whose three index bits have even parity, and the odd ones), a
    ds_read_b64_tr_b16 in two groups of 32 (the half-waves).  Returns the
    largest number of distinct dwords one bank serves within a group."""
    size = 16 if kind == 0 else 8
    groups = {}
    for l, o in enumerate(offsets):
        if o == LDS_SKIP:
            continue
        key = (l >> 5, bin((l >> 2) & 7).count("1") & 1) if kind == 0 else (l >> 5,)
        groups.setdefault(key, []).append(o)
    worst = 1
    for offs in groups.values():
        banks = {}
        for o in offs:
            for w in range(size // 4):
                dw = o // 4 + w
                banks.setdefault(dw % 64, set()).add(dw)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def run_lds_probe(blocks=256, iters=1024):
    """One launch per pattern of lds_probe_patterns(), in order (a warm-up
    launch of the first pattern precedes them).  Prints what each launch read;
    run under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS to get each
    pattern's conflict cycles per instruction."""
    import ctypes

    import torch
    from exact_io_aware_65_amd import build as libbuild
    if not os.path.exists(libbuild.PROBE_LIBRARY):
        raise RuntimeError(f"{libbuild.PROBE_LIBRARY} is missing: run python -m exact_io_aware_65_amd.build")
    lib = ctypes.CDLL(libbuild.PROBE_LIBRARY)
    lib.fa_probe_lds.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_uint), ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_lds.restype = ctypes.c_int
    sink = torch.empty(blocks * 64, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    pats = lds_probe_patterns()
    out = []
    for n, (name, kind, offs) in enumerate([pats[0]] + pats):
        arr = (ctypes.c_uint * 64)(*offs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.fa_probe_lds(kind, arr, blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        b.record(stream)
        if rc:
            raise RuntimeError(f"fa_probe_lds failed ({rc}) on pattern {name}")
        torch.cuda.synchronize()
        if n == 0:
            continue  # warm-up launch
        out.append({"pattern": name, "read": "ds_read_b128" if kind == 0 else "ds_read_b64_tr_b16",
                    "active_lanes": sum(o != LDS_SKIP for o in offs), "ms": round(a.elapsed_time(b), 4),
                    "model_conflict_degree": lds_model_conflict_degree(kind, offs)})
    return {"blocks": blocks, "iters": iters, "patterns": out}


def run_data_probe(warmup, steps, rounds=6):
    """fa_fwd on the two long prefill workloads with three kinds of input of
    the same shapes: the seeded workload inputs, all zeros, and constants
    (q = 0.5, k = 0.25, v = 1), and fa_bwd on the first of them with the same
    kinds of data; then, as a control, fa_decode on the decode
    workload's shapes with normal, zero and constant inputs.  The kernel runs the same instructions on all
    three (the rescale branch aside, which the workload inputs rarely take), so
    a difference in time is the data's switching activity in the datapaths,
    i.e. the chip's power limit.  The kinds are timed in interleaved rounds
    and the median round is reported.  Timing only: no parity claim."""
    import torch

    import exact_io_aware_65_amd as fa
    import fa_inputs as fi
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    out = []
    for name in DATA_PROBE:
        w = fi.WORKLOADS[name]
        x = fi.make_inputs(w)
        q, k, v = (fi.bits_to_torch(x[t], w.dtype).to(dev) for t in "qkv")
        x = None
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
        kinds = {"workload": (q, k, v),
                 "zeros": tuple(torch.zeros_like(t) for t in (q, k, v)),
                 "constant": (torch.full_like(q, 0.5), torch.full_like(k, 0.25), torch.full_like(v, 1.0))}
        times = {kind: [] for kind in kinds}
        for r in range(rounds):
            for kind in (list(kinds) if r % 2 == 0 else list(kinds)[::-1]):
                a, b, c = kinds[kind]
                times[kind].append(_event_ms(
                    lambda: fa.fa_fwd(a, b, c, o, lse, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal, w.scale, code, sp),
                    stream, warmup, steps))
        flops = metric_flops(w.B, w.H, w.Nq, w.Nkv, w.d, w.causal)
        base = statistics.median(times["workload"])
        for kind, ts in times.items():
            ms = statistics.median(ts)
            out.append({"workload": name, "inputs": kind, "ms": round(ms, 4),
                        "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "speed_vs_workload_inputs": round(base / ms, 3),
                        "rounds_ms": [round(t, 4) for t in ts]})
            print(f"[data-probe] {name} {kind}: {flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s", file=sys.stderr, flush=True)
        if name == PREFILL:
            # the backward on the same kinds of data: O and LSE from each kind's
            # forward, dO normal / zero / constant like the inputs
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            bws = torch.empty(max(fa.fa_bwd_workspace_size(w.B, w.H, w.Nq), 16), dtype=torch.uint8, device=dev)
            grads = {"workload": fi.device_normals(tuple(q.shape), w.dtype, 400, dev),
                     "zeros": torch.zeros_like(q), "constant": torch.full_like(q, 1.0)}
            saved = {}
            for kind, (a, b, c) in kinds.items():
                ok, lk = torch.empty_like(q), torch.empty_like(lse)
                fa.fa_fwd(a, b, c, ok, lk, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal, w.scale, code, sp)
                saved[kind] = (ok, lk)
            btimes = {kind: [] for kind in kinds}
            for r in range(rounds):
                for kind in (list(kinds) if r % 2 == 0 else list(kinds)[::-1]):
                    a, b, c = kinds[kind]
                    ok, lk = saved[kind]
                    do = grads[kind]
                    btimes[kind].append(_event_ms(
                        lambda: fa.fa_bwd(a, b, c, ok, do, lk, dq, dk, dv, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal,
                                          w.scale, code, bws, bws.numel(), sp), stream, warmup, steps))
            bflops = backward_flops(w.B, w.H, w.Nq, w.Nkv, w.d, w.causal)
            bbase = statistics.median(btimes["workload"])
            for kind, ts in btimes.items():
                ms = statistics.median(ts)
                out.append({"workload": name, "kernel": "fa_bwd", "inputs": kind, "ms": round(ms, 4),
                            "TFLOP/s": round(bflops / (ms * 1e-3) / 1e12, 1),
                            "speed_vs_workload_inputs": round(bbase / ms, 3), "rounds_ms": [round(t, 4) for t in ts]})
                print(f"[data-probe] {name} fa_bwd {kind}: {bflops / (ms * 1e-3) / 1e12:.0f} TFLOP/s", file=sys.stderr,
                      flush=True)
            dq = dk = dv = bws = grads = saved = None
        q = k = v = o = lse = kinds = None
        torch.cuda.empty_cache()
    # Control: decode streams its cache from HBM, so its speed should not
    # depend on the data.  Normal inputs are drawn on the device here.
    w = fi.WORKLOADS[DECODE]
    q = fi.device_normals((w.B, w.H, w.d), w.dtype, 300, dev)
    k, v = (fi.device_normals((w.B, w.H, w.Nkv, w.d), w.dtype, 301 + t, dev) for t in range(2))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    nbytes = fa.fa_decode_workspace_size(w.B, w.H, w.Nkv, w.d, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dcode = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
    kinds = {"normal": (q, k, v)}
    kinds["zeros"] = tuple(torch.zeros_like(t) for t in (q, k, v))
    kinds["constant"] = (torch.full_like(q, 0.5), torch.full_like(k, 0.25), torch.full_like(v, 1.0))
    times = {kind: [] for kind in kinds}
    for r in range(rounds):
        for kind in (list(kinds) if r % 2 == 0 else list(kinds)[::-1]):
            a, b, c = kinds[kind]
            times[kind].append(_event_ms(
                lambda: fa.fa_decode(a, b, c, o, lse, w.B, w.H, w.Nkv, w.d, w.scale, dcode, 0, ws, nbytes, sp),
                stream, warmup, steps))
    nb = algorithmic_bytes(w.B, w.H, 1, w.Nkv, w.d)
    base = statistics.median(times["normal"])
    for kind, ts in times.items():
        ms = statistics.median(ts)
        out.append({"workload": DECODE, "inputs": kind, "ms": round(ms, 4), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                    "speed_vs_workload_inputs": round(base / ms, 3), "rounds_ms": [round(t, 4) for t in ts]})
        print(f"[data-probe] {DECODE} {kind}: {nb / (ms * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    return out


OTHER_PREFILL = ("prefill_2k_d64", "prefill_16k_d128_bf16")


def time_other_prefill(fa, fi, names, dev, stream, warmup, steps, oracle_budget=None):
    """fa_fwd on the other prefill workloads (reported beside the headline one, not part of `value`);
    with oracle_budget the oracle runs beside each (cpu_baseline and parity of the timed outputs)."""
    import torch
    sp = stream.cuda_stream
    res = []
    for name in names:
        w = fi.WORKLOADS[name]
        x = fi.make_inputs(w)
        q, k, v = (fi.bits_to_torch(x[t], w.dtype).to(dev) for t in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
        call = lambda s: fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nkv, w.d, w.causal, w.scale, code, s)
        ms = _event_ms(lambda: call(sp), stream, warmup, steps)
        o_eager, lse_eager = o.clone(), lse.clone()
        ms_graph = _graph_ms(call, 1, steps)  # the eager calls above warmed the kernels
        same = bool(torch.equal(o, o_eager) and torch.equal(lse, lse_eager))
        flops = metric_flops(w.B, w.H, w.Nq, w.Nkv, w.d, w.causal)
        tf, tf_graph = flops / (ms * 1e-3) / 1e12, flops / (ms_graph * 1e-3) / 1e12
        res.append({"workload": name, "B": w.B, "H": w.H, "N": w.Nq, "d": w.d, "dtype": w.dtype, "causal": w.causal,
                    "ms_mean": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_of_mfma_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4),
                    "ms_graph": round(ms_graph, 4), "TFLOP/s_graph": round(tf_graph, 2),
                    "frac_of_mfma_peak_graph": round(tf_graph / PEAK_MFMA_F16_TFLOPS, 4),
                    "graph_output_equals_eager": same,
                    "note": "ms_mean: each call between its own HIP events (includes the host's launch gap for "
                            "short calls); ms_graph: the same calls captured once into a HIP graph and replayed "
                            "back to back"})
        if oracle_budget:
            cpu, parity = oracle_forward_leg(w, lambda b, h: (x["q"][b, h], x["k"][b, h], x["v"][b, h]), o, lse,
                                             budget_s=oracle_budget)
            res[-1]["cpu_baseline"], res[-1]["parity"] = cpu, parity
        q = k = v = o = lse = x = None
    return res


def oracle_paged_leg(w, plan, q, kp, vp, o, lse, budget_s):
    """The oracle beside the paged decode leg: whole sequences, one at a time,
    each over the pool pages its table names (copied back from wherever the
    pool lives, with the table renumbered to them), until budget_s seconds of
    oracle time have passed.  q and o are [B, H, 1, d] (o as timed, in the
    input type), lse [B, H], kp / vp the 'hnd' pool [P, H, ps, d].  Returns
    the parity record and the cpu_baseline."""
    import time

    import numpy as np
    import torch

    import fa_inputs as fi
    import oracle
    o_all = o.float().cpu().numpy().reshape(w.B, w.H, w.d)
    lse_all = lse.float().cpu().numpy().reshape(w.B, w.H)
    wo, wl = Worst(), Worst()
    spent, seqs, seq_keys = 0.0, 0, 0
    for b in range(w.B):
        n = int(plan.seq_lens[b])
        pages = plan.block_table[b, :-(-n // plan.page_size)].astype(np.int64)
        idx = torch.from_numpy(pages).to(kp.device)
        kb, vb = (fi.torch_to_bits(t[idx].cpu()) for t in (kp, vp))
        qb = fi.torch_to_bits(q[b:b + 1].reshape(1, w.H, w.d).cpu())
        table_b = np.arange(len(pages), dtype=np.int32)[None]
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.paged_decode(qb, kb, vb, table_b, np.array([n], dtype=np.int32), scale=w.scale,
                                             layout="hnd", dtype=w.dtype)
        spent += time.perf_counter() - t0
        seqs += 1
        seq_keys += n
        wo.add(o_all[b], o_ref[0], (b,))
        wl.add(lse_all[b], lse_ref[0], (b,))
        if spent >= budget_s:
            break
    ro, ok_o = wo.record("O", TOL_O[w.dtype])
    rl, ok_l = wl.record("LSE", TOL_LSE)
    sample_bytes = 2 * seq_keys * w.H * w.d * 2 + algorithmic_bytes(1, seqs * w.H, 1, 0, w.d)
    return {
        "parity": {**ro, **rl, "tol_O": TOL_O[w.dtype], "tol_LSE": TOL_LSE, "pass": ok_o and ok_l,
                   "compared": f"O ({w.dtype}, as timed) and LSE of {seqs} of {w.B} sequences (all heads)",
                   "index": "worst_O = [b, h, dim], worst_LSE = [b, h]"},
        "cpu_baseline": {"value": sample_bytes / max(spent, 1e-9) / 1e9, "unit": "GB/s", "cores": oracle.threads(),
                         "kind": "oracle", "seconds": round(spent, 2),
                         "sample": f"{seqs} of {w.B} sequences of {w.name} through the oracle's paged "
                                   f"gather (fp64), {spent:.1f} s"},
    }


def time_paged_decode(fa, fi, w, q, k, v, stream, warmup, steps, num_splits, dense_o=None, oracle_budget=None):
    """fa_decode_paged on workload w: the dense decode cache k, v scattered into a
    shuffled page pool, each call bracketed by HIP events.  dense_o (fa_decode's
    output on the dense cache) is compared bit for bit; with oracle_budget the
    oracle's paged decode runs on whole sequences (each over the pool pages its
    table names, copied back from the device, with the table renumbered to
    them) until that many seconds have passed."""
    import statistics

    import numpy as np
    import torch
    plan = fi.workload_plan(w)
    kp, vp = fi.scatter_to_pages_torch(k, plan), fi.scatter_to_pages_torch(v, plan)
    table = torch.from_numpy(plan.block_table).to(q.device)
    lens = torch.from_numpy(plan.seq_lens).to(q.device)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=q.device)
    nbytes = fa.fa_decode_workspace_size(w.B, w.H, w.Nkv, w.d, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    sp = stream.cuda_stream
    max_pages = plan.block_table.shape[1]

    def call():
        fa.fa_decode_paged(q, kp, vp, table, lens, o, lse, w.B, w.H, w.d, plan.num_pages, plan.page_size,
                           max_pages, fa.FA_PAGED_HND, w.Nkv, w.scale, fa.FA_F16, num_splits, ws, nbytes, sp)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    mean = statistics.fmean(ms)
    keys = int(np.asarray(plan.seq_lens, dtype=np.int64).sum())
    nbytes_alg = 2 * keys * w.H * w.d * 2 + algorithmic_bytes(w.B, w.H, 1, 0, w.d) + plan.block_table.nbytes + \
        plan.seq_lens.nbytes
    gbs = nbytes_alg / (mean * 1e-3) / 1e9
    extra = {}
    if dense_o is not None:
        extra["bitwise_equal_to_dense_decode"] = bool(torch.equal(o, dense_o))
    if oracle_budget:
        extra.update(oracle_paged_leg(w, plan, q, kp, vp, o, lse, oracle_budget))
    return {
        "workload": w.name,
        "page_size": plan.page_size,
        "layout": "hnd",
        "num_pages": plan.num_pages,
        "ms_mean": round(mean, 4),
        "ms_min": round(min(ms), 4),
        "algorithmic_bytes": nbytes_alg,
        "GB/s": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic("decode", "paged"),
        "note": "the dense decode cache scattered into a shuffled pool of 16-key pages; bytes are K and V "
                "once, q, o, lse, the block table and the lengths",
        **extra,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--num-splits", type=int, default=0, help="decode split count (0 = library choice)")
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all",
                    help="time only one half of the step (for profiling; the default is the whole path)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the separate timing of the backward (fa_bwd) on the prefill workload")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the separate timing of decode over a paged cache (fa_decode_paged)")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the speed-vs-length sweep of the fused kernels against the unfused baseline")
    ap.add_argument("--map", action="store_true",
                    help="only run the speed map of the fused kernels over sequence length, head dim, mask and type")
    ap.add_argument("--data-probe", action="store_true",
                    help="only time fa_fwd on the long prefill workloads (and fa_decode as a control) with workload, all-zero and constant inputs")
    ap.add_argument("--lds-probe", action="store_true",
                    help="only run the LDS bank probe (one launch per access pattern; counters from rocprofv3)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the timing of the other prefill workloads (2K d64, 16K d128 bf16)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the separate timing of the FP8 Q/K forward (fa_fwd_fp8) on the prefill workload")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep:
        if args.gpus != 1:
            sys.exit("bench.py --sweep measures one GPU only")
        res = run_sweep(max(1, args.warmup), max(1, args.steps))
        print(json.dumps({"metric": "fused vs unfused attention time over sequence length", "unit": "ms",
                          "higher_is_better": False, "dtype": "f16", "data": "synthetic", "sweep": res}), flush=True)
        return
    if args.map:
        if args.gpus != 1:
            sys.exit("bench.py --map measures one GPU only")
        res = run_map(max(1, args.warmup), max(1, args.steps))
        print(json.dumps({"metric": "fused kernel speed over shapes", "unit": "TFLOP/s, GB/s",
                          "higher_is_better": True, "data": "synthetic", "map": res}), flush=True)
        return
    if args.lds_probe:
        if args.gpus != 1:
            sys.exit("bench.py --lds-probe measures one GPU only")
        res = run_lds_probe()
        print(json.dumps({"metric": "LDS access patterns, one launch each (bank conflicts from SQ_LDS_BANK_CONFLICT)",
                          "unit": "ms", "higher_is_better": False, "data": "synthetic", "lds_probe": res}), flush=True)
        return
    if args.data_probe:
        if args.gpus != 1:
            sys.exit("bench.py --data-probe measures one GPU only")
        res = run_data_probe(max(1, args.warmup), max(1, args.steps))
        print(json.dumps({"metric": "fa_fwd speed by input data at fixed shapes", "unit": "TFLOP/s",
                          "higher_is_better": True, "data": "synthetic", "probe": res}), flush=True)
        return
    if args.gpus != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
                  "(across GPUs the kernels would shard by head, with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import exact_io_aware_65_amd as fa
    import fa_inputs as fi

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    pw, dw = fi.WORKLOADS[PREFILL], fi.WORKLOADS[DECODE]

    run_prefill = args.only in ("all", "prefill")
    run_decode = args.only in ("all", "decode")
    oracle_on = not args.no_cpu_baseline
    px = dx = None
    if run_prefill:
        log(f"generating {PREFILL}")
        px = fi.make_inputs(pw)
    if run_prefill:
        pq, pk, pv = (fi.bits_to_torch(px[t], pw.dtype).to(dev) for t in "qkv")
        po = torch.empty_like(pq)
        plse = torch.empty((pw.B, pw.H, pw.Nq), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_decode_workspace_size(dw.B, dw.H, dw.Nkv, dw.d, args.num_splits)
    splits = fa.fa_decode_num_splits(dw.B, dw.H, dw.Nkv, dw.d) if args.num_splits == 0 else \
        ws_bytes // (dw.B * dw.H * (dw.d + 1) * 4)
    if run_decode:
        log(f"generating {DECODE}")
        dx = fi.make_inputs(dw)
        dq, dk, dv = (fi.bits_to_torch(dx[t], dw.dtype).to(dev) for t in "qkv")
        if not oracle_on:
            dx = None  # the host copy only serves the oracle
        do = torch.empty_like(dq)
        dlse = torch.empty((dw.B, dw.H), dtype=torch.float32, device=dev)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def step(ev):
        ev[0].record(stream)
        if run_prefill:
            fa.fa_fwd(pq, pk, pv, po, plse, pw.B, pw.H, pw.Nq, pw.Nkv, pw.d, pw.causal, pw.scale, fa.FA_F16, sp)
        ev[1].record(stream)
        if run_decode:
            fa.fa_decode(dq, dk, dv, do, dlse, dw.B, dw.H, dw.Nkv, dw.d, dw.scale, fa.FA_F16, args.num_splits,
                         ws, ws_bytes, sp)
        ev[2].record(stream)

    def events():
        return tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [a.elapsed_time(b) for a, b, _ in evs]
    dec_ms = [b.elapsed_time(c) for _, b, c in evs]

    p_flops = metric_flops(pw.B, pw.H, pw.Nq, pw.Nkv, pw.d, pw.causal)
    p_bytes = algorithmic_bytes(pw.B, pw.H, pw.Nq, pw.Nkv, pw.d)
    d_bytes = algorithmic_bytes(dw.B, dw.H, 1, dw.Nkv, dw.d)
    fwd_mean = statistics.fmean(fwd_ms)
    dec_mean = statistics.fmean(dec_ms)
    tflops = p_flops / (fwd_mean * 1e-3) / 1e12 if run_prefill else 0.0
    gbs = d_bytes / (dec_mean * 1e-3) / 1e9 if run_decode else 0.0

    def pct(xs, q):
        xs = sorted(xs)
        return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{PREFILL} + {DECODE}",
            "prefill": {"B": pw.B, "H": pw.H, "Nq": pw.Nq, "Nkv": pw.Nkv, "d": pw.d, "causal": pw.causal,
                        "dtype": pw.dtype, "seed": pw.seed, "sigma_qk": pw.sigma_qk},
            "decode": {"B": dw.B, "H": dw.H, "Nq": 1, "Nkv": dw.Nkv, "d": dw.d, "dtype": dw.dtype,
                       "seed": dw.seed, "num_splits": splits},
        },
        "roofline": {
            "kernel": "fwd16_kernel<128, f16, causal, 8 waves>",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": measured_traffic("prefill"),
        },
        "roofline_decode": {
            "kernel": "decode_split_kernel<128, f16> + decode_combine_kernel",
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("decode"),
        },
        "prefill": {"ms_mean": round(fwd_mean, 4), "ms_p10": round(pct(fwd_ms, 0.1), 4),
                    "ms_p50": round(pct(fwd_ms, 0.5), 4), "ms_p90": round(pct(fwd_ms, 0.9), 4),
                    "flops": p_flops, "algorithmic_bytes": p_bytes},
        "decode": {"ms_mean": round(dec_mean, 4), "ms_p10": round(pct(dec_ms, 0.1), 4),
                   "ms_p50": round(pct(dec_ms, 0.5), 4), "ms_p90": round(pct(dec_ms, 0.9), 4),
                   "GB/s": round(gbs, 1), "algorithmic_bytes": d_bytes, "workspace_bytes": ws_bytes},
        "gpu": {"name": device_name(props), "cus": props.multi_processor_count,
                "arch": getattr(props, "gcnArchName", ""), "hip": torch.version.hip},
        "build": build_info(),
        "sources": {"prefill_digest": kernel_source_digest("prefill"),
                    "decode_digest": kernel_source_digest("decode")},
    }
    budget = ORACLE_BUDGET_S if oracle_on else None
    fwd_ref = None
    if oracle_on:
        result["host"] = host_info()
    if oracle_on and run_prefill:
        log("oracle beside the prefill leg (cpu baseline, parity of the timed outputs)")
        cpu, parity, fwd_ref = oracle_forward_leg(pw, lambda b, h: (px["q"][b, h], px["k"][b, h], px["v"][b, h]),
                                                  po, plse, keep_ref=True)
        result["cpu_baseline"] = cpu
        result["prefill"]["parity"] = parity
    if oracle_on and run_decode:
        log("oracle beside the decode leg")
        cpu, parity = oracle_decode_leg(dw, lambda b, h: (dx["q"][b, h], dx["k"][b, h], dx["v"][b, h]), do, dlse)
        result["decode"]["cpu_baseline"], result["decode"]["parity"] = cpu, parity
        if not run_prefill:
            result["cpu_baseline"] = cpu
        dx = None
    if run_prefill and not args.no_bwd:
        log("backward (fa_bwd) on the prefill workload")
        result["backward"] = time_backward(fa, fi, pw, pq, pk, pv, stream, args.warmup, args.steps, fwd_ref=fwd_ref,
                                           oracle_budget=budget)
    if run_prefill and not args.no_other:
        log("other prefill workloads (fa_fwd)")
        result["other_prefill"] = time_other_prefill(fa, fi, OTHER_PREFILL, dev, stream, args.warmup, args.steps,
                                                     oracle_budget=budget)
    if run_prefill and not args.no_fp8:
        log("FP8 Q/K forward (fa_fwd_fp8) on the prefill workload")
        result["fp8_forward"] = time_fp8_forward(
            fa, fi, pw, pq, pk, pv, stream, args.warmup, args.steps,
            head_inputs=(lambda b, h: (px["q"][b, h], px["k"][b, h], px["v"][b, h])) if oracle_on else None)
    if run_decode:
        log("streaming-read probe over the decode K cache")
        probe = measure_read_bandwidth(dk, stream, args.warmup, args.steps)
        result["read_probe"] = probe
        result["decode"]["frac_of_read_probe"] = round(gbs / probe["GB/s"], 4)
    if run_decode and not args.no_paged:
        log("decode over a paged cache (fa_decode_paged)")
        result["paged_decode"] = time_paged_decode(fa, fi, fi.WORKLOADS[PAGED], dq, dk, dv, stream, args.warmup,
                                                   args.steps, args.num_splits, dense_o=do, oracle_budget=budget)
    if args.only != "all":
        result["partial_step"] = args.only
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
