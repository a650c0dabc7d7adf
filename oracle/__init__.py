"""fp64 CPU reference for exact softmax attention.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU package never
imports this module, and this module imports nothing from the GPU package.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, materialises the
score matrix per head); this wrapper only marshals numpy arrays.  What it
computes, with citations, is stated at the top of that file:

    S = scale * Q K^T (masked entries -inf), P = softmax(S) row-wise,
    O = P V, LSE = m + ln(l)

and, for the backward with dL/dO = dO, the chain rule through that definition:

    dV = P^T dO, dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D),
    dQ = scale * dS K, dK = scale * dS^T Q

(with D optionally formed as rowsum(dO * O) from a given forward output O,
the O a training step hands its backward)
decode over a paged cache (the dense attention over each sequence's keys,
gathered through a block table), and the FP8 variant (Q and K rounded to
E4M3 -- nearest even, saturating at 448 -- before the first product).

All functions pinned by tests/test_oracle_pins.py (brute force at 50 digits,
torch float64 SDPA, closed forms and invariants); no function here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "attn_oracle.c")
LIBRARY = os.path.join(HERE, "libattn_oracle.so")

KINDS = {"f16": 1, "bf16": 2}


def build(source: str = SOURCE, out: str = LIBRARY, extra_flags=()) -> str:
    """Compile the reference with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           source, "-lm", "-o", out]
    subprocess.run(cmd, check=True)
    return out


_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """ctypes handle on one build of attn_oracle.c."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(out=path)
        lib = ctypes.CDLL(path)
        lib.fa_oracle_widen.argtypes = [ctypes.POINTER(ctypes.c_uint16), _dp, _i64, ctypes.c_int]
        lib.fa_oracle_widen.restype = ctypes.c_int
        lib.fa_oracle_attention.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_int, ctypes.c_double]
        lib.fa_oracle_attention.restype = ctypes.c_int
        lib.fa_oracle_attention_rows.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int,
                                                 ctypes.c_double, ctypes.POINTER(_i64), _i64,
                                                 _dp, _dp]
        lib.fa_oracle_attention_rows.restype = ctypes.c_int
        lib.fa_oracle_attention_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                                _i64, _i64, ctypes.c_int, ctypes.c_double]
        lib.fa_oracle_attention_bwd.restype = ctypes.c_int
        lib.fa_oracle_attention_bwd_sampled.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int,
                                                        ctypes.c_double, ctypes.POINTER(_i64), _i64,
                                                        ctypes.POINTER(_i64), _i64, _dp, _dp, _dp]
        lib.fa_oracle_attention_bwd_sampled.restype = ctypes.c_int
        _i32p = ctypes.POINTER(ctypes.c_int32)
        lib.fa_oracle_paged_decode.argtypes = [_dp, _dp, _dp, _i32p, _i32p, _dp, _dp, _i64, _i64, _i64, _i64,
                                               _i64, _i64, ctypes.c_int, ctypes.c_double]
        lib.fa_oracle_paged_decode.restype = ctypes.c_int
        lib.fa_oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.fa_oracle_e4m3_to_f64.restype = ctypes.c_double
        lib.fa_oracle_quantize_e4m3.argtypes = [_dp, ctypes.POINTER(ctypes.c_uint8), _i64]
        lib.fa_oracle_quantize_e4m3.restype = ctypes.c_int
        lib.fa_oracle_attention_fp8qk.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                                  ctypes.c_int, ctypes.c_double]
        lib.fa_oracle_attention_fp8qk.restype = ctypes.c_int
        lib.fa_oracle_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- inputs -----------------------------------------------------------
    def widen(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """Exact float64 values of uint16 bit patterns of type dtype ('f16' or 'bf16')."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        rc = self.lib.fa_oracle_widen(_ptr(bits, ctypes.c_uint16), _ptr(out), bits.size,
                                      KINDS[dtype])
        if rc:
            raise ValueError("widen failed")
        return out

    def _as_f64(self, x: np.ndarray, dtype):
        if dtype is None:
            return np.ascontiguousarray(x, dtype=np.float64)
        return self.widen(x, dtype)

    # -- attention --------------------------------------------------------
    def attention(self, q, k, v, *, causal: bool, scale: float, dtype=None):
        """O [B,H,Nq,d] and LSE [B,H,Nq] in float64.

        q, k, v are [B,H,N,d] (or [N,d] for a single head) float arrays, or
        uint16 bit patterns when dtype is 'f16'/'bf16'."""
        q, k, v = (self._as_f64(t, dtype) for t in (q, k, v))
        squeeze = q.ndim == 2
        if squeeze:
            q, k, v = q[None, None], k[None, None], v[None, None]
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d):
            raise ValueError("shape mismatch")
        o = np.empty((B, H, Nq, d), dtype=np.float64)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.fa_oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq,
                                          Nkv, d, int(bool(causal)), float(scale))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        if squeeze:
            return o[0, 0], lse[0, 0]
        return o, lse

    def attention_rows(self, q, k, v, rows, *, causal: bool, scale: float, dtype=None):
        """Selected query rows of one head: q [Nq,d], k/v [Nkv,d] -> O [n,d], LSE [n]."""
        q, k, v = (self._as_f64(t, dtype) for t in (q, k, v))
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        Nq, d = q.shape
        Nkv = k.shape[0]
        o = np.empty((rows.size, d), dtype=np.float64)
        lse = np.empty(rows.size, dtype=np.float64)
        rc = self.lib.fa_oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), Nq, Nkv, d,
                                               int(bool(causal)), float(scale),
                                               _ptr(rows, _i64), rows.size, _ptr(o), _ptr(lse))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        return o, lse

    def attention_bwd(self, q, k, v, dout, *, causal: bool, scale: float, dtype=None, o_for_d=None):
        """(dQ, dK, dV) in float64 for dL/dO = dout; shapes as for attention().

        o_for_d (like q; bits when dtype is given): the forward output the
        backward is handed, from which D_i = sum_c dout_ic o_ic is formed;
        None forms D from P itself (the same value for the exact O)."""
        q, k, v, dout = (self._as_f64(t, dtype) for t in (q, k, v, dout))
        od = None if o_for_d is None else self._as_f64(o_for_d, dtype)
        squeeze = q.ndim == 2
        if squeeze:
            q, k, v, dout = q[None, None], k[None, None], v[None, None], dout[None, None]
            od = None if od is None else od[None, None]
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d) or dout.shape != q.shape or \
                (od is not None and od.shape != q.shape):
            raise ValueError("shape mismatch")
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(v)
        rc = self.lib.fa_oracle_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                              None if od is None else _ptr(od), _ptr(dq), _ptr(dk),
                                              _ptr(dv), B, H, Nq, Nkv, d, int(bool(causal)), float(scale))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        if squeeze:
            return dq[0, 0], dk[0, 0], dv[0, 0]
        return dq, dk, dv

    def attention_bwd_sampled(self, q, k, v, dout, qrows, kcols, *, causal: bool, scale: float, dtype=None,
                              o_for_d=None):
        """One head: dQ at query rows qrows [n,d], dK and dV at key rows kcols [m,d]; o_for_d as for
        attention_bwd ([Nq,d])."""
        q, k, v, dout = (self._as_f64(t, dtype) for t in (q, k, v, dout))
        od = None if o_for_d is None else self._as_f64(o_for_d, dtype)
        if od is not None and od.shape != q.shape:
            raise ValueError("shape mismatch")
        qrows = np.ascontiguousarray(qrows, dtype=np.int64)
        kcols = np.ascontiguousarray(kcols, dtype=np.int64)
        Nq, d = q.shape
        Nkv = k.shape[0]
        dq = np.empty((qrows.size, d))
        dk = np.empty((kcols.size, d))
        dv = np.empty((kcols.size, d))
        rc = self.lib.fa_oracle_attention_bwd_sampled(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                                      None if od is None else _ptr(od), Nq, Nkv, d,
                                                      int(bool(causal)), float(scale), _ptr(qrows, _i64),
                                                      qrows.size, _ptr(kcols, _i64), kcols.size, _ptr(dq),
                                                      _ptr(dk), _ptr(dv))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        return dq, dk, dv

    def paged_decode(self, q, k_pages, v_pages, block_table, seq_lens, *, scale: float, layout: str = "hnd",
                     dtype=None):
        """Decode over a paged cache: O [B,H,d] and LSE [B,H] in float64.

        q is [B,H,d]; k_pages / v_pages are [num_pages,H,page_size,d] for
        layout 'hnd' or [num_pages,page_size,H,d] for 'nhd'; block_table is
        [B,max_pages] and seq_lens [B] (int32).  A sequence of length 0 gets
        O = 0 and LSE = -inf."""
        q, k_pages, v_pages = (self._as_f64(t, dtype) for t in (q, k_pages, v_pages))
        table = np.ascontiguousarray(block_table, dtype=np.int32)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, H, d = q.shape
        if layout == "hnd":
            P, Hk, ps, dk = k_pages.shape
        elif layout == "nhd":
            P, ps, Hk, dk = k_pages.shape
        else:
            raise ValueError(f"layout must be 'hnd' or 'nhd', got {layout!r}")
        if (Hk, dk) != (H, d) or v_pages.shape != k_pages.shape or table.ndim != 2 or table.shape[0] != B \
                or lens.shape != (B,):
            raise ValueError("shape mismatch")
        o = np.empty((B, H, d), dtype=np.float64)
        lse = np.empty((B, H), dtype=np.float64)
        rc = self.lib.fa_oracle_paged_decode(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(table, ctypes.c_int32),
                                             _ptr(lens, ctypes.c_int32), _ptr(o), _ptr(lse), B, H, P, ps,
                                             table.shape[1], d, 0 if layout == "hnd" else 1, float(scale))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        return o, lse

    # -- FP8 (E4M3) Q and K -------------------------------------------------
    def quantize_e4m3(self, x, dtype=None) -> np.ndarray:
        """E4M3 codes (uint8) of x: round to nearest even, saturate beyond 448."""
        x = self._as_f64(x, dtype)
        codes = np.empty(x.shape, dtype=np.uint8)
        rc = self.lib.fa_oracle_quantize_e4m3(_ptr(x), _ptr(codes, ctypes.c_uint8), x.size)
        if rc:
            raise ValueError("quantize failed")
        return codes

    def e4m3_to_f64(self, codes) -> np.ndarray:
        """Exact values of E4M3 codes."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        table = np.array([self.lib.fa_oracle_e4m3_to_f64(c) for c in range(256)], dtype=np.float64)
        return table[codes]

    def attention_fp8qk(self, q, k, v, *, causal: bool, scale: float, dtype=None, k_codes: bool = False):
        """Attention with Q and K quantised to E4M3 first: O [B,H,Nq,d], LSE [B,H,Nq].

        q, v are as for attention(); k is the same, or E4M3 codes (uint8) when
        k_codes is set (a cache already held in FP8)."""
        q, v = self._as_f64(q, dtype), self._as_f64(v, dtype)
        k = self.e4m3_to_f64(k) if k_codes else self._as_f64(k, dtype)
        squeeze = q.ndim == 2
        if squeeze:
            q, k, v = q[None, None], k[None, None], v[None, None]
        B, H, Nq, d = q.shape
        Nkv = k.shape[2]
        if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d):
            raise ValueError("shape mismatch")
        o = np.empty((B, H, Nq, d), dtype=np.float64)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.fa_oracle_attention_fp8qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nkv, d,
                                                int(bool(causal)), float(scale))
        if rc:
            raise ValueError(f"oracle rejected the call (rc={rc})")
        if squeeze:
            return o[0, 0], lse[0, 0]
        return o, lse

    def attention_fp8qk_rows(self, q, k, v, rows, *, causal: bool, scale: float, dtype=None, k_codes: bool = False):
        """Selected query rows of one head for the FP8 variant: Q and K are
        quantised (through the same codec), then attention_rows runs."""
        q8 = self.e4m3_to_f64(self.quantize_e4m3(q, dtype))
        k8 = self.e4m3_to_f64(k if k_codes else self.quantize_e4m3(k, dtype))
        return self.attention_rows(q8, k8, self._as_f64(v, dtype), rows, causal=causal, scale=scale)

    def threads(self) -> int:
        return int(self.lib.fa_oracle_threads())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def widen(bits, dtype):
    return default().widen(bits, dtype)


def attention(q, k, v, *, causal, scale, dtype=None):
    return default().attention(q, k, v, causal=causal, scale=scale, dtype=dtype)


def attention_rows(q, k, v, rows, *, causal, scale, dtype=None):
    return default().attention_rows(q, k, v, rows, causal=causal, scale=scale, dtype=dtype)


def attention_bwd(q, k, v, dout, *, causal, scale, dtype=None, o_for_d=None):
    return default().attention_bwd(q, k, v, dout, causal=causal, scale=scale, dtype=dtype, o_for_d=o_for_d)


def attention_bwd_sampled(q, k, v, dout, qrows, kcols, *, causal, scale, dtype=None, o_for_d=None):
    return default().attention_bwd_sampled(q, k, v, dout, qrows, kcols, causal=causal, scale=scale, dtype=dtype,
                                           o_for_d=o_for_d)


def paged_decode(q, k_pages, v_pages, block_table, seq_lens, *, scale, layout="hnd", dtype=None):
    return default().paged_decode(q, k_pages, v_pages, block_table, seq_lens, scale=scale, layout=layout,
                                  dtype=dtype)


def quantize_e4m3(x, dtype=None):
    return default().quantize_e4m3(x, dtype)


def e4m3_to_f64(codes):
    return default().e4m3_to_f64(codes)


def attention_fp8qk(q, k, v, *, causal, scale, dtype=None, k_codes=False):
    return default().attention_fp8qk(q, k, v, causal=causal, scale=scale, dtype=dtype, k_codes=k_codes)


def attention_fp8qk_rows(q, k, v, rows, *, causal, scale, dtype=None, k_codes=False):
    return default().attention_fp8qk_rows(q, k, v, rows, causal=causal, scale=scale, dtype=dtype, k_codes=k_codes)


def threads() -> int:
    return default().threads()
