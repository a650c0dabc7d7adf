"""ctypes binding of libfa355 (include/fa355.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfa355.so.  PyTorch supplies device memory and the current
stream.  The library must have been built (``python -m
exact_io_aware_65_amd.build``); there is no fallback of any kind.

Thin wrappers with the C names (``fa_fwd``, ``fa_fwd_fp8``, ``fa_decode``,
``fa_decode_noalloc``, ``fa_decode_paged``, ``fa_bwd``, ...)
take device pointers or tensors and raise :class:`FaError` on a non-OK
status.  The convenience functions :func:`fwd`, :func:`fwd_fp8`,
:func:`quantize_e4m3`, :func:`decode`, :func:`decode_paged` and :func:`bwd`
allocate the outputs.
"""
from __future__ import annotations

import ctypes
import math
import os

# FA355_LIBRARY selects another build of the same library (the LDS-poisoning
# debug build, for one); by default the in-tree libfa355.so.
LIBRARY = os.environ.get("FA355_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")

FA_F16 = 1
FA_BF16 = 2
FA_OUT_F32 = 0x100
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_PAGED_HND = 0  # pages [num_pages, H, page_size, d]
FA_PAGED_NHD = 1  # pages [num_pages, page_size, H, d]
FA_DECODE_NOALLOC_SCRATCH_BYTES = 4 << 20  # fa_decode_noalloc's device scratch


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{fa_status_str(status)}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libfa355.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"{LIBRARY} is missing: build it with `python -m exact_io_aware_65_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        lib.fa_decode.restype = i
        lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        lib.fa_decode_noalloc.restype = i
        lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i]
        lib.fa_decode_workspace_size.restype = ctypes.c_size_t
        lib.fa_decode_num_splits.argtypes = [i, i, i, i]
        lib.fa_decode_num_splits.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_quantize_e4m3.argtypes = [vp, vp, ctypes.c_size_t, i, vp]
        lib.fa_quantize_e4m3.restype = i
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.fa_decode_paged.argtypes = [vp, vp, vp, i32p, i32p, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp,
                                        ctypes.c_size_t, vp]
        lib.fa_decode_paged.restype = i
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_workspace_size.argtypes = [i, i, i]
        lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
        lib.fa_status_str.argtypes = [i]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_version.restype = i
        _lib = lib
    return _lib


def _addr(x):
    """Device address of a tensor, handle of a torch stream (an int or None passes through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "cuda_stream"):
        return x.cuda_stream
    return x.data_ptr()


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, fa_last_error())


# ---------------------------------------------------------------------------
# the C entry points, one to one

def fa_fwd(q, k, v, o, lse, B, H, Nq, Nkv, d, causal, scale, dtype, stream=None) -> None:
    _check(library().fa_fwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, H, Nq, Nkv, d,
                            int(bool(causal)), float(scale), int(dtype), _addr(stream)))


def fa_fwd_fp8(q, k8, v, o, lse, B, H, Nq, Nkv, d, causal, scale, dtype, stream=None) -> None:
    _check(library().fa_fwd_fp8(_addr(q), _addr(k8), _addr(v), _addr(o), _addr(lse), B, H, Nq, Nkv, d,
                                int(bool(causal)), float(scale), int(dtype), _addr(stream)))


def fa_quantize_e4m3(x, y, n, dtype, stream=None) -> None:
    _check(library().fa_quantize_e4m3(_addr(x), _addr(y), int(n), int(dtype), _addr(stream)))


def fa_decode(q, k, v, o, lse, B, H, Nkv, d, scale, dtype, num_splits, workspace, workspace_bytes,
              stream=None) -> None:
    _check(library().fa_decode(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, H, Nkv, d,
                               float(scale), int(dtype), int(num_splits), _addr(workspace),
                               int(workspace_bytes), _addr(stream)))


def fa_decode_noalloc(q, k, v, o, lse, B, H, Nkv, d, scale, dtype, num_splits, stream=None) -> None:
    _check(library().fa_decode_noalloc(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, H, Nkv, d,
                                       float(scale), int(dtype), int(num_splits), _addr(stream)))


def fa_decode_workspace_size(B, H, Nkv, d, num_splits=0) -> int:
    return int(library().fa_decode_workspace_size(B, H, Nkv, d, num_splits))


def fa_decode_num_splits(B, H, Nkv, d) -> int:
    return int(library().fa_decode_num_splits(B, H, Nkv, d))


def fa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, lse, B, H, d, num_pages, page_size, max_pages,
                    layout, max_seq_len, scale, dtype, num_splits, workspace, workspace_bytes, stream=None) -> None:
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check(library().fa_decode_paged(_addr(q), _addr(k_pages), _addr(v_pages),
                                     ctypes.cast(_addr(block_table), i32p), ctypes.cast(_addr(seq_lens), i32p),
                                     _addr(o), _addr(lse), B, H, d, num_pages, page_size, max_pages, int(layout),
                                     int(max_seq_len), float(scale), int(dtype), int(num_splits), _addr(workspace),
                                     int(workspace_bytes), _addr(stream)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, causal, scale, dtype, workspace,
           workspace_bytes, stream=None) -> None:
    _check(library().fa_bwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(dout), _addr(lse), _addr(dq),
                            _addr(dk), _addr(dv), B, H, Nq, Nkv, d, int(bool(causal)), float(scale), int(dtype),
                            _addr(workspace), int(workspace_bytes), _addr(stream)))


def fa_bwd_workspace_size(B, H, Nq) -> int:
    return int(library().fa_bwd_workspace_size(B, H, Nq))


def fa_status_str(status: int) -> str:
    return library().fa_status_str(status).decode()


def fa_last_error() -> str:
    return library().fa_last_error().decode()


def fa_version() -> int:
    return int(library().fa_version())


# ---------------------------------------------------------------------------
# tensor conveniences

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"q, k, v must be float16 or bfloat16, got {t.dtype}")


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _check_rank(dims, **tensors):
    for name, t in tensors.items():
        if t.dim() != dims:
            raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(t.shape)}")


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def fwd(q, k, v, *, causal=False, scale=None, out_dtype=None, with_lse=True):
    """O = softmax(scale * q k^T [causal]) v and LSE for [B, H, N, d] tensors.

    Returns (o, lse); lse is None when with_lse is False.  out_dtype may be
    torch.float32 to get O in fp32, else O has q's dtype."""
    import torch
    _check_inputs(q, k, v)
    _check_rank(4, q=q, k=k, v=v)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    code = _dtype_code(q)
    odt = q.dtype
    if out_dtype is not None and out_dtype != q.dtype:
        if out_dtype != torch.float32:
            raise TypeError("out_dtype must be None, q.dtype or torch.float32")
        code |= FA_OUT_F32
        odt = torch.float32
    o = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if with_lse else None
    with torch.cuda.device(q.device):
        fa_fwd(q, k, v, o, lse, B, H, Nq, Nkv, d, causal, scale, code, _stream(q.device))
    return o, lse


def quantize_e4m3(x):
    """E4M3 bytes (a uint8 tensor shaped like x) of a contiguous float16 / bfloat16 GPU tensor."""
    import torch
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        fa_quantize_e4m3(x, y, x.numel(), _dtype_code(x), _stream(x.device))
    return y


def fwd_fp8(q, k, v, *, causal=False, scale=None, out_dtype=None, with_lse=True):
    """fwd with Q and K rounded to E4M3 for the first product.

    k is either 16-bit like q (rounded here by fa_quantize_e4m3) or already
    E4M3: a uint8 or torch.float8_e4m3fn tensor [B, H, Nkv, d].  Returns (o, lse)."""
    import torch
    if k.dtype in (torch.float16, torch.bfloat16):
        if k.dtype != q.dtype:
            raise TypeError("a 16-bit k must have q's dtype")
        _check_inputs(q, k, v)
        k8 = quantize_e4m3(k)
    elif k.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        _check_inputs(q, v, v)
        if not k.is_cuda or not k.is_contiguous() or k.device != q.device:
            raise ValueError("k must be a contiguous GPU tensor on q's device")
        k8 = k
    else:
        raise TypeError(f"k must be float16, bfloat16, uint8 or float8_e4m3fn, got {k.dtype}")
    _check_rank(4, q=q, k=k, v=v)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    code = _dtype_code(q)
    odt = q.dtype
    if out_dtype is not None and out_dtype != q.dtype:
        if out_dtype != torch.float32:
            raise TypeError("out_dtype must be None, q.dtype or torch.float32")
        code |= FA_OUT_F32
        odt = torch.float32
    o = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if with_lse else None
    with torch.cuda.device(q.device):
        fa_fwd_fp8(q, k8, v, o, lse, B, H, Nq, Nkv, d, causal, scale, code, _stream(q.device))
    return o, lse


def decode(q, k, v, *, scale=None, num_splits=0, out_dtype=None):
    """One query per (b, h): q [B, H, d] (or [B, H, 1, d]), k/v [B, H, Nkv, d].

    Returns (o, lse) with o shaped like q."""
    import torch
    _check_inputs(q, k, v)
    _check_rank(4, k=k, v=v)
    B, H, Nkv, d = k.shape
    if v.shape != k.shape or q.numel() != B * H * d or q.shape[:2] != (B, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    code = _dtype_code(q)
    odt = q.dtype
    if out_dtype is not None and out_dtype != q.dtype:
        if out_dtype != torch.float32:
            raise TypeError("out_dtype must be None, q.dtype or torch.float32")
        code |= FA_OUT_F32
        odt = torch.float32
    o = torch.empty(q.shape, dtype=odt, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_size(B, H, Nkv, d, num_splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        fa_decode(q, k, v, o, lse, B, H, Nkv, d, scale, code, num_splits, ws, nbytes, _stream(q.device))
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, *, layout="hnd", max_seq_len=None, scale=None,
                 num_splits=0, out_dtype=None):
    """Decode over a paged cache.

    q [B, H, d]; k_pages / v_pages [num_pages, H, page_size, d] for layout
    'hnd' or [num_pages, page_size, H, d] for 'nhd'; block_table
    [B, max_pages] and seq_lens [B] int32 on the device.  max_seq_len bounds
    seq_lens and sizes the key-range splits; it defaults to the table's
    capacity max_pages * page_size (a tighter bound splits the work better).
    Returns (o, lse): o [B, H, d], lse [B, H]."""
    import torch
    _check_inputs(q, k_pages, v_pages)
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H, d], got {tuple(q.shape)}")
    _check_rank(4, k_pages=k_pages, v_pages=v_pages)
    B, H, d = q.shape
    if layout == "hnd":
        num_pages, Hk, page_size, dk = k_pages.shape
        code_layout = FA_PAGED_HND
    elif layout == "nhd":
        num_pages, page_size, Hk, dk = k_pages.shape
        code_layout = FA_PAGED_NHD
    else:
        raise ValueError(f"layout must be 'hnd' or 'nhd', got {layout!r}")
    if (Hk, dk) != (H, d) or v_pages.shape != k_pages.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, pages {tuple(k_pages.shape)} / {tuple(v_pages.shape)}")
    for name, t, shape in (("block_table", block_table, (B, None)), ("seq_lens", seq_lens, (B,))):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device or t.dim() != len(shape) \
                or t.shape[0] != B:
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device with leading dimension B")
    max_pages = block_table.shape[1]
    if max_seq_len is None:
        max_seq_len = max_pages * page_size
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    code = _dtype_code(q)
    odt = q.dtype
    if out_dtype is not None and out_dtype != q.dtype:
        if out_dtype != torch.float32:
            raise TypeError("out_dtype must be None, q.dtype or torch.float32")
        code |= FA_OUT_F32
        odt = torch.float32
    o = torch.empty((B, H, d), dtype=odt, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_size(B, H, max_seq_len, d, num_splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        fa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, lse, B, H, d, num_pages, page_size,
                        max_pages, code_layout, max_seq_len, scale, code, num_splits, ws, nbytes, _stream(q.device))
    return o, lse


def bwd(q, k, v, o, dout, lse, *, causal=False, scale=None, out_dtype=None):
    """Gradients (dq, dk, dv) of fwd for dL/do = dout, from fwd's o (q's dtype) and lse.

    out_dtype may be torch.float32 to get the gradients in fp32, else they
    have q's dtype."""
    import torch
    _check_inputs(q, k, v)
    _check_rank(4, q=q, k=k, v=v)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, d) or v.shape != (B, H, Nkv, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    code = _dtype_code(q)
    gdt = q.dtype
    if out_dtype is not None and out_dtype != q.dtype:
        if out_dtype != torch.float32:
            raise TypeError("out_dtype must be None, q.dtype or torch.float32")
        code |= FA_OUT_F32
        gdt = torch.float32
    dq = torch.empty(q.shape, dtype=gdt, device=q.device)
    dk = torch.empty(k.shape, dtype=gdt, device=q.device)
    dv = torch.empty(v.shape, dtype=gdt, device=q.device)
    nbytes = fa_bwd_workspace_size(B, H, Nq)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nkv, d, causal, scale, code, ws, nbytes,
               _stream(q.device))
    return dq, dk, dv
