"""libfa355: exact, IO-aware fused softmax attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI declared in
include/fa355.h; this package is a thin ctypes binding over it.
"""
from ._binding import (  # noqa: F401
    FA_BF16,
    FA_ERR_HIP,
    FA_ERR_INVALID,
    FA_ERR_UNSUPPORTED,
    FA_ERR_WORKSPACE,
    FA_F16,
    FA_OK,
    FA_OUT_F32,
    FA_PAGED_HND,
    FA_PAGED_NHD,
    LIBRARY,
    FaError,
    bwd,
    decode,
    decode_paged,
    fa_bwd,
    fa_bwd_workspace_size,
    fa_decode,
    fa_decode_num_splits,
    fa_decode_paged,
    fa_decode_workspace_size,
    fa_fwd,
    fa_fwd_fp8,
    fa_last_error,
    fa_quantize_e4m3,
    fa_status_str,
    fa_version,
    fwd,
    fwd_fp8,
    library,
    quantize_e4m3,
)
