"""libfa355: fused tiled scaled-dot-product attention for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind a C ABI
(include/fa355.h, built into ``libfa355.so`` next to this file); this package
is the thin binding.  The library is loaded on first use, never silently
replaced: if it is missing, calls raise.
"""

from .fa355 import (  # noqa: F401
    FA_BF16,
    FA_CHECK_LENGTH,
    FA_CHECK_PAGE,
    FA_FP16,
    FA_FP32,
    BWD_TUNE_CANDIDATES,
    DECODE_TUNE_CANDIDATES,
    TUNE_CANDIDATES,
    TUNE_FIELDS,
    TUNE_KINDS,
    FaError,
    fa_bwd,
    fa_bwd_auto_dq_rows,
    fa_bwd_tune,
    fa_bwd_workspace_size,
    fa_bwd_workspace_size_ds,
    fa_bwd_default_workspace_size,
    BWD_DS_WORKSPACE_CAP,
    FA_BWD_DQ_STORED,
    fa_decode,
    fa_decode_auto_chunk,
    fa_decode_check,
    fa_decode_noalloc,
    fa_decode_tune,
    fa_decode_paged,
    fa_decode_workspace_size,
    fa_fwd,
    fa_fwd_ex,
    fa_fwd_tune,
    fa_fwd_auto_block_q,
    fa_fwd_auto_tile,
    fa_tune_export,
    fa_tune_import,
    fa_tune_reset,
    load_tuning,
    save_tuning,
    last_error,
    lib,
    status_str,
)
