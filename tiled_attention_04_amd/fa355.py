"""Thin Python binding of libfa355's C ABI (include/fa355.h).

Argument marshalling only: the functions check that tensors live on the GPU
with the expected dtype/layout, allocate outputs and workspaces with torch
(device memory is all torch is used for), and call the library on the
current torch stream.  Every step of the computation runs in the HIP kernels.
There is no fallback: if the library cannot be loaded, calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_FP32, FA_BF16, FA_FP16 = 0, 1, 2

_DTYPE = {torch.float32: FA_FP32, torch.bfloat16: FA_BF16, torch.float16: FA_FP16}

_lib = None

# (name, restype, argtypes) for every symbol declared in include/fa355.h.
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_version": (_I, []),
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _I, _I]),
    "fa_fwd_tune": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _I, _P, _P, _P]),
    "fa_fwd_auto_block_q": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "fa_tune_reset": (None, []),
    "fa_tune_export": (_I, [_P, _I]),
    "fa_tune_import": (_I, [_P, _I]),
    "fa_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _I, _P]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z,
                             _I, _P]),
    "fa_bwd_workspace_size": (_Z, [_I, _I, _I, _I]),
    "fa_bwd_workspace_size_ds": (_Z, [_I, _I, _I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _I, _P]),
    "fa_decode_tune": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _Z, _I, _P, _I, _P, _P]),
    "fa_decode_auto_chunk": (_I, [_I, _I, _I, _I, _I, _I, _P]),
    "fa_bwd_tune": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _I, _P,
                         _I, _P, _P]),
    "fa_bwd_auto_dq_rows": (_I, [_I, _I, _I, _I, _I, _I, _I, _Z, _P]),
    "fa_decode_check": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
}


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{status_str(status)}: {message}")


def lib() -> ctypes.CDLL:
    """The loaded library (torch's HIP runtime is loaded first, so both share it)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "or python -m tiled_attention_04_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().fa_status_str(status).decode()


def last_error() -> str:
    return lib().fa_last_error().decode()


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, last_error())


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _default_scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fa_fwd_ex(q, k, v, block_q: int = 0, block_k: int = 0, *, causal: bool = False,
              window: int = -1, scale=None, o=None, lse=None, stream=None):
    """Forward pass; q, k, v: [B, H, N, d] GPU tensors (bf16, fp16 or fp32).
    Returns (o [B,H,N,d] in the input dtype, lse [B,H,N] float32)."""
    B, H, N, d = q.shape
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(k, "k", dt, q.shape)
    vp = _dev(v, "v", dt, q.shape)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (B, H, N))
    _check(lib().fa_fwd_ex(qp, kp, vp, op, lp, B, H, N, d, _default_scale(scale, d), int(causal),
                           int(window), _DTYPE[dt], _stream(stream), int(block_q), int(block_k)))
    return o, lse


def fa_fwd(q, k, v, *, causal: bool = False, window: int = -1, scale=None, o=None, lse=None,
           stream=None):
    """Forward pass with the library's automatic tile choice."""
    return fa_fwd_ex(q, k, v, 0, 0, causal=causal, window=window, scale=scale, o=o, lse=lse,
                     stream=stream)


# (block_q, block_k) tiles fa_fwd_tune measures, in its order.
TUNE_CANDIDATES = ((32, 32), (32, 64), (32, 128), (64, 32), (64, 64), (64, 128), (128, 32), (128, 64),
                   (128, 128), (256, 64))


def fa_fwd_tune(q, k, v, *, causal: bool = False, window: int = -1, scale=None, reps: int = 10,
                o=None, lse=None, stream=None):
    """Time every tile (block_q, block_k) of the 16-bit forward on these inputs
    and remember the fastest for later automatic calls (synchronises the
    stream).  Returns (best (block_q, block_k), {tile: mean ms per call}, o, lse)."""
    B, H, N, d = q.shape
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(k, "k", dt, q.shape)
    vp = _dev(v, "v", dt, q.shape)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (B, H, N))
    best_q, best_k = ctypes.c_int(0), ctypes.c_int(0)
    times = (ctypes.c_float * len(TUNE_CANDIDATES))()
    _check(lib().fa_fwd_tune(qp, kp, vp, op, lp, B, H, N, d, _default_scale(scale, d), int(causal),
                             int(window), _DTYPE[dt], _stream(stream), int(reps), ctypes.byref(best_q),
                             ctypes.byref(best_k), times))
    return (best_q.value, best_k.value), dict(zip(TUNE_CANDIDATES, list(times))), o, lse


def fa_fwd_auto_tile(B: int, H: int, N: int, d: int, *, causal: bool = False, window: int = -1,
                     dtype=torch.bfloat16):
    """((block_q, block_k) an automatic fa_fwd call uses, whether it was tuned)."""
    tuned, bk = ctypes.c_int(0), ctypes.c_int(0)
    bq = lib().fa_fwd_auto_block_q(B, H, N, d, int(causal), int(window), _DTYPE[dtype], ctypes.byref(bk),
                                   ctypes.byref(tuned))
    return (int(bq), int(bk.value)), bool(tuned.value)


def fa_fwd_auto_block_q(B: int, H: int, N: int, d: int, *, causal: bool = False, window: int = -1,
                        dtype=torch.bfloat16):
    """(block_q an automatic fa_fwd call uses, whether it was tuned)."""
    (bq, _), tuned = fa_fwd_auto_tile(B, H, N, d, causal=causal, window=window, dtype=dtype)
    return bq, tuned


def fa_tune_reset() -> None:
    lib().fa_tune_reset()


# Columns of a remembered tuning choice; "kind" is one of TUNE_KINDS, "rows"
# is B*H (S*H for decode), "n" is N (Lmax for decode) and "value" the choice:
# block_q * 1000 + block_k, the decode split length or the dQ kernel's query
# rows.
TUNE_FIELDS = ("kind", "dtype", "d", "causal", "window", "rows", "n", "value")
TUNE_KINDS = {"fwd_tile": 0, "decode_chunk": 1, "bwd_dq_rows": 2}
_ROW = len(TUNE_FIELDS)


def fa_tune_export() -> list:
    """The remembered tuning choices as dicts with the keys of TUNE_FIELDS."""
    n = int(lib().fa_tune_export(None, 0))
    buf = (ctypes.c_int64 * (_ROW * max(n, 1)))()
    n = min(n, int(lib().fa_tune_export(buf, n)))
    return [dict(zip(TUNE_FIELDS, buf[_ROW * i:_ROW * i + _ROW])) for i in range(n)]


def fa_tune_import(entries) -> None:
    """Add tuning choices (dicts as returned by fa_tune_export)."""
    entries = list(entries)
    buf = (ctypes.c_int64 * (_ROW * max(len(entries), 1)))()
    for i, e in enumerate(entries):
        for j, f in enumerate(TUNE_FIELDS):
            buf[_ROW * i + j] = int(e[f])
    _check(lib().fa_tune_import(buf, len(entries)))


def save_tuning(path: str) -> None:
    """Write the remembered tuning choices to a JSON file."""
    import json
    with open(path, "w") as f:
        json.dump(fa_tune_export(), f, indent=1)


def load_tuning(path: str) -> None:
    """Load tuning choices written by save_tuning."""
    import json
    with open(path) as f:
        fa_tune_import(json.load(f))


def fa_decode_workspace_size(S: int, H: int, Lmax: int, d: int, chunk: int = 0) -> int:
    return int(lib().fa_decode_workspace_size(S, H, Lmax, d, chunk))


def fa_decode(q, kcache, vcache, seqlens, *, scale=None, window: int = -1, chunk: int = 0,
              o=None, lse=None, workspace=None, stream=None):
    """Single-token decode; q: [S,H,d], caches: [S,H,Lmax,d], seqlens: int32 [S] on the GPU.
    Returns (o [S,H,d], lse [S,H] float32)."""
    S, H, d = q.shape
    Lmax = kcache.shape[2]
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(kcache, "kcache", dt, (S, H, Lmax, d))
    vp = _dev(vcache, "vcache", dt, (S, H, Lmax, d))
    sp = _dev(seqlens, "seqlens", torch.int32, (S,))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = fa_decode_workspace_size(S, H, Lmax, d, chunk)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (S, H))
    wp = _dev(workspace, "workspace")
    _check(lib().fa_decode(qp, kp, vp, sp, op, lp, S, H, Lmax, d, _default_scale(scale, d),
                           int(window), int(chunk), wp, workspace.numel() * workspace.element_size(),
                           _DTYPE[dt], _stream(stream)))
    return o, lse


FA_CHECK_LENGTH, FA_CHECK_PAGE = 1, 2


def fa_decode_check(seqlens, block_table=None, *, Lmax: int = 0, page_size: int = 0, num_pages: int = 0,
                    window: int = -1, flags=None, stream=None):
    """Per-sequence flags of the arguments the decode calls repair on the device
    (0: none; FA_CHECK_LENGTH: length outside [1, capacity]; FA_CHECK_PAGE: an
    entry outside the pool among the pages the decode reads).  seqlens: int32
    [S]; block_table: int32 [S, max_pages], or None for a dense cache of length
    Lmax.  Returns flags, int32 [S] on the GPU, written asynchronously."""
    S = seqlens.shape[0]
    if flags is None:
        flags = torch.empty(S, dtype=torch.int32, device=seqlens.device)
    if S == 0:
        return flags
    sp = _dev(seqlens, "seqlens", torch.int32, (S,))
    if block_table is None:
        tp, max_pages = None, 0
    else:
        max_pages = block_table.shape[1]
        tp = _dev(block_table, "block_table", torch.int32, (S, max_pages))
    fp = _dev(flags, "flags", torch.int32, (S,))
    _check(lib().fa_decode_check(sp, tp, S, int(Lmax), int(page_size), int(max_pages), int(num_pages),
                                 int(window), fp, _stream(stream)))
    return flags


DECODE_TUNE_CANDIDATES = (256, 512, 1024, 2048, 4096)


def fa_decode_tune(q, kcache, vcache, seqlens, *, scale=None, window: int = -1, reps: int = 10,
                   o=None, lse=None, workspace=None, stream=None):
    """Time the decode's split lengths on these inputs and remember the fastest
    for later automatic calls (synchronises the stream).  Returns (best chunk,
    {chunk: mean ms per call, or -1 when skipped}, o, lse)."""
    S, H, d = q.shape
    Lmax = kcache.shape[2]
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(kcache, "kcache", dt, (S, H, Lmax, d))
    vp = _dev(vcache, "vcache", dt, (S, H, Lmax, d))
    sp = _dev(seqlens, "seqlens", torch.int32, (S,))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = fa_decode_workspace_size(S, H, Lmax, d, 0)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (S, H))
    wp = _dev(workspace, "workspace")
    best = ctypes.c_int(0)
    times = (ctypes.c_float * len(DECODE_TUNE_CANDIDATES))()
    _check(lib().fa_decode_tune(qp, kp, vp, sp, op, lp, S, H, Lmax, d, _default_scale(scale, d),
                                int(window), wp, workspace.numel() * workspace.element_size(), _DTYPE[dt],
                                _stream(stream), int(reps), ctypes.byref(best), times))
    return best.value, dict(zip(DECODE_TUNE_CANDIDATES, list(times))), o, lse


def fa_decode_auto_chunk(S: int, H: int, Lmax: int, d: int, *, window: int = -1, dtype=torch.bfloat16):
    """(split length an automatic decode call uses, whether it was tuned)."""
    tuned = ctypes.c_int(0)
    c = lib().fa_decode_auto_chunk(S, H, Lmax, d, int(window), _DTYPE[dtype], ctypes.byref(tuned))
    return int(c), bool(tuned.value)


def fa_decode_noalloc(q, kcache, vcache, seqlens, *, scale=None, window: int = -1, chunk: int = 0,
                      o=None, lse=None, stream=None):
    """fa_decode without a workspace: the library keeps the split partials in
    a static 32 MiB device array (calls that overlap on one device race).
    Allocates only the outputs when o / lse are not given."""
    S, H, d = q.shape
    Lmax = kcache.shape[2]
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(kcache, "kcache", dt, (S, H, Lmax, d))
    vp = _dev(vcache, "vcache", dt, (S, H, Lmax, d))
    sp = _dev(seqlens, "seqlens", torch.int32, (S,))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (S, H))
    _check(lib().fa_decode_noalloc(qp, kp, vp, sp, op, lp, S, H, Lmax, d, _default_scale(scale, d),
                                   int(window), int(chunk), _DTYPE[dt], _stream(stream)))
    return o, lse


def fa_decode_paged(q, k_pages, v_pages, block_table, seqlens, *, scale=None, window: int = -1,
                    chunk: int = 0, o=None, lse=None, workspace=None, stream=None):
    """Single-token decode over a paged cache.  q: [S,H,d]; k_pages, v_pages:
    [num_pages,H,page_size,d]; block_table: int32 [S,max_pages] and seqlens: int32
    [S], both on the GPU.  Returns (o [S,H,d], lse [S,H] float32)."""
    S, H, d = q.shape
    num_pages, _, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    qp = _dev(q, "q", dt)
    kp = _dev(k_pages, "k_pages", dt, (num_pages, H, page_size, d))
    vp = _dev(v_pages, "v_pages", dt, (num_pages, H, page_size, d))
    tp = _dev(block_table, "block_table", torch.int32, (S, max_pages))
    sp = _dev(seqlens, "seqlens", torch.int32, (S,))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = fa_decode_workspace_size(S, H, max_pages * page_size, d, chunk)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    op = _dev(o, "o", dt, q.shape)
    lp = _dev(lse, "lse", torch.float32, (S, H))
    wp = _dev(workspace, "workspace")
    _check(lib().fa_decode_paged(qp, kp, vp, tp, sp, op, lp, S, H, d, num_pages, page_size, max_pages,
                                 _default_scale(scale, d), int(window), int(chunk), wp,
                                 workspace.numel() * workspace.element_size(), _DTYPE[dt],
                                 _stream(stream)))
    return o, lse


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, N, d))


def fa_bwd_workspace_size_ds(B: int, H: int, N: int, d: int, causal: bool = False, window: int = -1) -> int:
    return int(lib().fa_bwd_workspace_size_ds(B, H, N, d, int(causal), int(window)))


# The binding gives fa_bwd the stored-dS workspace by default when the
# product kernel's grid (128 query rows per workgroup) fills the chip at two
# workgroups per CU and the workspace stays within this many bytes (the dS
# blocks grow as N^2); else the minimum.  (Measured: the stored-dS path
# leads at 2x16x4096x128, causal or windowed, and trails the recompute
# kernels at 1x8x1024x64, whose 64 workgroups leave most CUs idle.)
BWD_DS_WORKSPACE_CAP = 8 << 30
BWD_DS_MIN_WORKGROUPS = 512
FA_BWD_DQ_STORED = 1


def fa_bwd_default_workspace_size(B: int, H: int, N: int, d: int, causal: bool = False, window: int = -1,
                                  dtype=torch.bfloat16, stored_ds=None) -> int:
    """Workspace bytes the binding allocates for an fa_bwd call: with the
    stored dS (16-bit types, d in {64, 128}) when stored_ds is True, or when
    it is None, the grid of B * H * ceil(N / 128) workgroups reaches
    BWD_DS_MIN_WORKGROUPS and that size is at most BWD_DS_WORKSPACE_CAP;
    else the minimum (dQ by recomputation)."""
    small = fa_bwd_workspace_size(B, H, N, d)
    if stored_ds is False or dtype == torch.float32:
        return small
    big = fa_bwd_workspace_size_ds(B, H, N, d, causal, window)
    if stored_ds and big == 0:
        raise ValueError("the stored-dS backward takes 16-bit inputs with d in {64, 128}")
    fills = B * H * ((N + 127) // 128) >= BWD_DS_MIN_WORKGROUPS
    return big if big and (stored_ds or (fills and big <= BWD_DS_WORKSPACE_CAP)) else small


def fa_bwd(q, k, v, o, dO, lse, *, causal: bool = False, window: int = -1, scale=None,
           dq=None, dk=None, dv=None, workspace=None, stream=None, stored_ds=None):
    """Backward pass from the forward's o and lse.  Returns float32 (dq, dk, dv).

    Without a workspace the binding allocates fa_bwd_default_workspace_size
    bytes (stored_ds: None = dS stored while its workspace stays within
    BWD_DS_WORKSPACE_CAP, True = stored, False = recomputed)."""
    B, H, N, d = q.shape
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    ptrs = [_dev(t, n, dt, q.shape) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"))]
    lp = _dev(lse, "lse", torch.float32, (B, H, N))
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty(q.shape, dtype=torch.float32, device=q.device) if t is None else t)
    gp = [_dev(t, n, torch.float32, q.shape) for t, n in zip(outs, ("dq", "dk", "dv"))]
    if workspace is None:
        need = fa_bwd_default_workspace_size(B, H, N, d, causal, window, dt, stored_ds)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace")
    _check(lib().fa_bwd(*ptrs, lp, *gp, B, H, N, d, _default_scale(scale, d), int(causal),
                        int(window), wp, workspace.numel() * workspace.element_size(), _DTYPE[dt],
                        _stream(stream)))
    return tuple(outs)


BWD_TUNE_CANDIDATES = (128, 256, FA_BWD_DQ_STORED)


def fa_bwd_tune(q, k, v, o, dO, lse, *, causal: bool = False, window: int = -1, scale=None, reps: int = 10,
                dq=None, dk=None, dv=None, workspace=None, stream=None, stored_ds=None):
    """Time the backward with each way of forming dQ (the recompute kernel with
    128 or 256 query rows per workgroup, and FA_BWD_DQ_STORED when the
    workspace holds the stored dS) and remember the fastest for later fa_bwd
    calls (synchronises the stream).  Returns (best, {candidate: mean ms per
    call, -1 if not tried}, (dq, dk, dv))."""
    B, H, N, d = q.shape
    dt = q.dtype
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}")
    ptrs = [_dev(t, n, dt, q.shape) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"))]
    lp = _dev(lse, "lse", torch.float32, (B, H, N))
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty(q.shape, dtype=torch.float32, device=q.device) if t is None else t)
    gp = [_dev(t, n, torch.float32, q.shape) for t, n in zip(outs, ("dq", "dk", "dv"))]
    if workspace is None:
        need = fa_bwd_default_workspace_size(B, H, N, d, causal, window, dt, stored_ds)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace")
    best = ctypes.c_int(0)
    times = (ctypes.c_float * len(BWD_TUNE_CANDIDATES))()
    _check(lib().fa_bwd_tune(*ptrs, lp, *gp, B, H, N, d, _default_scale(scale, d), int(causal),
                             int(window), wp, workspace.numel() * workspace.element_size(), _DTYPE[dt],
                             _stream(stream), int(reps), ctypes.byref(best), times))
    return best.value, dict(zip(BWD_TUNE_CANDIDATES, list(times))), tuple(outs)


def fa_bwd_auto_dq_rows(B: int, H: int, N: int, d: int, *, causal: bool = False, window: int = -1,
                        dtype=torch.bfloat16, workspace_bytes=None):
    """(How an fa_bwd call with workspace_bytes of workspace forms dQ -- 128 or
    256 recompute rows, or FA_BWD_DQ_STORED --, whether that was tuned).
    workspace_bytes defaults to what the binding's fa_bwd allocates."""
    if workspace_bytes is None:
        workspace_bytes = (fa_bwd_default_workspace_size(B, H, N, d, causal, window, dtype)
                           if B > 0 and H > 0 and N > 0 and d > 0 else 0)
    tuned = ctypes.c_int(0)
    r = lib().fa_bwd_auto_dq_rows(B, H, N, d, int(causal), int(window), _DTYPE[dtype], int(workspace_bytes),
                                  ctypes.byref(tuned))
    return int(r), bool(tuned.value)
