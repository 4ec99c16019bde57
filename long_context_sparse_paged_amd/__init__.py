"""Python binding of libdsa (gfx950 HIP kernels for the DSA step), via ctypes.

Argument marshalling only: each ``dsa_*`` function below checks tensor
devices/dtypes, passes raw pointers and sizes to the C entry point of the same
name (``include/dsa.h``), and raises ``DsaError`` on a non-zero status.  All
computation runs in the library's kernels.  There is no fallback: if the
library is not built, importing this package raises.

Tensors are torch tensors on the GPU; the stream defaults to torch's current
stream.  bf16 tensors are passed as their bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
from pathlib import Path

import torch

from .build import LIB as _BUILT_LIB

# DSA_LIB selects another build of the same library (e.g. a host-sanitizer build for CPU-only
# checks of argument validation); by default the in-tree build is loaded.
_LIB_PATH = Path(os.environ.get("DSA_LIB", str(_BUILT_LIB)))

DSA_OK, DSA_ERR_NULL_ARG, DSA_ERR_BAD_SHAPE, DSA_ERR_MISALIGNED = 0, 1, 2, 3
DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP, DSA_ERR_SCRATCH_LIMIT = 4, 5, 6, 7
DSA_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
DSA_DEVERR_BLOCK_RANGE, DSA_DEVERR_PAGE_COUNT, DSA_DEVERR_PAGE_OFFSET = 1, 2, 4
DSA_DEVERR_ROW_LEN, DSA_DEVERR_INDEX, DSA_DEVERR_REQUEST = 8, 16, 32
DSA_DEVERR_BOUND = 64
DSA_KEY_FP8_E4M3_SCALED, DSA_KEY_MXFP4 = 0, 1
DSA_LAT_FP8_E4M3, DSA_LAT_NVFP4 = 0, 1
DSA_Q_BF16, DSA_Q_FP8_E4M3, DSA_Q_MXFP4 = 0, 1, 2

__all__ = [
    "DsaError", "dsa_layout", "lib", "dsa_status_str", "dsa_version", "dsa_layout_make", "dsa_resolve_pages",
    "dsa_indexer_score_workspace_size", "dsa_indexer_score", "dsa_indexer_score_verify", "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_mla_decode_workspace_size",
    "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill_workspace_size", "dsa_sparse_mla_prefill",
    "dsa_dcp_topk_workspace_size", "dsa_dcp_topk", "dsa_sparse_mla_decode_noalloc",
    "dsa_indexer_select_workspace_size", "dsa_indexer_select", "dsa_sparse_mla_decode_phys",
    "dsa_indexer_score_pages", "dsa_topk_pages", "dsa_prefill_select_workspace_size", "dsa_prefill_select",
    "dsa_prefill_score_fp8", "dsa_prefill_topk_band", "dsa_prefill_prepare_fp8", "dsa_prefill_gemm_fp8",
]


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({dsa_status_str(status)})")
        self.status = status


class dsa_layout(C.Structure):
    _fields_ = [("page_size", C.c_int32), ("n_layers", C.c_int32), ("key_fmt", C.c_int32), ("lat_fmt", C.c_int32),
                ("key_bytes", C.c_int32), ("lat_bytes", C.c_int32), ("lat_page_bytes", C.c_int64),
                ("key_page_bytes", C.c_int64), ("layer_stride", C.c_int64), ("extra_row_bytes", C.c_int64),
                ("row_stride", C.c_int64)]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


def _load():
    if not _LIB_PATH.exists():
        raise ImportError(f"{_LIB_PATH} is not built; run `python long_context_sparse_paged_amd/build.py` "
                          "(the DSA kernels have no CPU fallback)")
    L = C.CDLL(str(_LIB_PATH))
    P, I32, I64, SZ, F = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    LP = C.POINTER(dsa_layout)
    sig = {
        "dsa_status_str": ([I32], C.c_char_p),
        "dsa_version": ([], C.c_char_p),
        "dsa_layout_make": ([I32, I32, I32, I32, I64, LP], I32),
        "dsa_resolve_pages": ([LP, I32, P, I64, P, I32, I32, I64, P, P, I64, P, P], I32),
        "dsa_indexer_score_workspace_size": ([I32, I32, C.POINTER(SZ)], I32),
        "dsa_indexer_score": ([LP, P, I64, P, I64, I32, P, I32, P, P, P, P, I32, P, I64, P, SZ, P, P], I32),
        "dsa_indexer_score_verify": ([LP, P, I64, P, I64, I32, I32, P, P, P, P, I64, P, P], I32),
        "dsa_topk_workspace_size": ([I32, I64, I32, C.POINTER(SZ)], I32),
        "dsa_topk": ([P, I64, P, I32, I32, P, I64, P, SZ, P, P], I32),
        "dsa_sparse_mla_decode_workspace_size": ([I32, I32, I32, C.POINTER(SZ)], I32),
        "dsa_sparse_mla_decode": ([LP, P, I64, P, I64, P, P, I64, I32, P, I32, I32, F, F, P, P, P, SZ, P, P], I32),
        "dsa_sparse_mla_decode_noalloc": ([LP, P, I64, P, I64, P, P, I64, I32, P, I32, I32, F, F, P, P, P, P], I32),
        "dsa_indexer_select_workspace_size": ([I32, I64, C.POINTER(SZ)], I32),
        "dsa_indexer_select": ([LP, I32, P, I64, P, I64, I32, P, I32, P, P, P, I32, I32, P, I64, P, P, I64, P, SZ, P, P],
                               I32),
        "dsa_sparse_mla_decode_phys": ([LP, I32, P, I64, P, I64, I32, P, I32, I32, F, F, P, P, P, SZ, P, P], I32),
        "dsa_indexer_score_pages": ([LP, I32, P, I64, P, I64, I32, P, I32, P, P, P, I32, P, I64, P, P], I32),
        "dsa_topk_pages": ([LP, I64, P, I64, I32, P, P, I64, P, I32, I32, P, SZ, P, P, I64, P, P], I32),
        "dsa_prefill_select_workspace_size": ([I32, I64, I32, I64, I32, C.POINTER(SZ)], I32),
        "dsa_prefill_select": ([LP, P, I64, P, I64, I32, P, P, P, P, P, P, I32, I32, P, I64, P, I64, P, P, SZ, P, P],
                               I32),
        "dsa_prefill_score_fp8": ([LP, P, I64, P, I64, I32, P, P, P, P, P, P, I32, I32, P, I64, P, P, SZ, P, P], I32),
        "dsa_prefill_prepare_fp8": ([LP, P, I64, P, I64, I32, P, P, P, P, P, P, I32, I32, P, I64, P, P, SZ, P, P], I32),
        "dsa_prefill_gemm_fp8": ([LP, P, I64, P, I64, I32, P, P, P, P, P, P, I32, I32, P, I64, P, P, SZ, P, P], I32),
        "dsa_prefill_topk_band": ([LP, P, I64, P, I64, I32, P, P, I32, I32, P, I64, P, I64, P, SZ, P, P], I32),
        "dsa_sparse_mla_prefill_workspace_size": ([I32, I32, I32, C.POINTER(SZ)], I32),
        "dsa_dcp_topk_workspace_size": ([I32, I32, I32, C.POINTER(SZ)], I32),
        "dsa_dcp_topk": ([P, I64, P, I32, I32, I32, P, I64, P, P, SZ, P, P], I32),
        "dsa_sparse_mla_prefill": ([LP, P, I64, P, I64, I32, P, P, I64, I32, P, I32, P, P, I32, I32, F, F, P, P, P,
                                    SZ, P, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def dsa_status_str(s: int) -> str:
    return lib.dsa_status_str(s).decode()


def dsa_version() -> str:
    return lib.dsa_version().decode()


def _check(fn: str, st: int):
    if st != DSA_OK:
        raise DsaError(fn, st)


def _ptr(t, dtypes=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a GPU tensor (no CPU path exists)")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise TypeError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


I32, I64, U8, F32 = (torch.int32,), (torch.int64,), (torch.uint8,), (torch.float32,)
BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_Q_DTYPE = {DSA_Q_BF16: BF16, DSA_Q_FP8_E4M3: U8, DSA_Q_MXFP4: U8}


def dsa_layout_make(page_size: int, n_layers: int, key_fmt: int, lat_fmt: int, extra_row_bytes: int = 0) -> dsa_layout:
    out = dsa_layout()
    _check("dsa_layout_make", lib.dsa_layout_make(page_size, n_layers, key_fmt, lat_fmt, extra_row_bytes, C.byref(out)))
    return out


def dsa_resolve_pages(layout: dsa_layout, layer: int, block_table, n_pages, pool_rows: int, lat_off, key_off,
                      err_flag=None, stream=None):
    n_req, max_pages = block_table.shape
    # the row stride is the leading dimension (a one-row table may carry any stride there)
    bt_ld = block_table.stride(0) if n_req > 1 else max_pages
    st = lib.dsa_resolve_pages(C.byref(layout), layer, _ptr(block_table, I32, "block_table"), bt_ld,
                               _ptr(n_pages, I32, "n_pages"), n_req, max_pages, pool_rows,
                               _ptr(lat_off, I64, "lat_off"), _ptr(key_off, I64, "key_off"), lat_off.shape[1],
                               _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_resolve_pages", st)


def dsa_indexer_score_workspace_size(n_q: int, q_fmt: int) -> int:
    out = C.c_size_t()
    _check("dsa_indexer_score_workspace_size", lib.dsa_indexer_score_workspace_size(n_q, q_fmt, C.byref(out)))
    return out.value


def dsa_indexer_score(layout: dsa_layout, pool, key_off, n_req: int, q, q_fmt: int, q_scale, w, q_req, row_len,
                      scores, workspace=None, err_flag=None, stream=None):
    qd = BF16 if q_fmt == DSA_Q_BF16 else U8
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.dsa_indexer_score(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(), _ptr(key_off, I64, "key_off"),
                               key_off.shape[1], n_req, _ptr(q, qd, "q"), q_fmt, _ptr(q_scale, F32, "q_scale"),
                               _ptr(w, F32, "w"), _ptr(q_req, I32, "q_req"), _ptr(row_len, I32, "row_len"),
                               row_len.shape[0], _ptr(scores, F32, "scores"), scores.shape[1],
                               _ptr(workspace, None, "workspace"), ws_bytes, _ptr(err_flag, I32, "err_flag"),
                               _stream(stream))
    _check("dsa_indexer_score", st)


def dsa_indexer_score_verify(layout: dsa_layout, pool, key_off, n_req: int, rows_per_req: int, q, w, row_len,
                             scores, err_flag=None, stream=None):
    """Rows r = b*rows_per_req + i belong to request b; each key page is read once per request."""
    st = lib.dsa_indexer_score_verify(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(),
                                      _ptr(key_off, I64, "key_off"), key_off.shape[1], n_req, rows_per_req,
                                      _ptr(q, BF16, "q"), _ptr(w, F32, "w"), _ptr(row_len, I32, "row_len"),
                                      _ptr(scores, F32, "scores"), scores.shape[1], _ptr(err_flag, I32, "err_flag"),
                                      _stream(stream))
    _check("dsa_indexer_score_verify", st)


def dsa_topk_workspace_size(n_rows: int, ld: int, k: int) -> int:
    out = C.c_size_t()
    _check("dsa_topk_workspace_size", lib.dsa_topk_workspace_size(n_rows, ld, k, C.byref(out)))
    return out.value


def dsa_topk(scores, row_len, k: int, idx, workspace, err_flag=None, stream=None):
    st = lib.dsa_topk(_ptr(scores, F32, "scores"), scores.shape[1], _ptr(row_len, I32, "row_len"), scores.shape[0], k,
                      _ptr(idx, I32, "idx"), idx.shape[1], _ptr(workspace, None, "workspace"),
                      workspace.numel() * workspace.element_size(), _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_topk", st)


def dsa_indexer_select_workspace_size(n_q: int, ld: int) -> int:
    out = C.c_size_t()
    _check("dsa_indexer_select_workspace_size", lib.dsa_indexer_select_workspace_size(n_q, ld, C.byref(out)))
    return out.value


def dsa_indexer_select(layout: dsa_layout, layer: int, pool, block_table, n_req: int, q, w, q_req, row_len, k: int,
                       scores, idx, phys, workspace, err_flag=None, stream=None, q_fmt: int = DSA_Q_BF16):
    """Fused decode indexer: scores, the exact top-k (ascending) and their physical rows."""
    n_q = q.shape[0]
    st = lib.dsa_indexer_select(C.byref(layout), layer, _ptr(pool, U8, "pool"), pool.numel(),
                                _ptr(block_table, I32, "block_table"), block_table.shape[1], n_req,
                                _ptr(q, _Q_DTYPE[q_fmt], "q"), q_fmt, _ptr(w, F32, "w"), _ptr(q_req, I32, "q_req"),
                                _ptr(row_len, I32, "row_len"), n_q, k, _ptr(scores, F32, "scores"), scores.shape[1],
                                _ptr(idx, I32, "idx"), _ptr(phys, I32, "phys"), idx.shape[1],
                                _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_indexer_select", st)


def dsa_prefill_select_workspace_size(n_q: int, ld: int, n_req: int, off_ld: int, k: int) -> int:
    out = C.c_size_t()
    _check("dsa_prefill_select_workspace_size",
           lib.dsa_prefill_select_workspace_size(n_q, ld, n_req, off_ld, k, C.byref(out)))
    return out.value


def dsa_prefill_select(layout: dsa_layout, pool, key_off, n_req: int, ctx_len, q, q_scale, w, q_req, row_len, k: int,
                       scores, idx, workspace, bound=None, err_flag=None, stream=None):
    """Prefill indexer on FP8 MFMA with its exact top-k: idx as dsa_topk on dsa_indexer_score's
    FP8 scores; scores hold the FP8 MFMA approximations, each within bound[r] of those."""
    st = lib.dsa_prefill_select(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(), _ptr(key_off, I64, "key_off"),
                                key_off.shape[1], n_req, _ptr(ctx_len, I32, "ctx_len"), _ptr(q, U8, "q"),
                                _ptr(q_scale, F32, "q_scale"), _ptr(w, F32, "w"), _ptr(q_req, I32, "q_req"),
                                _ptr(row_len, I32, "row_len"), row_len.shape[0], k, _ptr(scores, F32, "scores"),
                                scores.shape[1], _ptr(idx, I32, "idx"), idx.shape[1], _ptr(bound, F32, "bound"),
                                _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_prefill_select", st)


def _prefill_score_call(name: str, layout: dsa_layout, pool, key_off, n_req: int, ctx_len, q, q_scale, w, q_req,
                        row_len, k: int, scores, workspace, bound=None, err_flag=None, stream=None):
    st = getattr(lib, name)(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(), _ptr(key_off, I64, "key_off"),
                            key_off.shape[1], n_req, _ptr(ctx_len, I32, "ctx_len"), _ptr(q, U8, "q"),
                            _ptr(q_scale, F32, "q_scale"), _ptr(w, F32, "w"), _ptr(q_req, I32, "q_req"),
                            _ptr(row_len, I32, "row_len"), row_len.shape[0], k, _ptr(scores, F32, "scores"),
                            scores.shape[1], _ptr(bound, F32, "bound"), _ptr(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size(), _ptr(err_flag, I32, "err_flag"),
                            _stream(stream))
    _check(name, st)


def dsa_prefill_score_fp8(*args, **kw):
    """First half of dsa_prefill_select: FP8 MFMA scores (within bound[r] of the exact ones).
    Arguments: layout, pool, key_off, n_req, ctx_len, q, q_scale, w, q_req, row_len, k, scores,
    workspace, bound=None, err_flag=None, stream=None."""
    _prefill_score_call("dsa_prefill_score_fp8", *args, **kw)


def dsa_prefill_prepare_fp8(*args, **kw):
    """dsa_prefill_score_fp8's first part: pre-pass, key bound, sampled tiles and thresholds."""
    _prefill_score_call("dsa_prefill_prepare_fp8", *args, **kw)


def dsa_prefill_gemm_fp8(*args, **kw):
    """dsa_prefill_score_fp8's second part: the full FP8 GEMM (and its candidate lists)."""
    _prefill_score_call("dsa_prefill_gemm_fp8", *args, **kw)


def dsa_prefill_topk_band(layout: dsa_layout, pool, key_off, n_req: int, q_req, row_len, k: int, scores, idx,
                          workspace, err_flag=None, stream=None):
    """Second half of dsa_prefill_select: the exact top-k from the FP8 scores (same workspace)."""
    st = lib.dsa_prefill_topk_band(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(),
                                   _ptr(key_off, I64, "key_off"), key_off.shape[1], n_req,
                                   _ptr(q_req, I32, "q_req"), _ptr(row_len, I32, "row_len"), row_len.shape[0], k,
                                   _ptr(scores, F32, "scores"), scores.shape[1], _ptr(idx, I32, "idx"), idx.shape[1],
                                   _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                   _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_prefill_topk_band", st)


def dsa_indexer_score_pages(layout: dsa_layout, layer: int, pool, block_table, n_req: int, q, w, q_req, row_len,
                            scores, err_flag=None, stream=None, q_fmt: int = DSA_Q_BF16):
    """First half of dsa_indexer_select: the scan, pages read through the block table."""
    st = lib.dsa_indexer_score_pages(C.byref(layout), layer, _ptr(pool, U8, "pool"), pool.numel(),
                                     _ptr(block_table, I32, "block_table"), block_table.shape[1], n_req,
                                     _ptr(q, _Q_DTYPE[q_fmt], "q"), q_fmt, _ptr(w, F32, "w"),
                                     _ptr(q_req, I32, "q_req"),
                                     _ptr(row_len, I32, "row_len"), q.shape[0], _ptr(scores, F32, "scores"),
                                     scores.shape[1], _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_indexer_score_pages", st)


def dsa_topk_pages(layout: dsa_layout, pool, block_table, n_req: int, q_req, scores, row_len, k: int, workspace, idx,
                   phys=None, err_flag=None, stream=None):
    """Second half of dsa_indexer_select: dsa_topk plus each kept token's physical row."""
    st = lib.dsa_topk_pages(C.byref(layout), pool.numel(), _ptr(block_table, I32, "block_table"), block_table.shape[1],
                            n_req, _ptr(q_req, I32, "q_req"), _ptr(scores, F32, "scores"), scores.shape[1],
                            _ptr(row_len, I32, "row_len"), scores.shape[0], k, _ptr(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size(), _ptr(idx, I32, "idx"),
                            _ptr(phys, I32, "phys"), idx.shape[1], _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_topk_pages", st)


def dsa_sparse_mla_decode_phys(layout: dsa_layout, layer: int, pool, phys, k: int, q, sm_scale: float,
                               kv_scale: float, out, lse, workspace=None, err_flag=None, stream=None):
    n_req, n_heads = q.shape[0], q.shape[1]
    wp, wb = _ws(workspace)
    st = lib.dsa_sparse_mla_decode_phys(C.byref(layout), layer, _ptr(pool, U8, "pool"), pool.numel(),
                                        _ptr(phys, I32, "phys"), phys.shape[1], k, _ptr(q, BF16, "q"), n_req, n_heads,
                                        float(sm_scale), float(kv_scale), _ptr(out, BF16, "out"),
                                        _ptr(lse, F32, "lse"), wp, wb, _ptr(err_flag, I32, "err_flag"),
                                        _stream(stream))
    _check("dsa_sparse_mla_decode_phys", st)


def dsa_sparse_mla_decode_workspace_size(n_req: int, n_heads: int, k: int) -> int:
    out = C.c_size_t()
    _check("dsa_sparse_mla_decode_workspace_size",
           lib.dsa_sparse_mla_decode_workspace_size(n_req, n_heads, k, C.byref(out)))
    return out.value


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()


def dsa_sparse_mla_decode(layout: dsa_layout, pool, lat_off, ctx_len, idx, k: int, q, sm_scale: float,
                          kv_scale: float, out, lse, workspace=None, err_flag=None, stream=None):
    n_req, n_heads = q.shape[0], q.shape[1]
    wp, wb = _ws(workspace)
    st = lib.dsa_sparse_mla_decode(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(),
                                   _ptr(lat_off, I64, "lat_off"), lat_off.shape[1], _ptr(ctx_len, I32, "ctx_len"),
                                   _ptr(idx, I32, "idx"), idx.shape[1], k, _ptr(q, BF16, "q"), n_req, n_heads,
                                   float(sm_scale), float(kv_scale), _ptr(out, BF16, "out"), _ptr(lse, F32, "lse"),
                                   wp, wb, _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_sparse_mla_decode", st)


def dsa_sparse_mla_decode_noalloc(layout: dsa_layout, pool, lat_off, ctx_len, idx, k: int, q, sm_scale: float,
                                  kv_scale: float, out, lse, err_flag=None, stream=None):
    """dsa_sparse_mla_decode without a workspace: the library's static per-GPU scratch holds
    the split partials (calls that overlap on one GPU race)."""
    n_req, n_heads = q.shape[0], q.shape[1]
    st = lib.dsa_sparse_mla_decode_noalloc(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(),
                                           _ptr(lat_off, I64, "lat_off"), lat_off.shape[1],
                                           _ptr(ctx_len, I32, "ctx_len"), _ptr(idx, I32, "idx"), idx.shape[1], k,
                                           _ptr(q, BF16, "q"), n_req, n_heads, float(sm_scale), float(kv_scale),
                                           _ptr(out, BF16, "out"), _ptr(lse, F32, "lse"),
                                           _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_sparse_mla_decode_noalloc", st)


def dsa_sparse_mla_prefill_workspace_size(n_q: int, n_heads: int, k: int) -> int:
    out = C.c_size_t()
    _check("dsa_sparse_mla_prefill_workspace_size",
           lib.dsa_sparse_mla_prefill_workspace_size(n_q, n_heads, k, C.byref(out)))
    return out.value


def dsa_sparse_mla_prefill(layout: dsa_layout, pool, lat_off, n_req: int, ctx_len, idx, k: int, q, q_fmt: int,
                           q_scale, q_req, sm_scale: float, kv_scale: float, out, lse, workspace=None,
                           err_flag=None, stream=None):
    n_q, n_heads = q.shape[0], q.shape[1]
    qd = BF16 if q_fmt == DSA_Q_BF16 else U8
    wp, wb = _ws(workspace)
    st = lib.dsa_sparse_mla_prefill(C.byref(layout), _ptr(pool, U8, "pool"), pool.numel(),
                                    _ptr(lat_off, I64, "lat_off"), lat_off.shape[1], n_req,
                                    _ptr(ctx_len, I32, "ctx_len"), _ptr(idx, I32, "idx"), idx.shape[1], k,
                                    _ptr(q, qd, "q"), q_fmt, _ptr(q_scale, F32, "q_scale"), _ptr(q_req, I32, "q_req"),
                                    n_q, n_heads, float(sm_scale), float(kv_scale), _ptr(out, BF16, "out"),
                                    _ptr(lse, F32, "lse"), wp, wb, _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_sparse_mla_prefill", st)


def dsa_dcp_topk_workspace_size(n_rows: int, k: int, n_shards: int) -> int:
    out = C.c_size_t()
    _check("dsa_dcp_topk_workspace_size", lib.dsa_dcp_topk_workspace_size(n_rows, k, n_shards, C.byref(out)))
    return out.value


def dsa_dcp_topk(scores, row_len, k: int, n_shards: int, idx, workspace, resend_mask=None, err_flag=None,
                 stream=None):
    st = lib.dsa_dcp_topk(_ptr(scores, F32, "scores"), scores.shape[1], _ptr(row_len, I32, "row_len"),
                          scores.shape[0], k, n_shards, _ptr(idx, I32, "idx"), idx.shape[1],
                          _ptr(resend_mask, (torch.int32, torch.uint32), "resend_mask"),
                          _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                          _ptr(err_flag, I32, "err_flag"), _stream(stream))
    _check("dsa_dcp_topk", st)


from .step import DecodeStep, FusedDecodeStep, PrefillSelectStep, PrefillStep, VerifyStep  # noqa: E402,F401
