"""CPU oracle for the DSA step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``long_context_sparse_paged_amd``) never imports, links or
calls it, and the two share no code.

A thin ctypes wrapper over ``dsa_oracle.c`` (plain C, double precision,
built with ``-O2 -ffp-contract=off``).  Arrays are numpy, host memory.
See ``dsa_oracle.c`` for the definitions each function follows and the
pages they are taken from.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, special cases, brute force,
independent library routines, hand-computed golden values).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "dsa_oracle.c"
# DSA_ORACLE_LIB selects another build of the oracle (e.g. a sanitizer build)
_LIB_PATH = Path(os.environ.get("DSA_ORACLE_LIB", str(_HERE / "_build" / "libdsa_oracle.so")))

OK, ERR_ARG, ERR_RANGE, ERR_NONFINITE = 0, 1, 2, 3


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (plain C, OpenMP over independent rows)."""
    if force or not _LIB_PATH.exists():
        _LIB_PATH.parent.mkdir(parents=True, exist_ok=True)
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class OrLayout(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("page_size", "n_layers", "key_fmt", "lat_fmt", "key_bytes",
                                          "lat_bytes", "layer_stride", "row_stride", "extra_row_bytes")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        L = C.CDLL(str(_LIB_PATH))
        P, I64, D = C.c_void_p, C.c_int64, C.c_double
        L.or_e4m3.restype = D
        L.or_e4m3.argtypes = [C.c_uint]
        L.or_e2m1.restype = D
        L.or_e2m1.argtypes = [C.c_uint]
        L.or_e8m0.restype = D
        L.or_e8m0.argtypes = [C.c_uint]
        L.or_bf16.restype = D
        L.or_bf16.argtypes = [C.c_uint16]
        L.or_layout_make.argtypes = [I64, I64, I64, I64, I64, C.POINTER(OrLayout)]
        L.or_resolve_pages.argtypes = [C.POINTER(OrLayout), I64, P, I64, P, I64, I64, I64, P, P, I64]
        L.or_key_decode.argtypes = [I64, P, P, P]
        L.or_latent_decode.argtypes = [I64, P, D, P]
        L.or_indexer_score.argtypes = [C.POINTER(OrLayout), I64, P, I64, P, I64, P, I64, P, I64, P, P, P,
                                       P, I64, P, I64, P]
        L.or_topk.argtypes = [P, I64, P, I64, I64, P, I64]
        L.or_bf16_round.restype = D
        L.or_bf16_round.argtypes = [C.c_float]
        L.or_dcp_topk.argtypes = [P, I64, P, I64, I64, I64, P, I64, P]
        L.or_sparse_mla.argtypes = [C.POINTER(OrLayout), I64, P, I64, P, I64, P, P, I64, P, I64, I64, P, I64,
                                    P, P, I64, I64, D, D, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _np(a, dtype):
    """torch tensor / numpy array -> C-contiguous numpy array of dtype (host copy)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.view(__import__("torch").int16).numpy().view(np.uint16)
        else:
            a = a.numpy()
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3(code: int) -> float:
    return lib().or_e4m3(code)


def e2m1(nib: int) -> float:
    return lib().or_e2m1(nib)


def e8m0(code: int) -> float:
    return lib().or_e8m0(code)


def bf16(bits: int) -> float:
    return lib().or_bf16(bits)


def layout_make(page_size: int, n_layers: int, key_fmt: int, lat_fmt: int, extra_row_bytes: int = 0) -> OrLayout:
    out = OrLayout()
    rc = lib().or_layout_make(page_size, n_layers, key_fmt, lat_fmt, extra_row_bytes, C.byref(out))
    if rc != OK:
        raise ValueError("or_layout_make failed: %d" % rc)
    return out


def key_decode(key_fmt: int, row_bytes) -> tuple[np.ndarray, float]:
    row = _np(row_bytes, np.uint8)
    k = np.zeros(128, np.float64)
    s = np.zeros(1, np.float64)
    rc = lib().or_key_decode(key_fmt, _p(row), _p(k), _p(s))
    if rc != OK:
        raise ValueError(rc)
    return k, float(s[0])


def latent_decode(lat_fmt: int, row_bytes, kv_scale: float) -> np.ndarray:
    row = _np(row_bytes, np.uint8)
    kv = np.zeros(576, np.float64)
    rc = lib().or_latent_decode(lat_fmt, _p(row), kv_scale, _p(kv))
    if rc != OK:
        raise ValueError(rc)
    return kv


class OracleCache:
    """Host copies of one PagedCache (pool, block table, counts) plus the oracle's own layout."""

    def __init__(self, cache):
        lp = cache.layout
        self.layout = layout_make(lp["page_size"], lp["n_layers"], lp["key_fmt"], lp["lat_fmt"],
                                  lp["extra_row_bytes"])
        self.layer = cache.layer
        self.pool = _np(cache.pool, np.uint8)
        self.pool_rows = self.pool.shape[0]
        self.bt = _np(cache.block_table, np.int32)
        self.n_pages = _np(cache.n_pages, np.int32)
        self.ctx_len = _np(cache.ctx_len, np.int32)
        self.kv_scale = float(cache.kv_scale)
        self.n_req = self.bt.shape[0]


def resolve_pages(oc: OracleCache, off_ld: int | None = None):
    max_pages = oc.bt.shape[1]
    off_ld = max_pages if off_ld is None else off_ld
    lat = np.full((oc.n_req, off_ld), -2, np.int64)   # -2: never written
    key = np.full((oc.n_req, off_ld), -2, np.int64)
    rc = lib().or_resolve_pages(C.byref(oc.layout), oc.layer, _p(oc.bt), oc.bt.shape[1], _p(oc.n_pages),
                                oc.n_req, max_pages, oc.pool_rows, _p(lat), _p(key), off_ld)
    return rc, lat, key


def indexer_score(oc: OracleCache, q, q_fmt: int, q_scale, w, q_req, row_len, ld: int | None = None,
                  count_bytes: bool = False):
    """Scores [n_q, ld] float32 (entries past row_len are NaN-filled, never written)."""
    qa = _np(q, np.uint16 if q_fmt == 0 else np.uint8)
    qs = _np(q_scale, np.float32)
    wa = _np(w, np.float32)
    qr = _np(q_req, np.int32)
    rl = _np(row_len, np.int32)
    n_q = rl.shape[0]
    ld = int(rl.max()) if ld is None else ld
    sc = np.full((n_q, ld), np.nan, np.float32)
    nb = np.zeros(n_q, np.int64) if count_bytes else None
    rc = lib().or_indexer_score(C.byref(oc.layout), oc.layer, _p(oc.pool), oc.pool_rows, _p(oc.bt),
                                oc.bt.shape[1], _p(oc.n_pages), oc.n_req, _p(qa), q_fmt, _p(qs), _p(wa), _p(qr),
                                _p(rl), n_q, _p(sc), ld, _p(nb))
    if rc != OK:
        raise ValueError("or_indexer_score failed: %d" % rc)
    return (sc, nb) if count_bytes else sc


def topk(scores, row_len, k: int) -> np.ndarray:
    s = _np(scores, np.float32)
    rl = _np(row_len, np.int32)
    out = np.zeros((s.shape[0], k), np.int32)
    rc = lib().or_topk(_p(s), s.shape[1], _p(rl), s.shape[0], k, _p(out), k)
    if rc != OK:
        raise ValueError("or_topk failed: %d" % rc)
    return out


def bf16_round(x: float) -> float:
    """x (as fp32) rounded to the nearest BF16 value, ties to even (normal range)."""
    return lib().or_bf16_round(float(x))


def dcp_topk(scores, row_len, k: int, n_shards: int):
    """Outcome of the exact top-k merge across n_shards decode-context-parallel shards
    (token t on shard t mod n_shards): (idx [n_rows][k] ascending, -1 padded, under the
    order BF16(score) desc then index asc; resend [n_rows] bit mask of flagged shards)."""
    s = _np(scores, np.float32)
    rl = _np(row_len, np.int32)
    out = np.zeros((s.shape[0], k), np.int32)
    rs = np.zeros(s.shape[0], np.uint32)
    rc = lib().or_dcp_topk(_p(s), s.shape[1], _p(rl), s.shape[0], k, n_shards, _p(out), k, _p(rs))
    if rc != OK:
        raise ValueError("or_dcp_topk failed: %d" % rc)
    return out, rs


def sparse_mla(oc: OracleCache, idx, q, q_fmt: int, q_scale, q_req, n_heads: int, sm_scale: float,
               count_bytes: bool = False):
    """Exact attention over idx's entries: out [n_q, H, 512] float64, lse [n_q, H] float64."""
    ia = _np(idx, np.int32)
    qa = _np(q, np.uint16 if q_fmt == 0 else np.uint8)
    qs = _np(q_scale, np.float32)
    qr = _np(q_req, np.int32)
    n_q, k = ia.shape
    out = np.zeros((n_q, n_heads, 512), np.float64)
    lse = np.zeros((n_q, n_heads), np.float64)
    nb = np.zeros(n_q, np.int64) if count_bytes else None
    rc = lib().or_sparse_mla(C.byref(oc.layout), oc.layer, _p(oc.pool), oc.pool_rows, _p(oc.bt), oc.bt.shape[1],
                             _p(oc.n_pages), _p(oc.ctx_len), oc.n_req, _p(ia), k, k, _p(qa), q_fmt, _p(qs),
                             _p(qr), n_q, n_heads, float(sm_scale), oc.kv_scale, _p(out), _p(lse), _p(nb))
    if rc != OK:
        raise ValueError("or_sparse_mla failed: %d" % rc)
    return (out, lse, nb) if count_bytes else (out, lse)
