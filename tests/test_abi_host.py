"""Host-only checks of the C ABI: the library loads without a GPU, exports every
function include/dsa.h declares, and rejects bad arguments with the documented
status before enqueuing anything (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def d():
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(d):
    names = declared_functions()
    assert len(names) == 27
    for n in names:
        assert hasattr(d.lib, n), n


def test_layout_make_matches_pages(d):
    L = d.dsa_layout_make(64, 24, d.DSA_KEY_FP8_E4M3_SCALED, d.DSA_LAT_FP8_E4M3, 0)
    assert (L.key_bytes, L.lat_bytes, L.layer_stride, L.row_stride) == (132, 576, 45312, 24 * 45312)
    L = d.dsa_layout_make(64, 1, d.DSA_KEY_MXFP4, d.DSA_LAT_NVFP4, 300)
    assert (L.key_bytes, L.lat_bytes, L.layer_stride, L.row_stride) == (68, 352, 26880, 27392)


def test_layout_agrees_with_generator_and_oracle(d):
    import oracle
    from synth import workloads as W
    for kf in (0, 1):
        for lf in (0, 1):
            for nl, ex in ((1, 0), (3, 17), (24, 4096)):
                got = d.dsa_layout_make(64, nl, kf, lf, ex).as_dict()
                gen = W.layout_params(kf, lf, nl, 64, ex)
                orc = oracle.layout_make(64, nl, kf, lf, ex).as_dict()
                for k in ("key_bytes", "lat_bytes", "layer_stride", "row_stride"):
                    assert got[k] == gen[k] == orc[k], (kf, lf, nl, ex, k)


def test_layout_make_errors(d):
    out = d.dsa_layout()
    assert d.lib.dsa_layout_make(64, 1, 0, 0, 0, None) == d.DSA_ERR_NULL_ARG
    assert d.lib.dsa_layout_make(0, 1, 0, 0, 0, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert d.lib.dsa_layout_make(64, 0, 0, 0, 0, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert d.lib.dsa_layout_make(64, 1, 0, 0, -1, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert d.lib.dsa_layout_make(64, 1, 2, 0, 0, C.byref(out)) == d.DSA_ERR_UNSUPPORTED
    assert d.lib.dsa_layout_make(64, 1, 0, 5, 0, C.byref(out)) == d.DSA_ERR_UNSUPPORTED


FAKE = C.c_void_p(1 << 20)      # aligned, never dereferenced: every call below fails validation first
ODD = C.c_void_p((1 << 20) + 2)


def test_prefill_select_errors(d):
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_prefill_select
    n_q, ld, n_req, off_ld, k = 40, 5000, 2, 80, 2048
    need = d.dsa_prefill_select_workspace_size(n_q, ld, n_req, off_ld, k)
    # bf16 + e4m3 query rows, the band lists and the top-k's own workspace
    assert need >= n_q * 32 * 128 * 3 + n_q * (8192 * 8 + 4096 * 4) + d.dsa_topk_workspace_size(n_q, ld, k)
    args = [C.byref(L), FAKE, 1 << 30, FAKE, off_ld, n_req, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n_q, k, FAKE, ld,
            FAKE, k, None, FAKE, need, None, None]
    a = list(args); a[1] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[6] = None     # ctx_len
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[8] = None     # q_scale
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[19] = None    # workspace
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[20] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[19] = C.c_void_p(FAKE.value + 16)
    assert f(*a) == d.DSA_ERR_MISALIGNED
    a = list(args); a[14] = C.c_void_p(FAKE.value + 4)   # scores: 16-B aligned
    assert f(*a) == d.DSA_ERR_MISALIGNED
    a = list(args); a[17] = k - 1   # idx_ld < k
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[13] = 0
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[13] = 4097; a[17] = 4097
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    Lm = d.dsa_layout_make(64, 1, 1, 1, 0)
    a = list(args); a[0] = C.byref(Lm)   # FP8 keys only
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[12] = 0
    assert f(*a) == d.DSA_OK
    # the halves: the same checks
    h = d.lib.dsa_prefill_score_fp8
    hargs = [C.byref(L), FAKE, 1 << 30, FAKE, off_ld, n_req, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n_q, k, FAKE, ld,
             None, FAKE, need, None, None]
    a = list(hargs); a[6] = None
    assert h(*a) == d.DSA_ERR_NULL_ARG
    a = list(hargs); a[13] = 0      # k
    assert h(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(hargs); a[18] = need - 1
    assert h(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(hargs); a[0] = C.byref(Lm)
    assert h(*a) == d.DSA_ERR_UNSUPPORTED
    t = d.lib.dsa_prefill_topk_band
    targs = [C.byref(L), FAKE, 1 << 30, FAKE, off_ld, n_req, FAKE, FAKE, n_q, k, FAKE, ld, FAKE, k, FAKE, need, None,
             None]
    a = list(targs); a[12] = None
    assert t(*a) == d.DSA_ERR_NULL_ARG
    a = list(targs); a[13] = k - 1
    assert t(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(targs); a[14] = C.c_void_p(FAKE.value + 16)
    assert t(*a) == d.DSA_ERR_MISALIGNED
    a = list(targs); a[8] = 0
    assert t(*a) == d.DSA_OK
    out = C.c_size_t()
    g = d.lib.dsa_prefill_select_workspace_size
    assert g(-1, ld, n_req, off_ld, k, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert g(n_q, ld, n_req, 0, k, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert g(n_q, 1 << 24, n_req, off_ld, k, C.byref(out)) == d.DSA_ERR_UNSUPPORTED
    assert g(n_q, ld, n_req, off_ld, k, None) == d.DSA_ERR_NULL_ARG


def test_resolve_errors(d):
    L = d.dsa_layout_make(64, 2, 0, 0, 0)
    f = d.lib.dsa_resolve_pages
    assert f(None, 0, FAKE, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_NULL_ARG
    assert f(C.byref(L), 0, None, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_NULL_ARG
    assert f(C.byref(L), 2, FAKE, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_BAD_SHAPE   # layer
    assert f(C.byref(L), 0, FAKE, 4, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_BAD_SHAPE   # bt_ld
    assert f(C.byref(L), 0, FAKE, 8, FAKE, 1, 8, 10, FAKE, FAKE, 7, None, None) == d.DSA_ERR_BAD_SHAPE   # off_ld
    assert f(C.byref(L), 0, ODD, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_MISALIGNED
    bad = d.dsa_layout_make(64, 2, 0, 0, 0)
    bad.row_stride += 256
    assert f(C.byref(bad), 0, FAKE, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_BAD_SHAPE
    p32 = d.dsa_layout_make(32, 2, 0, 0, 0)
    assert f(C.byref(p32), 0, FAKE, 8, FAKE, 1, 8, 10, FAKE, FAKE, 8, None, None) == d.DSA_ERR_UNSUPPORTED


def test_score_errors(d):
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_indexer_score
    args = [C.byref(L), FAKE, 1 << 30, FAKE, 16, 1, FAKE, 0, None, FAKE, FAKE, FAKE, 4, FAKE, 1024, None, 0, None,
            None]
    a = list(args); a[1] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[7] = 1        # FP8 queries without q_scale
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[7] = 3
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[1] = ODD
    assert f(*a) == d.DSA_ERR_MISALIGNED
    a = list(args); a[12] = -1
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[12] = 5000    # the streaming (bf16) path takes <= 4096 rows
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    Lm = d.dsa_layout_make(64, 1, 1, 1, 0)
    a = list(args); a[0] = C.byref(Lm); a[7] = 1; a[8] = FAKE   # FP8 queries need FP8 keys
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[7] = d.DSA_Q_MXFP4                        # MXFP4 queries need MXFP4 keys
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    assert d.dsa_indexer_score_workspace_size(4, d.DSA_Q_MXFP4) == 0
    a = list(args); a[12] = 0       # nothing to do
    assert f(*a) == d.DSA_OK
    # FP8 queries take a workspace: rows of bf16 query heads, and the weights
    need = d.dsa_indexer_score_workspace_size(4, d.DSA_Q_FP8_E4M3)
    assert need >= 4 * 32 * 128 * 2 + 32 * 32 * 4
    assert d.dsa_indexer_score_workspace_size(4, d.DSA_Q_BF16) == 0
    assert d.dsa_indexer_score_workspace_size(0, d.DSA_Q_FP8_E4M3) == 0
    a = list(args); a[7] = 1; a[8] = FAKE; a[15] = FAKE; a[16] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[7] = 1; a[8] = FAKE; a[15] = None; a[16] = need
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[7] = 1; a[8] = FAKE; a[15] = C.c_void_p(FAKE.value + 16); a[16] = need
    assert f(*a) == d.DSA_ERR_MISALIGNED
    out = C.c_size_t()
    assert d.lib.dsa_indexer_score_workspace_size(-1, 1, C.byref(out)) == d.DSA_ERR_BAD_SHAPE
    assert d.lib.dsa_indexer_score_workspace_size(4, 7, C.byref(out)) == d.DSA_ERR_UNSUPPORTED
    assert d.lib.dsa_indexer_score_workspace_size(4, 1, None) == d.DSA_ERR_NULL_ARG



def test_score_verify_errors(d):
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_indexer_score_verify
    args = [C.byref(L), FAKE, 1 << 30, FAKE, 16, 2, 8, FAKE, FAKE, FAKE, FAKE, 1024, None, None]
    a = list(args); a[0] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[7] = None     # q
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[6] = 0        # rows per request
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[6] = 9        # more rows than the kernel stages
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[5] = 1025     # requests
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[5] = -1
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[4] = 0        # off_ld
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[7] = C.c_void_p((1 << 20) + 8)   # q must be 16-B aligned
    assert f(*a) == d.DSA_ERR_MISALIGNED
    a = list(args); a[10] = ODD     # scores
    assert f(*a) == d.DSA_ERR_MISALIGNED
    bad = d.dsa_layout_make(64, 1, 0, 0, 0)
    bad.layer_stride += 256
    a = list(args); a[0] = C.byref(bad)
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[5] = 0        # nothing to do
    assert f(*a) == d.DSA_OK

def test_topk_errors(d):
    f = d.lib.dsa_topk
    need = d.dsa_topk_workspace_size(4, 20000, 2048)
    args = [FAKE, 20000, FAKE, 4, 2048, FAKE, 2048, FAKE, need, None, None]
    a = list(args); a[4] = 0
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[4] = 5000
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[6] = 100
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[8] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[7] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[7] = C.c_void_p((1 << 20) + 8)
    assert f(*a) == d.DSA_ERR_MISALIGNED
    with pytest.raises(d.DsaError):
        d.dsa_topk_workspace_size(1, 1 << 30, 2048)


def test_dcp_topk_errors(d):
    f = d.lib.dsa_dcp_topk
    need = d.dsa_dcp_topk_workspace_size(4, 2048, 8)
    # counts, first candidate lists (c = 384), flags, resend counts and lists
    assert need >= 4 * 8 * 4 * 2 + 4 * 8 * 384 * 4 + 4 * 4 + 4 * 8 * 2048 * 4
    args = [FAKE, 131072, FAKE, 4, 2048, 8, FAKE, 2048, None, FAKE, need, None, None]
    a = list(args); a[5] = 0
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[5] = 9
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[4] = 4096
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[1] = 65536 * 8 + 1   # local index past 16 bits
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[7] = 100
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[10] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[9] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[8] = C.c_void_p((1 << 20) + 2)
    assert f(*a) == d.DSA_ERR_MISALIGNED
    a = list(args); a[3] = 0               # nothing to do
    assert f(*a) == d.DSA_OK


def test_mla_errors(d):
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_sparse_mla_decode
    need = d.dsa_sparse_mla_decode_workspace_size(2, 12, 2048)
    assert need > 0
    args = [C.byref(L), FAKE, 1 << 30, FAKE, 16, FAKE, FAKE, 2048, 2048, FAKE, 2, 12, 0.04, 0.01, FAKE, FAKE, FAKE,
            need, None, None]
    a = list(args); a[11] = 0
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[11] = 129
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[17] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[7] = 100     # idx_ld < k
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[9] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    g = d.lib.dsa_sparse_mla_prefill
    pargs = [C.byref(L), FAKE, 1 << 30, FAKE, 16, 1, FAKE, FAKE, 2048, 2048, FAKE, 1, None, None, 4, 96, 0.04, 0.01,
             FAKE, FAKE, None, 0, None, None]
    assert g(*pargs) == d.DSA_ERR_NULL_ARG    # q_req and FP8 q_scale missing
    assert d.dsa_sparse_mla_prefill_workspace_size(2048, 96, 2048) == 0   # one split per prefill row


def test_status_strings(d):
    for s in range(8):
        assert d.dsa_status_str(s) and "unknown" not in d.dsa_status_str(s)
    assert "unknown" in d.dsa_status_str(99)


def test_binding_refuses_cpu_tensors(d):
    import torch
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    with pytest.raises(TypeError):
        d.dsa_resolve_pages(L, 0, torch.zeros(1, 4, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 4,
                            torch.zeros(1, 4, dtype=torch.int64), torch.zeros(1, 4, dtype=torch.int64))


def test_noalloc_rejects_beyond_its_scratch(d):
    """The no-allocation decode checks its partials against the static scratch size before
    any HIP call: 1000 requests x 128 heads at k = 2048 need about 4.2 GB."""
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_sparse_mla_decode_noalloc
    args = [C.byref(L), FAKE, 1 << 30, FAKE, 2048, FAKE, FAKE, 2048, 2048, FAKE, 1000, 128, 0.1, 1.0, FAKE, FAKE,
            None, None]
    assert f(*args) == d.DSA_ERR_SCRATCH_LIMIT
    need = d.dsa_sparse_mla_decode_workspace_size(64, 12, 2048)
    assert need <= d.DSA_NOALLOC_SCRATCH_BYTES   # the largest decode batch of the workloads fits
    a = list(args); a[10] = -1
    assert f(*a) == d.DSA_ERR_BAD_SHAPE


def test_fused_select_errors(d):
    """dsa_indexer_select and its two halves reject bad arguments before any launch."""
    L = d.dsa_layout_make(64, 2, 0, 0, 0)
    need = d.dsa_indexer_select_workspace_size(4, 1024)
    assert need == d.dsa_topk_workspace_size(4, 1024, 2048)  # the top-k's own workspace
    f = d.lib.dsa_indexer_select
    # layout, layer, pool, pool_bytes, bt, bt_ld, n_req, q, q_fmt, w, q_req, row_len, n_q, k, scores, ld,
    # idx, phys, idx_ld, ws, ws_bytes, err, stream
    args = [C.byref(L), 0, FAKE, 1 << 30, FAKE, 16, 4, FAKE, 0, FAKE, FAKE, FAKE, 4, 2048, FAKE, 1024, FAKE, FAKE,
            2048, FAKE, need, None, None]
    a = list(args); a[1] = 2
    assert f(*a) == d.DSA_ERR_BAD_SHAPE           # layer past n_layers
    a = list(args); a[8] = d.DSA_Q_MXFP4
    assert f(*a) == d.DSA_ERR_UNSUPPORTED         # MXFP4 queries on FP8 keys
    a = list(args); a[8] = d.DSA_Q_FP8_E4M3
    assert f(*a) == d.DSA_ERR_UNSUPPORTED         # the fused scan takes bf16 or MXFP4 queries
    a = list(args); a[15] = (1 << 23) + 4
    assert f(*a) == d.DSA_ERR_UNSUPPORTED         # rows past 2^23 scores
    a = list(args); a[13] = 4097; a[18] = 4097
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[13] = 0
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[18] = 100
    assert f(*a) == d.DSA_ERR_BAD_SHAPE           # idx_ld < k
    a = list(args); a[20] = need - 1
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[7] = ODD
    assert f(*a) == d.DSA_ERR_MISALIGNED          # q must be 16-B aligned
    a = list(args); a[4] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
    a = list(args); a[19] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG            # no workspace
    a = list(args); a[12] = 0
    assert f(*a) == d.DSA_OK                      # nothing to do
    a = list(args); a[12] = 5000
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    # phys output needs pool_row * 64 + slot to fit int32
    a = list(args); a[3] = (1 << 25) * L.row_stride
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    g = d.lib.dsa_topk_pages
    # layout, pool_bytes, bt, bt_ld, n_req, q_req, scores, ld, row_len, n_q, k, ws, ws_bytes, idx, phys, idx_ld,
    # err, stream
    targs = [C.byref(L), 1 << 30, FAKE, 16, 4, FAKE, FAKE, 1024, FAKE, 4, 2048, FAKE, need, FAKE, FAKE, 2048, None,
             None]
    a = list(targs); a[10] = 0
    assert g(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(targs); a[12] = 0
    assert g(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(targs); a[2] = None
    assert g(*a) == d.DSA_ERR_NULL_ARG
    h = d.lib.dsa_indexer_score_pages
    # layout, layer, pool, pool_bytes, bt, bt_ld, n_req, q, q_fmt, w, q_req, row_len, n_q, scores, ld, err, stream
    sargs = [C.byref(L), 0, FAKE, 1 << 30, FAKE, 16, 4, FAKE, 0, FAKE, FAKE, FAKE, 4, FAKE, 1024, None, None]
    a = list(sargs); a[1] = -1
    assert h(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(sargs); a[5] = 0
    assert h(*a) == d.DSA_ERR_BAD_SHAPE           # bt_ld < 1
    a = list(sargs); a[9] = None
    assert h(*a) == d.DSA_ERR_NULL_ARG


def test_mla_phys_errors(d):
    L = d.dsa_layout_make(64, 1, 0, 0, 0)
    f = d.lib.dsa_sparse_mla_decode_phys
    args = [C.byref(L), 0, FAKE, 1 << 30, FAKE, 2048, 2048, FAKE, 4, 12, 0.1, 1.0, FAKE, FAKE, FAKE, 1 << 30, None, None]
    a = list(args); a[1] = 1
    assert f(*a) == d.DSA_ERR_BAD_SHAPE
    a = list(args); a[9] = 129
    assert f(*a) == d.DSA_ERR_UNSUPPORTED
    a = list(args); a[15] = 16
    assert f(*a) == d.DSA_ERR_WORKSPACE_TOO_SMALL
    a = list(args); a[4] = None
    assert f(*a) == d.DSA_ERR_NULL_ARG
