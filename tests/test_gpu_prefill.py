"""GPU parity of the prefill path (FP8 indexer GEMM, per-row top-k, sparse MLA prefill)."""
import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import workloads as W
from tests.helpers import topk_set_ok, torch_e4m3_values
from tests.test_gpu_decode import check_attention, check_scores, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def make_prefill(d, prefix, chunk, heads=96, seed=0, q_fmt=1, k=2048, spare_rows=3):
    log(f"[case] prefill prefix={prefix} chunk={chunk} heads={heads} q_fmt={q_fmt} seed={seed}")
    cache = W.build_cache([prefix + chunk], seed=seed, device="cuda", spare_rows=spare_rows)
    pq = W.prefill_queries(prefix, chunk, heads, seed=seed, device="cuda")
    return cache, pq, d.PrefillStep(cache, pq, k=k, q_fmt=q_fmt)


def oracle_prefill_scores(cache, pq, q_fmt):
    oc = oracle.OracleCache(cache)
    if q_fmt == 1:
        q, qs = pq.q_idx_fp8, pq.q_idx_scale
    else:
        q, qs = pq.q_idx_bf16, None
    rl = pq.row_len.cpu().numpy()
    return oc, oracle.indexer_score(oc, q, q_fmt, qs, pq.w, pq.q_req, rl, ld=int(cache.ctx_len.max()))


@pytest.mark.parametrize("q_fmt", [1, 0])
def test_prefill_scores_match_oracle(d, q_fmt):
    cache, pq, step = make_prefill(d, 3000, 70, seed=1, q_fmt=q_fmt)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    _, ref = oracle_prefill_scores(cache, pq, q_fmt)
    rl = pq.row_len.cpu().numpy()
    check_scores(got, ref, rl)
    for r, L in enumerate(rl):     # causal: nothing written past the row's position
        assert np.isnan(got[r, L:]).all()


def test_prefill_gemm_rows_of_several_requests(d):
    """Rows of one 32-row tile from different requests (interleaved) and negative query scales."""
    ctx = [1500, 700, 2100]
    cache = W.build_cache(ctx, seed=5, device="cuda", spare_rows=2)
    rng = np.random.default_rng(5)
    n_q = 45
    q_req = rng.integers(0, 3, size=n_q).astype(np.int32)
    row_len = np.array([rng.integers(1, ctx[b] + 1) for b in q_req], np.int32)
    q = torch.randn(n_q, 32, 128, generator=torch.Generator().manual_seed(5))
    codes, qs = F.fp8_rowhead_quant(q)
    qs[::5, 3] *= -1.0                     # a negative query scale: ReLU sees the sign
    w = torch.rand(n_q, 32, generator=torch.Generator().manual_seed(6)) / 32
    layout = d.dsa_layout_make(64, 1, 0, 0, 0)
    lat_off = torch.empty(3, cache.max_pages, dtype=torch.int64, device="cuda")
    key_off = torch.empty_like(lat_off)
    d.dsa_resolve_pages(layout, 0, cache.block_table, cache.n_pages, cache.pool_rows, lat_off, key_off)
    scores = torch.full((n_q, max(ctx)), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(d.dsa_indexer_score_workspace_size(n_q, d.DSA_Q_FP8_E4M3), dtype=torch.uint8, device="cuda")
    d.dsa_indexer_score(layout, cache.pool, key_off, 3, codes.cuda(), d.DSA_Q_FP8_E4M3, qs.cuda(), w.cuda(),
                        torch.from_numpy(q_req).cuda(), torch.from_numpy(row_len).cuda(), scores, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    oc = oracle.OracleCache(cache)
    ref = oracle.indexer_score(oc, codes, 1, qs, w, q_req, row_len, ld=max(ctx))
    check_scores(scores.cpu().numpy(), ref, row_len)


@pytest.mark.parametrize("q_fmt", [1, 0])
def test_prefill_chain(d, q_fmt):
    cache, pq, step = make_prefill(d, 2500, 40, heads=96, seed=2 + q_fmt, q_fmt=q_fmt)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    rl = pq.row_len.cpu().numpy()
    got_s = step.scores.cpu().numpy()
    oc, ref_s = oracle_prefill_scores(cache, pq, q_fmt)
    check_scores(got_s, ref_s, rl)
    got_idx = step.idx.cpu().numpy()
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s), rl, 2048))
    topk_set_ok(ref_s, oracle.topk(np.nan_to_num(ref_s), rl, 2048), got_idx, rl, 2048)
    if q_fmt == 1:
        q, qs = pq.q_mla_fp8, pq.q_mla_scale
    else:
        q, qs = pq.q_mla_bf16, None
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, q, q_fmt, qs, pq.q_req, 96, pq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


@pytest.mark.parametrize("lat_fmt,heads,k", [(0, 48, 2048), (1, 96, 2048), (0, 128, 4096), (1, 40, 4096)])
def test_mla_prefill_all_heads_per_row(d, lat_fmt, heads, k):
    """FP8 queries with more than two 16-head tiles take the kernel that serves every head of
    a row from one gather; k = 4096 adds a second token split and the merge."""
    cache, pq, step = make_prefill(d, 5000, 24, heads=heads, seed=40 + heads, q_fmt=1, k=k)
    if lat_fmt == 1:  # same geometry, MXFP4 keys and NVFP4 latents
        cache = W.build_cache([5000 + 24], key_fmt=1, lat_fmt=1, seed=41 + heads, device="cuda", spare_rows=3)
        step = d.PrefillStep(cache, pq, k=k, q_fmt=1)
    rng = np.random.default_rng(heads + k)
    rl = pq.row_len.cpu().numpy()
    idx = np.full((pq.n_q, k), -1, np.int32)
    for r in range(pq.n_q):
        n = min(k, int(rl[r]))
        sel = np.sort(rng.choice(int(rl[r]), n, replace=False)).astype(np.int32)
        sel = sel[rng.random(n) >= 0.05]  # some -1 padding
        idx[r, :len(sel)] = sel
    idx[3, :7] = 11                       # one token seven times
    idx[5, :] = -1                        # an empty row
    step.resolve()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, pq.q_mla_fp8, 1, pq.q_mla_scale, pq.q_req, heads, pq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)
    assert np.isneginf(step.lse[5].cpu().numpy()).all() and (step.out[5].float() == 0).all()


@pytest.mark.parametrize("lat_fmt,heads,q_fmt", [(0, 96, 1), (1, 96, 1), (0, 12, 0)])
def test_mla_prefill_padding_with_nan_at_pool_start(d, lat_fmt, heads, q_fmt):
    """Index sets with -1 padding, and the pool's first row all 0xFF (NaN in every format, as an
    unused or uninitialised row may be): the kernels must not let the bytes they read for a
    padding entry reach the output, where a zero softmax weight times NaN would give NaN."""
    seed = 90 + heads + lat_fmt
    base = W.build_cache([3000 + 16], key_fmt=lat_fmt, lat_fmt=lat_fmt, seed=seed, device="cuda", spare_rows=2)
    rs = base.pool.shape[1]
    pool = torch.cat([torch.full((1, rs), 0xFF, dtype=torch.uint8, device="cuda"), base.pool])
    bt = torch.where(base.block_table >= 0, base.block_table + 1, base.block_table)
    cache = W.PagedCache(**{**base.__dict__, "pool": pool, "block_table": bt.contiguous()})
    pq = W.prefill_queries(3000, 16, heads, seed=seed, device="cuda")
    log(f"[case] poisoned pool start: lat_fmt={lat_fmt} heads={heads} q_fmt={q_fmt}")
    step = d.PrefillStep(cache, pq, k=2048, q_fmt=q_fmt)
    rng = np.random.default_rng(seed)
    rl = pq.row_len.cpu().numpy()
    idx = np.full((pq.n_q, 2048), -1, np.int32)
    for r in range(pq.n_q):
        sel = np.sort(rng.choice(int(rl[r]), 1500, replace=False)).astype(np.int32)
        idx[r, :len(sel)] = sel
        idx[r, 700:710] = -1  # padding inside the set as well as after it
    step.resolve()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    assert torch.isfinite(step.out.float()).all() and torch.isfinite(step.lse).all()
    q, qs = (pq.q_mla_fp8, pq.q_mla_scale) if q_fmt == 1 else (pq.q_mla_bf16, None)
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, q, q_fmt, qs, pq.q_req, heads, pq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


def test_mla_prefill_reference_far_below_a_later_max(d):
    """The FP8-latent prefill kernel fixes each head's softmax reference at its first subtile's
    max.  Here row 2 head 0's first subtile scores far below a later token (log2 logit gap
    > 64), so the row is computed again with the true max.  The logits stay small in absolute
    terms (first subtile about -58, the later token about +8), so the comparison keeps the
    usual tolerances; the result must be the oracle's exact softmax."""
    cache, pq, step = make_prefill(d, 3000, 8, heads=96, seed=77, q_fmt=1, k=2048)
    step.resolve()
    torch.cuda.synchronize()
    k, H = 2048, 96
    rl = pq.row_len.cpu().numpy()
    idx = np.full((pq.n_q, k), -1, np.int32)
    for r in range(pq.n_q):
        n = min(k, int(rl[r]))
        idx[r, :n] = np.arange(n, dtype=np.int32)  # tokens 0 .. n-1 in order: 0 .. 31 is subtile 0
    # e4m3 latent codes of one magnitude with the signs of row 2 head 0's query (or against them)
    qd = pq.q_mla_fp8[2, 0].cpu().numpy()
    qv = torch_e4m3_values(qd).astype(np.float64) * float(pq.q_mla_scale[2, 0])
    base = abs(qv).sum() * pq.sm_scale * cache.kv_scale / np.log(2.0)  # log2 logit per unit code value
    grid = [((c >> 3) & 15, c & 7) for c in range(1, 127)]
    vals = sorted(((1 + mm / 8) * 2.0 ** (ee - 7) if ee else mm / 8 * 2.0 ** -6, (ee << 3) | mm) for ee, mm in grid)
    m0, c0 = max((x for x in vals if base * x[0] <= 60.0), key=lambda x: x[0])
    m1, c1 = min((x for x in vals if base * (m0 + x[0]) > 65.0), key=lambda x: x[0])
    assert base * m0 > 50.0 and base * m1 < 16.0, f"no e4m3 pair fits: {base:.3g} per unit"
    low = np.where(qv < 0, c0, c0 | 0x80).astype(np.uint8)   # against the query: logit -base m0
    high = np.where(qv < 0, c1 | 0x80, c1).astype(np.uint8)  # along it: logit +base m1
    lat_off = step.lat_off.cpu().numpy()
    row_off = lambda t: int(lat_off[0, t >> 6]) + (t & 63) * 576
    flat = cache.pool.view(-1)  # the offsets are bytes from the pool base; the pool is [rows, row_stride]
    for t, codes in [(t, low) for t in range(32)] + [(1000, high)]:
        o = row_off(t)
        assert 0 <= o and o + 576 <= flat.numel()
        flat[o:o + 576] = torch.from_numpy(codes).cuda()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, pq.q_mla_fp8, 1, pq.q_mla_scale, pq.q_req, H, pq.sm_scale)
    assert base * (m0 + m1) > 64.0  # the gap the second pass exists for
    check_attention(step.out, step.lse, ref_o, ref_l)
