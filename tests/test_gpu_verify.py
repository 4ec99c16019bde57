"""GPU parity of speculative-verify decode (dsa_indexer_score_verify): m query rows per
request share one read of every key page, then each row gets its own top-k and attention.

Bars:
  * scores: |gpu - ref| <= 1e-5*|ref| + 1e-5*rms(row) against the oracle, with each row
    scored for its own request (q_req = r // m); in addition bit-equal to the one-row
    indexer (dsa_indexer_score with that q_req), since both run the same per-row arithmetic;
    nothing is written past a row's length;
  * top-k: bit-exact on the GPU's scores, tie window against the oracle's scores;
  * attention on the GPU's index set: max|dout| <= 1e-2*max|ref|, max|dlse| <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.helpers import topk_set_ok
from tests.test_gpu_decode import check_attention, check_scores, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def make(d, ctx, m, key_fmt=0, lat_fmt=0, seed=0, heads=12, k=2048, row_len=None, **kw):
    log(f"[case] verify ctx={ctx[:6]}{'...' if len(ctx) > 6 else ''} n={len(ctx)} m={m} key_fmt={key_fmt} "
        f"lat_fmt={lat_fmt} seed={seed} k={k}")
    cache = W.build_cache(ctx, key_fmt=key_fmt, lat_fmt=lat_fmt, seed=seed, device="cuda", **kw)
    vq = W.verify_queries(ctx, m, heads, seed=seed, device="cuda")
    if row_len is not None:
        vq.row_len = torch.tensor(row_len, dtype=torch.int32, device="cuda")
    step = d.VerifyStep(cache, vq, k=k)
    return cache, vq, step


def one_row_scores(d, step, vq):
    """The same rows through the one-row indexer (q_req = r // m)."""
    c = step.cache
    s = torch.full_like(step.scores, float("nan"))
    d.dsa_indexer_score(step.layout, c.pool, step.key_off, c.n_req, vq.q_idx, d.DSA_Q_BF16, None, vq.w, vq.q_req,
                        vq.row_len, s, None, step.err)
    return s


@pytest.mark.parametrize("m,key_fmt", [(1, 0), (2, 0), (3, 1), (4, 0), (5, 0), (7, 1), (8, 0), (8, 1)])
def test_verify_scores_match_oracle(d, m, key_fmt):
    ctx = [4096, 777, 64, 1 + m, 130, 3000, 65]
    cache, vq, step = make(d, ctx, m, key_fmt=key_fmt, lat_fmt=key_fmt, seed=20 + m + 10 * key_fmt, spare_rows=5,
                           n_layers=2, layer=1)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    ref_gpu = one_row_scores(d, step, vq)
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    rl = vq.row_len.cpu().numpy()
    oc = oracle.OracleCache(cache)
    ref = oracle.indexer_score(oc, vq.q_idx, 0, None, vq.w, vq.q_req, rl, ld=step.scores.shape[1])
    check_scores(got, ref, rl)
    one = ref_gpu.cpu().numpy()
    for r, L in enumerate(rl):
        assert np.array_equal(got[r, :L].view(np.uint32), one[r, :L].view(np.uint32)), f"row {r}"
        assert np.isnan(got[r, L:]).all(), f"row {r} written past its length"


def test_verify_ragged_row_lengths(d):
    """Rows of one request with unrelated lengths (0, 1, a page edge, shorter and longer than
    their neighbours): every row stops at its own length, pages past the longest are not read."""
    ctx = [5000, 300, 2100]
    m = 4
    rl = [5000, 0, 64, 4097, 1, 300, 299, 129, 2100, 2000, 65, 2099]
    cache, vq, step = make(d, ctx, m, seed=31, row_len=rl, spare_rows=3)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    oc = oracle.OracleCache(cache)
    ref = oracle.indexer_score(oc, vq.q_idx, 0, None, vq.w, vq.q_req, np.array(rl, np.int32),
                               ld=step.scores.shape[1])
    check_scores(got, ref, rl)
    for r, L in enumerate(rl):
        assert np.isnan(got[r, L:]).all(), f"row {r} written past its length"


def test_verify_row_len_past_pages_flags(d):
    ctx = [640, 200]
    cache, vq, step = make(d, ctx, 2, seed=32, row_len=[640, 641, 200, 199], max_pages=10)
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) & d.DSA_DEVERR_ROW_LEN


def test_verify_errors(d):
    cache, vq, step = make(d, [256], 2, seed=33)
    c = cache
    with pytest.raises(d.DsaError) as e:
        d.dsa_indexer_score_verify(step.layout, c.pool, step.key_off, 1, 9, vq.q_idx, vq.w, vq.row_len, step.scores)
    assert e.value.status == d.DSA_ERR_UNSUPPORTED
    with pytest.raises(d.DsaError) as e:
        d.dsa_indexer_score_verify(step.layout, c.pool, step.key_off, 1, 0, vq.q_idx, vq.w, vq.row_len, step.scores)
    assert e.value.status == d.DSA_ERR_BAD_SHAPE


@pytest.mark.parametrize("m,key_fmt,lat_fmt", [(8, 0, 0), (3, 1, 1)])
def test_verify_chain(d, m, key_fmt, lat_fmt):
    """resolve -> verify scores -> top-2048 per row -> attention per row, against the oracle."""
    ctx = [9000, 2500, 4096]
    cache, vq, step = make(d, ctx, m, key_fmt=key_fmt, lat_fmt=lat_fmt, seed=40 + m, spare_rows=4)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    rl = vq.row_len.cpu().numpy()
    oc = oracle.OracleCache(cache)
    ref_s = oracle.indexer_score(oc, vq.q_idx, 0, None, vq.w, vq.q_req, rl, ld=step.scores.shape[1])
    got_s = step.scores.cpu().numpy()
    check_scores(got_s, ref_s, rl)
    got_idx = step.idx.cpu().numpy()
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s, nan=0.0), rl, 2048))
    topk_set_ok(np.nan_to_num(ref_s, nan=0.0), oracle.topk(np.nan_to_num(ref_s, nan=0.0), rl, 2048), got_idx, rl,
                2048)
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, vq.q_mla, 0, None, vq.q_req, vq.q_mla.shape[1], vq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


def test_verify_rows_match_decode_of_their_own(d):
    """Row i of a verify batch equals a one-row decode of the same query at the same length:
    the same scores bit for bit and the same top-k (batch invariance across the two paths)."""
    ctx = [7000, 3000]
    m = 4
    cache, vq, step = make(d, ctx, m, seed=45)
    step.run()
    torch.cuda.synchronize()
    for r in (0, 3, 6):
        b = r // m
        L = int(vq.row_len[r].item())
        dstep = d.DecodeStep(cache, vq.q_idx[r:r + 1].contiguous(), vq.w[r:r + 1].contiguous(),
                             vq.q_mla[r:r + 1].contiguous(), vq.sm_scale, k=2048)
        dstep.q_req = torch.tensor([b], dtype=torch.int32, device="cuda")
        dstep.row_len = torch.tensor([L], dtype=torch.int32, device="cuda")
        dstep.resolve()
        dstep.score()
        dstep.topk()
        torch.cuda.synchronize()
        a = step.scores[r, :L].cpu().numpy().view(np.uint32)
        bb = dstep.scores[0, :L].cpu().numpy().view(np.uint32)
        assert np.array_equal(a, bb), f"row {r}"
        assert np.array_equal(step.idx[r].cpu().numpy(), dstep.idx[0].cpu().numpy()), f"row {r}"


def test_verify_full_size_sampled_rows(d):
    """The verify workload bench.py times (32 requests x 8 rows at 131,072 tokens), sampled rows
    against the oracle."""
    cfg = 5
    wl = W.WORKLOADS[cfg]
    ctx = W.workload_ctx(cfg)
    k, m = wl["topk"], wl["rows"]
    log(f"[case] full size {wl['name']}: {len(ctx)} requests x {m} rows, {sum(ctx)} tokens")
    cache = W.build_cache(ctx, key_fmt=wl["key_fmt"], lat_fmt=wl["lat_fmt"], seed=cfg, device="cuda",
                          spare_rows=wl["spare_rows"])
    vq = W.verify_queries(ctx, m, wl["heads"], seed=cfg, device="cuda")
    step = d.VerifyStep(cache, vq, k=k)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    for r in (0, 7, 8 * 17 + 3, 8 * 32 - 1):
        L = int(vq.row_len[r].item())
        req = vq.q_req[r:r + 1].cpu().numpy()
        log(f"[row] {wl['name']} row {r} length {L}")
        ref_s = oracle.indexer_score(oc, vq.q_idx[r:r + 1], 0, None, vq.w[r:r + 1], req, np.array([L], np.int32))
        got_s = step.scores[r:r + 1, :L].cpu().numpy()
        check_scores(got_s, ref_s, [L])
        got_idx = step.idx[r:r + 1].cpu().numpy()
        assert np.array_equal(got_idx, oracle.topk(got_s, np.array([L], np.int32), k))
        topk_set_ok(ref_s, oracle.topk(ref_s, np.array([L], np.int32), k), got_idx, [L], k)
        ref_o, ref_l = oracle.sparse_mla(oc, got_idx, vq.q_mla[r:r + 1], 0, None, req, wl["heads"], vq.sm_scale)
        check_attention(step.out[r:r + 1], step.lse[r:r + 1], ref_o, ref_l)


@pytest.mark.parametrize("m", [1, 6])
def test_verify_empty_and_single_token_requests(d, m):
    """Requests whose rows are all empty, a one-token request, and many short requests (the
    request table lives in LDS): scores match the oracle and nothing past a length is written."""
    rng = np.random.default_rng(50 + m)
    ctx = [m + 1, 1, 900] + [int(x) for x in rng.integers(1, 400, size=300)]
    rl = []
    for b, L in enumerate(ctx):
        for i in range(m):
            rl.append(0 if b == 0 else max(0, L - m + 1 + i))
    cache, vq, step = make(d, ctx, m, seed=52 + m, row_len=rl)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    oc = oracle.OracleCache(cache)
    ref = oracle.indexer_score(oc, vq.q_idx, 0, None, vq.w, vq.q_req, np.array(rl, np.int32),
                               ld=step.scores.shape[1])
    check_scores(got, ref, rl)
    for r, L in enumerate(rl):
        assert np.isnan(got[r, L:]).all(), f"row {r} written past its length"


def test_verify_max_requests(d):
    """The largest request count the entry point takes (1024) at 8 rows each with FP8 keys:
    the request table in LDS then brings the workgroup to 158,788 of 163,840 bytes of LDS."""
    rng = np.random.default_rng(60)
    m = 8
    ctx = [int(x) for x in rng.integers(m, 100, size=1024)]
    cache, vq, step = make(d, ctx, m, seed=61)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    rl = vq.row_len.cpu().numpy()
    oc = oracle.OracleCache(cache)
    ref = oracle.indexer_score(oc, vq.q_idx, 0, None, vq.w, vq.q_req, rl, ld=step.scores.shape[1])
    check_scores(got, ref, rl)
    for r, L in enumerate(rl):
        assert np.isnan(got[r, L:]).all(), f"row {r} written past its length"
