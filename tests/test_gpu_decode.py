"""GPU parity of the decode path against the CPU oracle, through the C ABI.

Bars (the attention bar and the top-k tie window are the method's stated
acceptance; the score bar is derived from fp32 accumulation of exact products,
see the design notes):
  * resolve: bit-exact offsets;
  * scores:  |gpu - ref| <= 1e-5*|ref| + 1e-5*rms(row);
  * top-k:   bit-exact against the oracle's sort of the *same* scores; against the
             oracle's own scores, any swapped token lies within 1e-5*|T| of the k-th
             score T;
  * attention on the GPU's index set: max|dout| <= 1e-2*max|ref|, max|dlse| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.helpers import topk_set_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def log(msg):
    print(msg, flush=True)


def make(d, ctx, key_fmt=0, lat_fmt=0, seed=0, heads=12, k=2048, **kw):
    log(f"[case] ctx={ctx[:6]}{'...' if len(ctx) > 6 else ''} n={len(ctx)} key_fmt={key_fmt} lat_fmt={lat_fmt} "
        f"seed={seed} heads={heads} k={k}")
    cache = W.build_cache(ctx, key_fmt=key_fmt, lat_fmt=lat_fmt, seed=seed, device="cuda", **kw)
    dq = W.decode_queries(len(ctx), heads, seed=seed, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    return cache, dq, step


def check_scores(got, ref, row_len):
    for r, L in enumerate(row_len):
        g, f = got[r, :L].astype(np.float64), ref[r, :L].astype(np.float64)
        rms = math.sqrt(float(np.mean(f * f))) if L else 0.0
        err = np.abs(g - f)
        lim = 1e-5 * np.abs(f) + 1e-5 * rms
        assert (err <= lim).all(), f"row {r}: max err {err.max():.3g}, worst at {int(np.argmax(err - lim))}"


def check_attention(out, lse, ref_o, ref_l):
    """The bar per query row (stricter than over the whole tensor): max|dout| <= 1e-2 of the
    row's max|ref|, and |dlse| <= 1e-3."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    finite = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(l), finite), "empty sets must give lse = -inf exactly where the oracle does"
    assert (o[~finite] == 0).all()
    for r in range(o.shape[0]):
        scale = np.abs(ref_o[r]).max()
        err = np.abs(o[r] - ref_o[r]).max()
        assert err <= 1e-2 * scale, f"row {r}: out err {err:.3g} vs {scale:.3g}"
    if finite.any():
        assert np.abs(l[finite] - ref_l[finite]).max() <= 1e-3


def oracle_scores(cache, dq, row_len=None):
    oc = oracle.OracleCache(cache)
    n = cache.n_req
    rl = cache.ctx_len.cpu().numpy() if row_len is None else np.asarray(row_len, np.int32)
    return oc, oracle.indexer_score(oc, dq.q_idx, 0, None, dq.w, np.arange(n, dtype=np.int32), rl,
                                    ld=int(max(rl.max(), 1)))


# ------------------------------------------------------------------- resolve

def test_resolve_matches_oracle(d):
    cache, dq, step = make(d, [700, 64, 1, 300, 4096], key_fmt=0, lat_fmt=1, seed=1, spare_rows=7, n_layers=3,
                           layer=1, max_pages=80)
    step.lat_off.fill_(-7)
    step.key_off.fill_(-7)
    step.resolve()
    torch.cuda.synchronize()
    rc, lat, key = oracle.resolve_pages(oracle.OracleCache(cache))
    assert rc == oracle.OK
    assert np.array_equal(step.lat_off.cpu().numpy(), lat) and np.array_equal(step.key_off.cpu().numpy(), key)
    assert int(step.err.item()) == 0


def test_resolve_flags_bad_block(d):
    cache, dq, step = make(d, [300, 200], seed=2, spare_rows=2)
    cache.block_table[1, 2] = cache.pool_rows + 5
    step.resolve()
    torch.cuda.synchronize()
    assert int(step.err.item()) & d.DSA_DEVERR_BLOCK_RANGE
    assert int(step.lat_off[1, 2]) == -1 and int(step.key_off[1, 2]) == -1 and int(step.lat_off[1, 1]) >= 0


# ------------------------------------------------------------------- scores

@pytest.mark.parametrize("key_fmt", [0, 1])
def test_scores_match_oracle(d, key_fmt):
    ctx = [4096, 777, 64, 1, 130, 2000, 65, 3000]
    cache, dq, step = make(d, ctx, key_fmt=key_fmt, lat_fmt=key_fmt, seed=3 + key_fmt, spare_rows=5, n_layers=2,
                           layer=1)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    _, ref = oracle_scores(cache, dq)
    check_scores(got, ref, ctx)
    for r, L in enumerate(ctx):   # nothing written past a row's length
        assert np.isnan(got[r, L:]).all()


def test_scores_many_rows_key_balanced(d):
    rng = np.random.default_rng(7)
    ctx = [int(x) for x in rng.integers(1, 3000, size=37)]
    cache, dq, step = make(d, ctx, seed=7)
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    _, ref = oracle_scores(cache, dq)
    check_scores(step.scores.cpu().numpy(), ref, ctx)


def test_scores_max_rows(d):
    """The largest row count the one-row scan takes (4096 requests, one row each): its row
    table in LDS grows to 16 KB, and the key-balanced split spreads many short rows over
    the waves."""
    rng = np.random.default_rng(8)
    ctx = [int(x) for x in rng.integers(1, 200, size=4096)]
    cache, dq, step = make(d, ctx, seed=8)
    step.scores.fill_(float("nan"))
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    got = step.scores.cpu().numpy()
    _, ref = oracle_scores(cache, dq)
    check_scores(got, ref, ctx)
    for r, L in enumerate(ctx):
        assert np.isnan(got[r, L:]).all(), f"row {r} written past its length"


# ------------------------------------------------------------------- top-k

def gpu_topk(d, scores, row_len, k):
    s = torch.as_tensor(scores).cuda().contiguous()
    rl = torch.as_tensor(np.asarray(row_len, np.int32)).cuda()
    idx = torch.full((s.shape[0], k), -9, dtype=torch.int32, device="cuda")
    ws = torch.empty(d.dsa_topk_workspace_size(s.shape[0], s.shape[1], k), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d.dsa_topk(s, rl, k, idx, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return idx.cpu().numpy()


@pytest.mark.parametrize("k", [2048, 1, 7, 4096])
def test_topk_bitexact_random(d, k):
    rng = np.random.default_rng(k)
    lens = [0, 1, 5, 2047, 2048, 2049, 4096, 12288, 12289, 20000, 65536, 131072]
    ld = max(lens) + 3
    s = np.full((len(lens), ld), np.nan, np.float32)
    for r, L in enumerate(lens):
        s[r, :L] = rng.standard_normal(L).astype(np.float32) * 0.7 + 2.5
    log(f"[topk] k={k} lens={lens}")
    got = gpu_topk(d, s, lens, k)
    ref = oracle.topk(np.nan_to_num(s, nan=0.0), lens, k)
    assert np.array_equal(got, ref)


def test_topk_ties_signs_and_fallback(d):
    rng = np.random.default_rng(11)
    rows = []
    L = 50000
    rows.append(np.full(L, 1.5, np.float32))                      # all equal: candidate overflow -> exact fallback
    r = np.zeros(L, np.float32); r[::3] = -0.0; rows.append(r)    # zeros of both signs
    r = rng.standard_normal(L).astype(np.float32); rows.append(r)  # negative scores
    r = np.round(rng.standard_normal(L) * 4).astype(np.float32); rows.append(r)  # heavy ties at the threshold
    r = np.sort(rng.standard_normal(L)).astype(np.float32); rows.append(r)        # sorted: a biased sample
    r = np.zeros(L, np.float32); r[-3000:] = 1.0; rows.append(r)                 # all mass in the tail
    r = np.zeros(L, np.float32); r[7] = 2.0; rows.append(r)
    s = np.stack(rows)
    got = gpu_topk(d, s, [L] * len(rows), 2048)
    ref = oracle.topk(s, [L] * len(rows), 2048)
    assert np.array_equal(got, ref)
    assert got[0].tolist() == list(range(2048))


def test_topk_row_len_shorter_than_ld(d):
    rng = np.random.default_rng(12)
    s = rng.standard_normal((6, 40000)).astype(np.float32)
    lens = [40000, 39999, 12290, 3000, 2048, 100]
    assert np.array_equal(gpu_topk(d, s, lens, 2048), oracle.topk(s, lens, 2048))


def test_topk_clustered_slice_overflow(d):
    """Top scores packed into one 8192-score slice, so that slice's candidate list
    overflows and is filtered again from the scores; other rows spread the top scores over
    a few neighbouring slices, or over far-apart single tokens."""
    rng = np.random.default_rng(13)
    L = 131072
    s = rng.standard_normal((3, L)).astype(np.float32)
    s[0, 16384:16384 + 7000] = 10.0                      # ties at the threshold, one slice
    s[0, rng.choice(np.arange(16384, 23384), 20, replace=False)] = 11.0
    s[1, 40000:52000] += 6.0
    s[2, ::977] += 8.0
    log("[topk] clustered rows")
    got = gpu_topk(d, s, [L] * 3, 2048)
    assert np.array_equal(got, oracle.topk(s, [L] * 3, 2048))


def test_topk_lists_longer_than_their_share(d):
    """Rows of 2^20 scores (128 slices): finalize reads the first 64 entries of every slice's
    candidate list in its first round trip and fetches the entries past 64 afterwards.  With
    k = 4096 most lists are longer than 64; in row 1 two lists (first and last slice) hold
    thousands of entries each, so the entries past 64 take several batches; row 2 has an
    overflowed slice (re-filtered from the scores) next to a long list."""
    rng = np.random.default_rng(15)
    L = 1 << 20
    s = rng.standard_normal((3, L)).astype(np.float32)
    s[1, :3000] += 3.0
    s[1, -3000:] += 3.0
    s[2, 500000:509000] = 9.0
    s[2, :200] += 4.0
    log("[topk] 3 rows of 2^20, k=4096")
    got = gpu_topk(d, s, [L, L, L - 5], 4096)
    assert np.array_equal(got, oracle.topk(s, [L, L, L - 5], 4096))


def test_topk_rows_past_512_slices(d):
    """Rows of more than 512 slices, up to the largest ld the entry point takes (1024 slices
    of 8192 scores): finalize's speculative share of every candidate list drops to 8 entries
    so that one round trip still covers every slice.  The 5M-score row (both k) and the
    8M-score row at k = 1000 take the candidate path; the 8M row at k = 2048 holds more
    candidates than LDS and is selected from the whole row."""
    rng = np.random.default_rng(16)
    ld = 1024 * 8192
    lens = [5_000_000, ld]
    s = np.zeros((2, ld), np.float32)
    for r, L in enumerate(lens):
        s[r, :L] = rng.standard_normal(L).astype(np.float32)
    for k in (2048, 1000):
        log(f"[topk] rows of {lens} scores, k={k}")
        got = gpu_topk(d, s, lens, k)
        assert np.array_equal(got, oracle.topk(s, lens, k))


def test_topk_many_rows_and_long_rows(d):
    """Batches that take the separate sample launch: many rows, and rows over 256K long."""
    rng = np.random.default_rng(14)
    s = (rng.standard_normal((80, 20000)) * 0.5 + 1.0).astype(np.float32)
    lens = [int(x) for x in rng.integers(12289, 20001, 80)]
    lens[3], lens[5] = 20000, 100
    log("[topk] 80 rows")
    assert np.array_equal(gpu_topk(d, s, lens, 2048), oracle.topk(s, lens, 2048))
    L = 300_000
    s = rng.standard_normal((2, L)).astype(np.float32)
    log("[topk] 2 rows of 300000")
    assert np.array_equal(gpu_topk(d, s, [L, L - 77], 2048), oracle.topk(s, [L, L - 77], 2048))


# ------------------------------------------------------------------- attention

def random_sets(rng, ctx, k, drop=0.0):
    idx = np.full((len(ctx), k), -1, np.int32)
    for r, L in enumerate(ctx):
        n = min(k, L)
        sel = np.sort(rng.choice(L, n, replace=False)).astype(np.int32)
        if drop:
            sel = sel[rng.random(n) >= drop]
        idx[r, :len(sel)] = sel
    return idx


@pytest.mark.parametrize("lat_fmt,heads", [(0, 12), (1, 12), (0, 20), (1, 128)])
def test_mla_decode_matches_oracle(d, lat_fmt, heads):
    ctx = [5000, 2048, 300, 1, 4096]
    cache, dq, step = make(d, ctx, key_fmt=lat_fmt, lat_fmt=lat_fmt, seed=20 + heads, heads=heads, spare_rows=3)
    rng = np.random.default_rng(heads)
    idx = random_sets(rng, ctx, 2048, drop=0.1)
    step.resolve()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, dq.q_mla, 0, None, np.arange(len(ctx), dtype=np.int32), heads,
                                     dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


def test_mla_empty_single_and_duplicates(d):
    ctx = [400, 400, 400]
    cache, dq, step = make(d, ctx, seed=31)
    idx = np.full((3, 2048), -1, np.int32)
    idx[1, 100] = 77                        # one token: out = v, lse = z
    idx[2, :5] = 9                          # the same token five times: out = v, lse = z + ln 5
    step.resolve()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, dq.q_mla, 0, None, np.arange(3, dtype=np.int32), 12, dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)
    assert np.isneginf(step.lse[0].cpu().numpy()).all() and (step.out[0].float() == 0).all()


def test_mla_flags_out_of_range_index(d):
    ctx = [500, 300]
    cache, dq, step = make(d, ctx, seed=32)
    rng = np.random.default_rng(3)
    idx = random_sets(rng, ctx, 2048)
    bad = idx.copy()
    bad[1, 3] = 300          # == ctx_len: skipped and flagged
    step.resolve()
    step.idx.copy_(torch.from_numpy(bad))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) & d.DSA_DEVERR_INDEX
    clean = bad.copy()
    clean[1, 3] = -1
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, clean, dq.q_mla, 0, None, np.arange(2, dtype=np.int32), 12, dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


@pytest.mark.parametrize("lat_fmt", [0, 1])
def test_mla_large_batch_matches_oracle_and_small_batches(d, lat_fmt):
    """80 rows x 9 token splits (k = 1100 in 128-token splits, the last one short): 720
    workgroups, more than run at once.  Every row matches the oracle, and rows run again in a
    three-row batch give the same bits."""
    rng = np.random.default_rng(70 + lat_fmt)
    ctx = [int(x) for x in rng.integers(1200, 3000, size=80)]
    k = 1100
    cache, dq, step = make(d, ctx, key_fmt=lat_fmt, lat_fmt=lat_fmt, seed=71 + lat_fmt, k=k, spare_rows=4)
    idx = random_sets(rng, ctx, k, drop=0.05)
    step.resolve()
    step.idx.copy_(torch.from_numpy(idx))
    step.attend()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    ref_o, ref_l = oracle.sparse_mla(oc, idx, dq.q_mla, 0, None, np.arange(len(ctx), dtype=np.int32), 12,
                                     dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)
    rows = [0, 41, 79]
    sel = torch.tensor(rows, device="cuda")
    sub = W.PagedCache(**{**cache.__dict__, "block_table": cache.block_table[sel].contiguous(),
                          "n_pages": cache.n_pages[sel].contiguous(), "ctx_len": cache.ctx_len[sel].contiguous()})
    s3 = d.DecodeStep(sub, dq.q_idx[sel].contiguous(), dq.w[sel].contiguous(), dq.q_mla[sel].contiguous(),
                      dq.sm_scale, k=k)
    s3.resolve()
    s3.idx.copy_(torch.from_numpy(idx[rows]))
    s3.attend()
    torch.cuda.synchronize()
    assert int(s3.err.item()) == 0
    for i, r in enumerate(rows):
        assert torch.equal(s3.out[i].view(torch.int16), step.out[r].view(torch.int16)), f"row {r}"
        assert torch.equal(s3.lse[i], step.lse[r]), f"row {r}"


# ------------------------------------------------------------------- the chain

def run_chain_and_check(d, cache, dq, step, k=2048):
    step.scores.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    ctx = cache.ctx_len.cpu().numpy()
    got_s = step.scores.cpu().numpy()
    oc, ref_s = oracle_scores(cache, dq)
    check_scores(got_s, ref_s, ctx)
    got_idx = step.idx.cpu().numpy()
    # the selection kernel alone: bit-exact on the GPU's own scores
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s), ctx, k))
    # the chain: equal to the oracle's selection up to the tie window
    topk_set_ok(ref_s, oracle.topk(np.nan_to_num(ref_s), ctx, k), got_idx, ctx, k)
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, dq.q_mla, 0, None, np.arange(cache.n_req, dtype=np.int32),
                                     dq.q_mla.shape[1], dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


def test_chain_tiny_decode_workload(d):
    """B=1, L=4096, 64-token pages behind a permuted table, 64 poison rows, 12 heads, top-2048."""
    w = W.WORKLOADS[0]
    cache, dq, step = make(d, W.workload_ctx(0), key_fmt=0, lat_fmt=0, seed=0, heads=w["heads"],
                           spare_rows=w["spare_rows"])
    run_chain_and_check(d, cache, dq, step)


@pytest.mark.parametrize("fmt", [0, 1])
def test_chain_ragged_batch(d, fmt):
    ctx = [1, 64, 2048, 2049, 5000, 13000, 9000]
    cache, dq, step = make(d, ctx, key_fmt=fmt, lat_fmt=fmt, seed=40 + fmt, spare_rows=9)
    run_chain_and_check(d, cache, dq, step)


@pytest.mark.parametrize("fmt", [0, 1])
def test_chain_largest_k(d, fmt):
    """k = 4096, the largest the entry points take: 32 token splits per decode row and a
    combine over 32 partial results; rows shorter than k keep every token."""
    ctx = [20000, 4096, 4095, 9000, 1]
    cache, dq, step = make(d, ctx, key_fmt=fmt, lat_fmt=fmt, seed=45 + fmt, spare_rows=5, k=4096)
    run_chain_and_check(d, cache, dq, step, k=4096)


def test_determinism_and_batch_invariance(d):
    ctx = [3000, 20000, 700]
    cache, dq, step = make(d, ctx, seed=50, spare_rows=4)
    step.run()
    torch.cuda.synchronize()
    first = [t.clone() for t in (step.scores, step.idx, step.out, step.lse)]
    step.run()
    torch.cuda.synchronize()
    # bit patterns (NaN-safe); scores only where written (past row_len the buffer is untouched
    # and may hold anything, NaN included)
    for r, L in enumerate(ctx):
        assert torch.equal(first[0][r, :L].view(torch.int32), step.scores[r, :L].view(torch.int32)), f"row {r}"
    for a, b in zip(first[1:], (step.idx, step.out, step.lse)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    # request 1 alone: same pool, a one-row block table
    solo = W.PagedCache(**{**cache.__dict__, "block_table": cache.block_table[1:2].contiguous(),
                           "n_pages": cache.n_pages[1:2].contiguous(), "ctx_len": cache.ctx_len[1:2].contiguous()})
    s1 = d.DecodeStep(solo, dq.q_idx[1:2].contiguous(), dq.w[1:2].contiguous(), dq.q_mla[1:2].contiguous(),
                      dq.sm_scale)
    s1.run()
    torch.cuda.synchronize()
    L = ctx[1]
    assert torch.equal(s1.scores[0, :L], first[0][1, :L])
    assert torch.equal(s1.idx[0], first[1][1])
    assert torch.equal(s1.out[0].view(torch.int16), first[2][1].view(torch.int16))
    assert torch.equal(s1.lse[0], first[3][1])
