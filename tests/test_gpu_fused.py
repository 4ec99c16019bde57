"""GPU parity of the fused decode path (dsa_indexer_select -> dsa_sparse_mla_decode_phys).

The fused path must give exactly what the four-call path gives -- same scores, same top-k,
same attention, bit for bit -- plus the physical rows of the kept tokens, and both are checked
against the oracle (scores 1e-5 of the score + 1e-5 of the row rms; top-k within the 1e-5 tie
window of the oracle's k-th score; attention max|dout| <= 1e-2 max|ref| per row, |dlse| <=
1e-3).  The row lengths cover every branch of the top-k's last kernel, which writes the
physical rows: rows of at most k tokens, rows of at most 12,288 tokens (selected whole in
LDS), and longer rows selected from the slices' candidate lists; constructed score orders
(ascending, clustered, heavily tied) drive slices whose lists overflow and the full-row
fallback.
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


def run_both(d, cache, dq, k):
    """The fused step and the four-call step on the same inputs."""
    f = d.FusedDecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    u = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    f.phys.fill_(-7)
    f.run()
    u.run()
    torch.cuda.synchronize()
    return f, u


def check_same(f, u, cache, k):
    """Fused == four-call path bit for bit, and phys = the block table's mapping of idx."""
    ctx = cache.ctx_len.cpu().numpy()
    fs, us = f.scores.cpu().numpy(), u.scores.cpu().numpy()
    for r, L in enumerate(ctx):
        assert np.array_equal(fs[r, :L].view(np.uint32), us[r, :L].view(np.uint32)), f"row {r}: scores differ"
    fi, ui = f.idx.cpu().numpy(), u.idx.cpu().numpy()
    assert np.array_equal(fi, ui), "top-k differs from the four-call path"
    bt = cache.block_table.cpu().numpy()
    ph = f.phys.cpu().numpy()
    want = np.where(fi >= 0, bt[np.arange(len(ctx))[:, None], np.maximum(fi, 0) >> 6] * 64 + (fi & 63), -1)
    assert np.array_equal(ph, want), "physical rows"
    assert torch.equal(f.out.view(torch.int16), u.out.view(torch.int16)), "attention output differs"
    assert np.array_equal(f.lse.cpu().numpy().view(np.uint32), u.lse.cpu().numpy().view(np.uint32)), "lse differs"


def check_oracle(f, cache, dq, k, n_heads=12):
    ctx = cache.ctx_len.cpu().numpy()
    oc = oracle.OracleCache(cache)
    req = np.arange(len(ctx), dtype=np.int32)
    ref_s = oracle.indexer_score(oc, dq.q_idx, 0, None, dq.w, req, ctx, ld=int(f.scores.shape[1]))
    got_s = f.scores.cpu().numpy()
    check_scores(got_s, ref_s, ctx)
    got_idx = f.idx.cpu().numpy()
    topk_set_ok(ref_s, oracle.topk(np.nan_to_num(ref_s), ctx, k), got_idx, ctx, k)
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, dq.q_mla, 0, None, req, n_heads, dq.sm_scale)
    check_attention(f.out, f.lse, ref_o, ref_l)


# at k = 2048: rows of <= k tokens (1, 2048), whole rows in LDS (4096, 12288), and rows of 2 to
# 37 slices of 8192 scores
BRANCH_CTX = [1, 2048, 4096, 12288, 12289, 20000, 32000, 40000, 60001, 131072, 300000]


@pytest.mark.parametrize("key_fmt", [0, 1])
def test_fused_matches_four_call_path_and_oracle(d, key_fmt):
    log(f"[case] fused branches key_fmt={key_fmt} ctx={BRANCH_CTX}")
    cache = W.build_cache(BRANCH_CTX, key_fmt=key_fmt, lat_fmt=key_fmt, seed=60 + key_fmt, device="cuda",
                          spare_rows=5, n_layers=2, layer=1)
    dq = W.decode_queries(len(BRANCH_CTX), 12, seed=60 + key_fmt, device="cuda")
    f, u = run_both(d, cache, dq, 2048)
    assert int(f.err.item()) == 0 and int(u.err.item()) == 0
    check_same(f, u, cache, 2048)
    check_oracle(f, cache, dq, 2048)


@pytest.mark.parametrize("k", [1, 7, 4096])
def test_fused_other_k(d, k):
    ctx = [4000, 50000, 131072, 8192, 700000]
    log(f"[case] fused k={k} ctx={ctx}")
    cache = W.build_cache(ctx, seed=70 + k, device="cuda", spare_rows=2)
    dq = W.decode_queries(len(ctx), 12, seed=70 + k, device="cuda")
    f, u = run_both(d, cache, dq, k)
    assert int(f.err.item()) == 0
    check_same(f, u, cache, k)
    check_oracle(f, cache, dq, k)
    # the two halves called one by one give the same as the one call
    idx, phys = f.idx.clone(), f.phys.clone()
    f.idx.fill_(-9)
    f.phys.fill_(-9)
    f.score()
    f.topk()
    torch.cuda.synchronize()
    assert torch.equal(f.idx, idx) and torch.equal(f.phys, phys)


def ordered_cache(ctx, pattern, seed):
    """Keys c_t * V for one shared direction V: every token gets the same e4m3 codes and a
    scale proportional to c_t, so the score order follows c_t (c_t = 0: the zero key)."""
    V = np.random.default_rng(seed).standard_normal(128)
    base = np.concatenate([[0], np.cumsum(ctx)])
    cs = []
    for b, L in enumerate(ctx):
        rng = np.random.default_rng(seed + 1 + b)
        t = np.arange(L, dtype=np.float64)
        if pattern == "ascending":            # the top-k is the last k tokens: 32+ full pages
            c = 1.0 + t / L
        elif pattern == "clustered":          # 20 pages hold every high score, the rest is low
            c = 0.2 + 0.1 * rng.random(L)
            pages = rng.choice((L + 63) // 64, 20, replace=False)
            for p in pages:
                c[64 * p:64 * p + 64] = 2.0 + rng.random(min(64, L - 64 * p))
        elif pattern == "ties":               # 12 levels only: huge ties at the threshold
            c = rng.integers(1, 13, L).astype(np.float64)
        else:                                 # "halfzero": half the keys zero, rest random
            c = np.where(rng.random(L) < 0.5, 0.0, 0.5 + rng.random(L))
        cs.append(c)
    allc = np.concatenate(cs)
    assert base[-1] == allc.shape[0]

    def hook(t0, xk):
        n = xk.shape[0]
        x = allc[t0:t0 + n, None] * V[None, :]
        xk.copy_(torch.from_numpy(x.astype(np.float32)).to(xk.device))
        return xk

    return W.build_cache(ctx, seed=seed, device="cuda", spare_rows=2, key_hook=hook)


@pytest.mark.parametrize("pattern", ["ascending", "clustered", "ties", "halfzero"])
def test_fused_constructed_orders(d, pattern):
    ctx = [131072, 65536 + 17, 20000, 300001]
    log(f"[case] fused order={pattern} ctx={ctx}")
    cache = ordered_cache(ctx, pattern, seed=80 + len(pattern))
    # queries along V's sign pattern keep every head's dot product of one sign
    dq = W.decode_queries(len(ctx), 12, seed=81, device="cuda")
    f, u = run_both(d, cache, dq, 2048)
    assert int(f.err.item()) == 0
    check_same(f, u, cache, 2048)
    check_oracle(f, cache, dq, 2048)


def test_fused_flags_bad_block(d):
    ctx = [3000, 40000]
    log(f"[case] fused bad block ctx={ctx}")
    cache = W.build_cache(ctx, seed=90, device="cuda", spare_rows=2)
    cache.block_table[1, 7] = cache.pool_rows + 3
    dq = W.decode_queries(len(ctx), 12, seed=90, device="cuda")
    f = d.FusedDecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=2048)
    f.run()
    torch.cuda.synchronize()
    assert int(f.err.item()) & d.DSA_DEVERR_BLOCK_RANGE
    ph = f.phys.cpu().numpy()
    ix = f.idx.cpu().numpy()
    # row 0 never touches the bad block: exact as usual
    assert np.array_equal(ph[0][:2048] >= 0, ix[0][:2048] >= 0)
    # no kept token of row 1 maps into the bad block's page
    assert not ((ix[1] >> 6 == 7) & (ph[1] >= 0)).any()
