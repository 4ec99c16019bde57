"""GPU parity of the exact top-k merge across emulated decode-context-parallel shards
(dsa_dcp_topk) against the oracle, through the C ABI.

Both the kept indices and the resend mask must match the oracle bit for bit: the order
(BF16 score desc, token asc) is total, and a shard is flagged exactly when it kept tokens
back and its last sent candidate is among the k best of all candidates, so both answers are
unique.  Cases: several shard
counts, row lengths that are empty, shorter than k, not multiples of W, and full size;
scores with many BF16 ties; rows whose best tokens sit on one shard (forcing resends);
and the indexer scores of the 32 x 128K decode workload.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.test_oracle_dcp import brute_resend, skew_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def run_dcp(d, scores, row_len, k, n_shards):
    s = torch.as_tensor(np.ascontiguousarray(scores, np.float32), device="cuda")
    rl = torch.as_tensor(np.asarray(row_len, np.int32), device="cuda")
    n = s.shape[0]
    idx = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    rs = torch.full((n,), 0x7777, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(d.dsa_dcp_topk_workspace_size(n, k, n_shards), 16), dtype=torch.uint8, device="cuda")
    print(f"[dcp] rows {n} ld {s.shape[1]} k {k} W {n_shards}", flush=True)
    d.dsa_dcp_topk(s, rl, k, n_shards, idx, ws, rs, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return idx.cpu().numpy(), rs.cpu().numpy().astype(np.uint32)


def check(d, scores, row_len, k, n_shards):
    got_idx, got_rs = run_dcp(d, scores, row_len, k, n_shards)
    ref_idx, ref_rs = oracle.dcp_topk(scores, row_len, k, n_shards)
    for r in range(len(row_len)):
        assert np.array_equal(got_idx[r], ref_idx[r]), (r, n_shards)
    assert np.array_equal(got_rs, ref_rs), (got_rs, ref_rs)
    return got_rs


@pytest.mark.parametrize("n_shards", [1, 2, 3, 8])
def test_random_rows(d, n_shards):
    rng = np.random.default_rng(100 + n_shards)
    L, k = 20000, 2048
    s = rng.standard_normal((8, L)).astype(np.float32)
    s[1] = np.abs(s[1]) * 1e-3                            # a narrow positive range
    s[2] = (np.round(s[2] * 8) / 8).astype(np.float32)    # coarse: many BF16 ties
    s[3, ::5] = 0.0                                       # exact zeros
    rl = np.array([L, 19999, 12345, 2049, 2048, 1000, 0, 8193], np.int32)
    check(d, s, rl, k, n_shards)


def test_small_k_and_short_shards(d):
    rng = np.random.default_rng(5)
    s = rng.standard_normal((6, 700)).astype(np.float32)
    rl = np.array([700, 3, 9, 64, 65, 699], np.int32)
    for k, w in ((1, 8), (7, 3), (50, 8), (64, 5)):
        check(d, s, rl, k, w)


def test_one_shard_holds_the_top_k(d):
    """Every token of one shard outscores the rest, so that shard's c-th candidate is kept
    and it must resend; a second row boosts two shards."""
    L, k, w = 40000, 2048, 8
    rng = np.random.default_rng(9)
    s = rng.standard_normal((3, L)).astype(np.float32)
    t = np.arange(L)
    s[0, t % w == 5] += 10.0
    s[1, (t % w == 1) | (t % w == 6)] += 10.0
    s[2] = np.where(t % w == 2, 1.0, 0.5)                 # ties everywhere: lower token first
    rs = check(d, s, np.array([L, L, L], np.int32), k, w)
    assert rs[0] == 1 << 5 and rs[1] == (1 << 1) | (1 << 6) and rs[2] == 1 << 2


def test_decode_workload_scores(d):
    """The indexer scores of the 32-request, 131,072-token decode workload, W = 8."""
    cfg = 1
    wl = W.WORKLOADS[cfg]
    ctx = W.workload_ctx(cfg)
    cache = W.build_cache(ctx, key_fmt=wl["key_fmt"], lat_fmt=wl["lat_fmt"], seed=cfg, device="cuda",
                          spare_rows=wl["spare_rows"])
    dq = W.decode_queries(len(ctx), wl["heads"], seed=cfg, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=wl["topk"])
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    scores = step.scores.cpu().numpy()
    rl = cache.ctx_len.cpu().numpy()
    check(d, scores, rl, 2048, 8)


@pytest.mark.parametrize("n_shards", [1, 8])
def test_largest_shards(d, n_shards):
    """Shards of 65,536 tokens, the most a shard may hold (ld = 65,536 W): random rows, a row
    of coarse values with many BF16 ties, and a row one token short."""
    rng = np.random.default_rng(110 + n_shards)
    L = 65536 * n_shards
    s = rng.standard_normal((3, L)).astype(np.float32)
    s[1] = (np.round(s[1] * 8) / 8).astype(np.float32)
    check(d, s, np.array([L, L, L - 1], np.int32), 2048, n_shards)


@pytest.mark.parametrize("W_,second,expect", [(8, [1, 2, 3, 4], 0b11111), (3, [1], 0b011)])
def test_skew_rows_flag_what_the_candidates_show(d, W_, second, expect):
    """Shard 0 holds 3000 tokens at 10 (more than k, so the true top-k is all its own), and
    the shards in `second` hold c tokens each at 5: the candidates cannot show that shard 0
    alone fills the top-k, so those shards are flagged too (masks derived by hand in the
    oracle's pins).  A two-tier row of the same kind (shard 0 +20, shard 1 +10 on N(0,1)
    scores) runs beside it."""
    k = 2048
    c = -(-3 * k // (2 * W_))
    L = 4000 * W_
    rows = [skew_row(W_, 3000, second, c, L)]
    t = np.arange(L)
    two = np.random.default_rng(31).standard_normal(L).astype(np.float32)
    two[t % W_ == 0] += 20.0
    two[t % W_ == 1] += 10.0
    rows.append(two)
    s = np.stack(rows)
    rs = check(d, s, np.array([L, L], np.int32), k, W_)
    assert rs[0] == expect
    assert rs[1] == brute_resend(s[1], L, k, W_)
