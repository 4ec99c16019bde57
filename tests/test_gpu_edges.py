"""Edge cases of the whole chain (indexer -> top-k -> attention) on constructed keys, through
both indexer paths: the decode scan (bf16 queries) and the prefill GEMM (FP8 queries).

A shared direction U (128 dims, seeded) shapes queries and keys:
  * "zero"  queries q_j = U + 0.3 n_j for every head.  Six tokens in ten have keys against U
            (every head's dot product < 0: score exactly +0), one in ten is the zero key,
            two are random, one is one of seven duplicated random keys.  Fewer than k tokens
            score above zero, so the k-th score is 0, the tie window is empty and the kept
            zero-score tokens must be exactly the lowest-index ones.
  * "small" head 0 is 0.01 U (+ small noise), heads 1..31 are -U + 0.3 n_j; keys are
            (1 + u/2) U + noise.  Every token scores w_0 * (a small positive dot product)
            while every other head contributes a large negative one: the k-th score is
            about 3000x below sum_j w_j |x_j|, the case where a linear/absolute split of
            the ReLU loses its relative precision.
  * "tie"   as "zero" for the queries; a block of tokens shares one key 4U that outscores
            every random key, and there are more of them than k: the top-k is the lowest k
            indices of that block (the lower index wins ties).
Checks: scores against the oracle (1e-5 of the score + 1e-5 of the row rms; zero scores
exactly zero), the top-k bit-exact on the GPU's scores and within the tie window of the
oracle's (which is empty, hence exact, when the k-th score is 0), the closed-form set of
the "tie" rows, and attention on the GPU's set.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import workloads as W
from tests.helpers import topk_set_ok
from tests.test_gpu_decode import check_attention, check_scores, log

pytestmark = pytest.mark.gpu

K = 2048
U = np.random.default_rng(900).standard_normal(128)


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def key_vectors(kind, L, seed, tie_mod=3):
    """Float keys [L, 128] of one request of the given kind."""
    rng = np.random.default_rng(seed)
    rnd = rng.standard_normal((L, 128))
    t = np.arange(L)
    if kind == "zero":
        x = -U + 0.05 * rnd
        dup = rng.standard_normal((7, 128))
        x[t % 10 == 6] = 0.0
        sel = np.isin(t % 10, [7, 8])
        x[sel] = rnd[sel]
        sel = t % 10 == 9
        x[sel] = dup[(t[sel] // 10) % 7]
    elif kind == "small":
        x = (1.0 + 0.5 * rng.random((L, 1))) * U + 0.05 * rnd
        x[t % 7 == 0] = 1.2 * U + 0.05 * rnd[0]     # duplicates: identical keys, identical scores
    else:  # tie
        x = rnd.copy()
        x[t % 8 < tie_mod] = 4.0 * U
    return x


def query_heads(kind, n_rows, seed):
    """Float indexer queries [n_rows, 32, 128] of the given kind."""
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal((n_rows, 32, 128))
    if kind == "small":
        q = -U + 0.3 * noise
        q[:, 0] = 0.01 * U + 0.003 * noise[:, 0]
    else:
        q = U + 0.3 * noise
    return q


def structured_cache(ctx, kinds, seed, tie_mod=3):
    base = np.concatenate([[0], np.cumsum(ctx)])
    keys = [key_vectors(kd, L, seed + 11 * b, tie_mod) for b, (kd, L) in enumerate(zip(kinds, ctx))]
    allk = np.concatenate(keys).astype(np.float32)

    def hook(t0, xk):
        n = xk.shape[0]
        xk.copy_(torch.from_numpy(allk[t0:t0 + n]).to(xk.device))
        return xk

    assert base[-1] == allk.shape[0]
    return W.build_cache(ctx, seed=seed, device="cuda", spare_rows=3, key_hook=hook)


def check_chain(got_s, ref_s, got_idx, rl, kinds, k=K, tie_rows=None):
    check_scores(got_s, ref_s, rl)
    for r, L in enumerate(rl):
        z = ref_s[r, :L] == 0
        assert (got_s[r, :L][z] == 0).all(), f"row {r}: a zero score came out non-zero"
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s), rl, k))
    ref_idx = oracle.topk(np.nan_to_num(ref_s), rl, k)
    topk_set_ok(ref_s, ref_idx, got_idx, rl, k)
    for r, L in enumerate(rl):
        s = np.sort(ref_s[r, :L])[::-1]
        if L > k and s[k - 1] == 0:          # k-th score 0: the set is exact
            assert (s[:k] > 0).sum() < k
            assert np.array_equal(got_idx[r], ref_idx[r]), f"row {r}: zero-threshold row differs"
    for r, expect in (tie_rows or {}).items():
        assert np.array_equal(got_idx[r], expect), f"row {r}: tie rule"


def test_decode_chain_edge_rows(d):
    kinds = ["zero", "small", "tie", "zero"]
    ctx = [8192, 6000, 8192, 3001]
    log(f"[case] decode edge rows {list(zip(kinds, ctx))}")
    cache = structured_cache(ctx, kinds, seed=501)
    q = np.stack([query_heads(kd, 1, 600 + b)[0] for b, kd in enumerate(kinds)])
    g = torch.Generator().manual_seed(601)
    dq = W.DecodeQueries(q_idx=torch.from_numpy(q).to(torch.bfloat16).cuda(),
                         w=(torch.rand(len(ctx), 32, generator=g) / 32).cuda(),
                         q_mla=torch.randn(len(ctx), 12, 576, generator=g).to(torch.bfloat16).cuda(),
                         sm_scale=float(np.float32(1 / 24)))
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=K)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    rl = np.asarray(ctx, np.int32)
    req = np.arange(len(ctx), dtype=np.int32)
    ref_s = oracle.indexer_score(oc, dq.q_idx, 0, None, dq.w, req, rl, ld=int(step.scores.shape[1]))
    got_s = step.scores.cpu().numpy()
    got_idx = step.idx.cpu().numpy()
    t = np.arange(ctx[2])
    check_chain(got_s, ref_s, got_idx, rl, kinds, tie_rows={2: t[t % 8 < 3][:K].astype(np.int32)})
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, dq.q_mla, 0, None, req, 12, dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


@pytest.mark.parametrize("kind", ["zero", "small", "tie"])
@pytest.mark.parametrize("q_fmt", [1, 0])
def test_prefill_chain_edge_rows(d, kind, q_fmt):
    """A 64-row prefill chunk on a 3000-token prefix, all rows of one kind, through the FP8
    GEMM (q_fmt 1) or the bf16 scan (q_fmt 0).  "tie" uses six tokens in eight at 4U, so
    every row holds more than k of them."""
    P, C, H = 3000, 64, 16
    log(f"[case] prefill edge rows kind={kind} q_fmt={q_fmt}")
    cache = structured_cache([P + C], [kind], seed=700 + len(kind), tie_mod=6)
    q = torch.from_numpy(query_heads(kind, C, 800 + len(kind))).float()
    g = torch.Generator().manual_seed(801)
    qi = q.to(torch.bfloat16)
    qi8, qis = F.fp8_rowhead_quant(qi.float())
    qm = torch.randn(C, H, 576, generator=g).to(torch.bfloat16)
    qm8, qms = F.fp8_rowhead_quant(qm.float())
    pos = torch.arange(P, P + C, dtype=torch.int32)
    pq = W.PrefillQueries(n_q=C, q_req=torch.zeros(C, dtype=torch.int32).cuda(), row_len=(pos + 1).cuda(),
                          q_idx_bf16=qi.cuda(), q_idx_fp8=qi8.cuda(), q_idx_scale=qis.cuda(),
                          w=(torch.rand(C, 32, generator=g) / 32).cuda(), q_mla_bf16=qm.cuda(),
                          q_mla_fp8=qm8.cuda(), q_mla_scale=qms.cuda(), sm_scale=float(np.float32(1 / 24)))
    step = d.PrefillStep(cache, pq, k=K, q_fmt=q_fmt)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    rl = pq.row_len.cpu().numpy()
    req = pq.q_req.cpu().numpy()
    if q_fmt == 1:
        ref_s = oracle.indexer_score(oc, pq.q_idx_fp8, 1, pq.q_idx_scale, pq.w, req, rl, ld=P + C)
    else:
        ref_s = oracle.indexer_score(oc, pq.q_idx_bf16, 0, None, pq.w, req, rl, ld=P + C)
    got_s = step.scores.cpu().numpy()
    got_idx = step.idx.cpu().numpy()
    ties = None
    if kind == "tie":
        t = np.arange(P + C)
        ties = {r: t[t % 8 < 6][:K].astype(np.int32) for r in range(C)}
    check_chain(got_s, ref_s, got_idx, rl, [kind] * C, tie_rows=ties)
    if kind == "zero":   # the construction really gives a zero threshold on every row
        assert all((ref_s[r, :rl[r]] > 0).sum() < K for r in range(C))
    if q_fmt == 1:
        ref_o, ref_l = oracle.sparse_mla(oc, got_idx, pq.q_mla_fp8, 1, pq.q_mla_scale, req, H, pq.sm_scale)
    else:
        ref_o, ref_l = oracle.sparse_mla(oc, got_idx, pq.q_mla_bf16, 0, None, req, H, pq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)
