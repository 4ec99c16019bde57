"""GPU parity of native FP4 scoring: MXFP4 index keys scored against MXFP4 queries on
v_mfma_scale_f32_32x32x64_f8f6f4 (both operands e2m1 with their E8M0 block scales).

The reference is the oracle's score for the decoded MXFP4 query (q_fmt 2), in fp64.  Every
e2m1 x e2m1 product is exact and the products of one 32-element block share one power of
two, so the bars are the fp32 ones of the other decode paths: scores 1e-5 of the score +
1e-5 of the row rms; top-k bit-exact on the GPU's scores and within the 1e-5 tie window of
the oracle's; attention max|dout| <= 1e-2 max|ref| per row, |dlse| <= 1e-3.
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


def fp4_case(d, ctx, seed, k=2048, fused=False, **kw):
    log(f"[case] fp4 ctx={ctx[:6]}{'...' if len(ctx) > 6 else ''} n={len(ctx)} seed={seed} k={k} fused={fused}")
    cache = W.build_cache(ctx, key_fmt=1, lat_fmt=1, seed=seed, device="cuda", **kw)
    dq = W.decode_queries(len(ctx), 12, seed=seed, device="cuda")
    cls = d.FusedDecodeStep if fused else d.DecodeStep
    step = cls(cache, dq.q_idx_mxfp4, dq.w, dq.q_mla, dq.sm_scale, k=k, q_fmt=d.DSA_Q_MXFP4)
    return cache, dq, step


def oracle_fp4_scores(cache, dq, ld):
    oc = oracle.OracleCache(cache)
    rl = cache.ctx_len.cpu().numpy()
    return oc, oracle.indexer_score(oc, dq.q_idx_mxfp4, 2, None, dq.w, np.arange(cache.n_req, dtype=np.int32), rl,
                                    ld=ld)


# ragged lengths: one token, part pages, page edges, many pages, and a row past 2^17
CTX = [1, 63, 64, 65, 1000, 4096, 4097, 20000, 131072, 150001]


def test_fp4_scores_match_oracle(d):
    cache, dq, step = fp4_case(d, CTX, seed=41)
    step.resolve()
    step.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    ld = step.scores.shape[1]
    _, ref = oracle_fp4_scores(cache, dq, ld)
    check_scores(step.scores.cpu().numpy(), ref, cache.ctx_len.cpu().numpy())


def test_fp4_decode_step_matches_oracle(d):
    ctx = [3000, 131072, 40000, 9000]
    cache, dq, step = fp4_case(d, ctx, seed=42)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    ld = step.scores.shape[1]
    oc, ref = oracle_fp4_scores(cache, dq, ld)
    got_s = step.scores.cpu().numpy()
    check_scores(got_s, ref, ctx)
    got_i = step.idx.cpu().numpy()
    # bit-exact on the GPU's own scores, within the tie window on the oracle's
    assert np.array_equal(got_i, oracle.topk(np.nan_to_num(got_s), np.array(ctx, np.int32), 2048))
    topk_set_ok(ref, oracle.topk(np.nan_to_num(ref), np.array(ctx, np.int32), 2048), got_i, ctx, 2048)
    req = np.arange(len(ctx), dtype=np.int32)
    ref_o, ref_l = oracle.sparse_mla(oc, got_i, dq.q_mla, 0, None, req, 12, dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


def test_fp4_fused_path_equals_four_call_path(d):
    ctx = [2048, 70000, 131072, 12288, 500]
    cache, dq, f = fp4_case(d, ctx, seed=43, fused=True, spare_rows=3)
    u = d.DecodeStep(cache, dq.q_idx_mxfp4, dq.w, dq.q_mla, dq.sm_scale, k=2048, q_fmt=d.DSA_Q_MXFP4)
    f.run()
    u.run()
    torch.cuda.synchronize()
    assert int(f.err.item()) == 0 and int(u.err.item()) == 0
    fs, us = f.scores.cpu().numpy(), u.scores.cpu().numpy()
    for r, L in enumerate(ctx):
        assert np.array_equal(fs[r, :L].view(np.uint32), us[r, :L].view(np.uint32)), f"row {r}"
    assert torch.equal(f.idx, u.idx)
    bt = cache.block_table.cpu().numpy()
    fi, ph = f.idx.cpu().numpy(), f.phys.cpu().numpy()
    want = np.where(fi >= 0, bt[np.arange(len(ctx))[:, None], np.maximum(fi, 0) >> 6] * 64 + (fi & 63), -1)
    assert np.array_equal(ph, want)
    assert torch.equal(f.out.view(torch.int16), u.out.view(torch.int16))


def test_fp4_zero_and_tied_keys(d):
    """Edge keys through the FP4 MFMA: all-zero keys score +0; duplicated keys tie exactly and
    the lower index wins."""
    ctx = [5000]
    z = np.zeros(5000, bool)
    z[100:1100] = True                      # zero keys
    dup = np.arange(2000, 5000, 7)          # copies of key 1999
    same = np.zeros(5000, bool)
    same[dup] = True
    same[1999] = True
    V = 2.0 * np.random.default_rng(44).standard_normal(128).astype(np.float32)  # scores high

    def hook(t0, xk):
        x = xk.cpu().numpy()
        idx = np.arange(t0, t0 + x.shape[0])
        x[z[idx]] = 0.0
        x[same[idx]] = V
        xk.copy_(torch.from_numpy(x).to(xk.device))
        return xk

    log("[case] fp4 zero and tied keys")
    cache = W.build_cache(ctx, key_fmt=1, lat_fmt=1, seed=44, device="cuda", key_hook=hook)
    dq = W.decode_queries(1, 12, seed=44, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx_mxfp4, dq.w, dq.q_mla, dq.sm_scale, k=2048, q_fmt=d.DSA_Q_MXFP4)
    step.run()
    torch.cuda.synchronize()
    s = step.scores.cpu().numpy()[0, :5000]
    assert (s[100:1100].view(np.uint32) == 0).all()          # exactly +0
    assert (s[dup].view(np.uint32) == s[1999].view(np.uint32)).all()
    _, ref = oracle_fp4_scores(cache, dq, step.scores.shape[1])
    check_scores(step.scores.cpu().numpy(), ref, ctx)
    got = step.idx.cpu().numpy()
    assert np.array_equal(got, oracle.topk(np.nan_to_num(step.scores.cpu().numpy()), np.array(ctx, np.int32), 2048))
