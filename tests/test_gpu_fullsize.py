"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

Each workload (the decode configurations at 32 x 128K, 8 x 1M and 64 mixed MXFP4/NVFP4
requests, and the 2048-row prefill chunk on a 153,600-token prefix) is built with the same
seeds and runs the same four calls as bench.py.  Sampled rows are then checked against the
oracle: the whole row of scores (tolerance 1e-5 of each score + 1e-5 of the row's rms), the
top-k (bit-exact selection on the GPU's own scores, and within the 1e-5 tie window of the
oracle's k-th score), and attention on the GPU's index set (max|dout| <= 1e-2 max|ref|,
|dlse| <= 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.helpers import topk_set_ok
from tests.test_gpu_decode import check_attention, check_scores, log

pytestmark = pytest.mark.gpu

# rows checked against the oracle, per workload (first, last and a few between)
SAMPLES = {1: [0, 17, 31], 2: [0, 7], 3: [0, 1, 40, 63], 4: [0, 1023, 2047]}


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_step_sampled_rows(d, cfg):
    wl = W.WORKLOADS[cfg]
    ctx = W.workload_ctx(cfg)
    k = wl["topk"]
    log(f"[case] full size {wl['name']}: {len(ctx)} cache requests, {sum(ctx)} tokens")
    cache = W.build_cache(ctx, key_fmt=wl["key_fmt"], lat_fmt=wl["lat_fmt"], seed=cfg, device="cuda",
                          spare_rows=wl["spare_rows"])
    decode = wl["kind"] == "decode"
    if decode:
        dq = W.decode_queries(len(ctx), wl["heads"], seed=cfg, device="cuda")
        step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    else:
        pq = W.prefill_queries(wl["prefix"], wl["chunk"], wl["heads"], seed=cfg, device="cuda")
        step = d.PrefillStep(cache, pq, k=k, q_fmt=d.DSA_Q_FP8_E4M3)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    oc = oracle.OracleCache(cache)
    for r in SAMPLES[cfg]:
        if decode:
            L = int(ctx[r])
            q, fmt, qs, w, req = dq.q_idx[r:r + 1], 0, None, dq.w[r:r + 1], np.array([r], np.int32)
            qm, qms, H, sm = dq.q_mla[r:r + 1], None, wl["heads"], dq.sm_scale
        else:
            L = int(pq.row_len[r].item())
            q, fmt, qs, w = pq.q_idx_fp8[r:r + 1], 1, pq.q_idx_scale[r:r + 1], pq.w[r:r + 1]
            req = pq.q_req[r:r + 1].cpu().numpy()
            qm, qms, H, sm = pq.q_mla_fp8[r:r + 1], pq.q_mla_scale[r:r + 1], wl["heads"], pq.sm_scale
        log(f"[row] {wl['name']} row {r} length {L}")
        ref_s = oracle.indexer_score(oc, q, fmt, qs, w, req, np.array([L], np.int32))
        got_s = step.scores[r:r + 1, :L].cpu().numpy()
        check_scores(got_s, ref_s, [L])
        got_idx = step.idx[r:r + 1].cpu().numpy()
        assert np.array_equal(got_idx, oracle.topk(got_s, np.array([L], np.int32), k))
        topk_set_ok(ref_s, oracle.topk(ref_s, np.array([L], np.int32), k), got_idx, [L], k)
        ref_o, ref_l = oracle.sparse_mla(oc, got_idx, qm, fmt, qms, req, H, sm)
        check_attention(step.out[r:r + 1], step.lse[r:r + 1], ref_o, ref_l)


def test_scans_past_one_offset_batch(d):
    """Both key scans cache their pages' offsets 64 units at a time (one per lane).  With
    9 requests of ~1M tokens a wave of the one-row scan takes 72 pages and a workgroup of the
    verify scan (2 rows per request) 72 tiles, so both refill that cache mid-range: sampled
    rows are checked against the oracle over their whole length."""
    ctx = [1048576 + 37 * i for i in range(9)]
    log(f"[case] offset-cache refill: {len(ctx)} requests, {sum(ctx)} tokens")
    cache = W.build_cache(ctx, key_fmt=0, lat_fmt=0, seed=77, device="cuda")
    dq = W.decode_queries(len(ctx), 12, seed=77, device="cuda")
    step = d.DecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=2048)
    step.resolve()
    step.score()
    vq = W.verify_queries(ctx, 2, 12, seed=78, device="cuda")
    vs = d.VerifyStep(cache, vq, k=2048)
    vs.resolve()
    vs.score()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0 and int(vs.err.item()) == 0
    oc = oracle.OracleCache(cache)
    for r in (0, 8):
        L = ctx[r]
        log(f"[row] one-row scan row {r} length {L}")
        ref = oracle.indexer_score(oc, dq.q_idx[r:r + 1], 0, None, dq.w[r:r + 1], np.array([r], np.int32),
                                   np.array([L], np.int32))
        check_scores(step.scores[r:r + 1, :L].cpu().numpy(), ref, [L])
    for r in (1, 16):
        L = int(vq.row_len[r].item())
        log(f"[row] verify scan row {r} length {L}")
        ref = oracle.indexer_score(oc, vq.q_idx[r:r + 1], 0, None, vq.w[r:r + 1], vq.q_req[r:r + 1].cpu().numpy(),
                                   np.array([L], np.int32))
        check_scores(vs.scores[r:r + 1, :L].cpu().numpy(), ref, [L])
