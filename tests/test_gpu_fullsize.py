"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

Each workload (the decode configurations at 32 x 128K, 8 x 1M and 64 mixed MXFP4/NVFP4
requests, and the 2048-row prefill chunk on a 153,600-token prefix) is built with the same
seeds and runs the same calls as bench.py: the fused decode path (with MXFP4 queries on the
MXFP4 keys of the mixed workload; that workload also once more with bf16 queries through the
four separate calls) and the prefill step.  Then, for EVERY row of the decode
workloads: the whole row of scores against the oracle (tolerance 1e-5 of each score + 1e-5
of the row's rms), the top-k (bit-exact selection on the GPU's own scores, and within the
1e-5 tie window of the oracle's k-th score), and attention on the GPU's index set (per row,
max|dout| <= 1e-2 max|ref|, |dlse| <= 1e-3).  The prefill chunk is checked the same way on
all 2048 rows for scores and top-k (in eight tests of 256 rows, each a few seconds of oracle
work), and on a seeded sample of 128 rows for attention.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.helpers import topk_set_ok
from tests.test_gpu_decode import check_attention, check_scores, log

pytestmark = pytest.mark.gpu

PREFILL_CHUNK = 256
PREFILL_ATTN_SAMPLE = 128


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def build_step(d, cfg, bench_path=True):
    """bench_path: the decode step bench.py times (the fused calls, MXFP4 queries on MXFP4
    keys); else the four separate calls with bf16 queries."""
    wl = W.WORKLOADS[cfg]
    ctx = W.workload_ctx(cfg)
    log(f"[case] full size {wl['name']}: {len(ctx)} cache requests, {sum(ctx)} tokens, bench path {bench_path}")
    cache = W.build_cache(ctx, key_fmt=wl["key_fmt"], lat_fmt=wl["lat_fmt"], seed=cfg, device="cuda",
                          spare_rows=wl["spare_rows"])
    if wl["kind"] == "decode":
        qs = W.decode_queries(len(ctx), wl["heads"], seed=cfg, device="cuda")
        if bench_path:
            q_fmt = d.DSA_Q_MXFP4 if wl["key_fmt"] == 1 else d.DSA_Q_BF16
            qi = qs.q_idx_mxfp4 if q_fmt == d.DSA_Q_MXFP4 else qs.q_idx
            step = d.FusedDecodeStep(cache, qi, qs.w, qs.q_mla, qs.sm_scale, k=wl["topk"], q_fmt=q_fmt)
        else:
            step = d.DecodeStep(cache, qs.q_idx, qs.w, qs.q_mla, qs.sm_scale, k=wl["topk"])
    else:
        qs = W.prefill_queries(wl["prefix"], wl["chunk"], wl["heads"], seed=cfg, device="cuda")
        step = d.PrefillStep(cache, qs, k=wl["topk"], q_fmt=d.DSA_Q_FP8_E4M3)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    return wl, ctx, cache, qs, step


@pytest.mark.parametrize("cfg,bench_path", [(1, True), (2, True), (3, True), (3, False)])
def test_full_size_decode_every_row(d, cfg, bench_path):
    wl, ctx, cache, dq, step = build_step(d, cfg, bench_path)
    k, n = wl["topk"], len(ctx)
    oc = oracle.OracleCache(cache)
    rl = np.asarray(ctx, np.int32)
    req = np.arange(n, dtype=np.int32)
    ld = int(step.scores.shape[1])
    got_s = step.scores.cpu().numpy()
    got_idx = step.idx.cpu().numpy()
    if bench_path:  # physical rows: the block table's mapping of the kept tokens
        bt = cache.block_table.cpu().numpy()
        want = np.where(got_idx >= 0, bt[req[:, None], np.maximum(got_idx, 0) >> 6] * 64 + (got_idx & 63), -1)
        assert np.array_equal(step.phys.cpu().numpy(), want)
    log(f"[rows] {wl['name']}: oracle scores of all {n} rows")
    ref_s = oracle.indexer_score(oc, step.q_idx, step.q_fmt, None, dq.w, req, rl, ld=ld)
    check_scores(got_s, ref_s, ctx)
    log(f"[rows] {wl['name']}: top-k of all {n} rows")
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s), rl, k))
    topk_set_ok(ref_s, oracle.topk(ref_s, rl, k), got_idx, ctx, k)
    log(f"[rows] {wl['name']}: attention of all {n} rows")
    ref_o, ref_l = oracle.sparse_mla(oc, got_idx, dq.q_mla, 0, None, req, wl["heads"], dq.sm_scale)
    check_attention(step.out, step.lse, ref_o, ref_l)


@pytest.fixture(scope="module")
def prefill(d):
    wl, ctx, cache, pq, step = build_step(d, 4)
    host = dict(scores=step.scores.cpu().numpy(), idx=step.idx.cpu().numpy(),
                row_len=pq.row_len.cpu().numpy().astype(np.int32), q_req=pq.q_req.cpu().numpy())
    return wl, cache, pq, step, oracle.OracleCache(cache), host


@pytest.mark.parametrize("chunk", range(2048 // PREFILL_CHUNK))
def test_full_size_prefill_scores_and_topk(prefill, chunk):
    """Rows [256 chunk, 256 chunk + 256) of the 2048-row prefill chunk: whole score rows, and
    the top-k bit-exact on the GPU's scores and within the tie window of the oracle's."""
    wl, cache, pq, step, oc, h = prefill
    k = wl["topk"]
    rows = slice(chunk * PREFILL_CHUNK, (chunk + 1) * PREFILL_CHUNK)
    rl = h["row_len"][rows]
    ld = int(rl.max())
    log(f"[rows] prefill rows {rows.start}..{rows.stop - 1}, lengths {rl.min()}..{rl.max()}")
    ref_s = oracle.indexer_score(oc, pq.q_idx_fp8[rows], 1, pq.q_idx_scale[rows], pq.w[rows], h["q_req"][rows], rl,
                                 ld=ld)
    got_s = h["scores"][rows, :ld]
    check_scores(got_s, ref_s, rl)
    got_idx = h["idx"][rows]
    assert np.array_equal(got_idx, oracle.topk(np.nan_to_num(got_s), rl, k))
    topk_set_ok(ref_s, oracle.topk(ref_s, rl, k), got_idx, rl, k)


def test_full_size_prefill_select_every_row(d, prefill):
    """The prefill step bench.py times: the indexer on FP8 MFMA with the band top-k
    (PrefillSelectStep) on the same inputs.  For every one of the 2048 rows: the indices equal
    the bf16-GEMM path's bit for bit (which the tests above pin to the oracle), every FP8
    score lies within the row's reported bound of the bf16 GEMM's score, and the attention
    output is the same."""
    import torch
    wl, cache, pq, step, oc, h = prefill
    log("[case] full size prefill, FP8 select path on every row")
    sel = d.PrefillSelectStep(cache, pq, k=wl["topk"])
    sel.run()
    torch.cuda.synchronize()
    assert int(sel.err.item()) == 0
    assert np.array_equal(sel.idx.cpu().numpy(), h["idx"])
    rl = h["row_len"]
    bound = sel.bound.double()
    for r0 in range(0, len(rl), 128):
        L = int(rl[r0 + 127])
        a = sel.scores[r0:r0 + 128, :L].double()
        b = step.scores[r0:r0 + 128, :L].double()
        mask = torch.arange(L, device=a.device)[None, :] < torch.from_numpy(rl[r0:r0 + 128]).to(a.device)[:, None]
        diff = torch.where(mask, (a - b).abs(), torch.zeros_like(a))
        assert bool((diff <= bound[r0:r0 + 128, None]).all()), f"rows {r0}.."
    assert torch.equal(sel.out.view(torch.int16), step.out.view(torch.int16))
    assert torch.equal(sel.lse.view(torch.int32), step.lse.view(torch.int32))


def test_full_size_prefill_attention_sample(prefill):
    """Attention of a seeded sample of 128 of the 2048 prefill rows (a sample: the other rows
    run the same kernel on the same launch)."""
    wl, cache, pq, step, oc, h = prefill
    rows = np.sort(np.random.default_rng(2048).choice(2048, PREFILL_ATTN_SAMPLE, replace=False))
    rows[0], rows[-1] = 0, 2047
    log(f"[rows] prefill attention on {len(rows)} sampled rows")
    ref_o, ref_l = oracle.sparse_mla(oc, h["idx"][rows], pq.q_mla_fp8[rows], 1, pq.q_mla_scale[rows],
                                     h["q_req"][rows], wl["heads"], pq.sm_scale)
    check_attention(step.out[rows], step.lse[rows], ref_o, ref_l)


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
