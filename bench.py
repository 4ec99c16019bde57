"""Benchmark of the DSA hot path on one MI355X.

Default workload: one decode layer-step (indexer scan, top-2048 and sparse MLA, through
the fused path: dsa_indexer_select, whose scan finds the pages through the block table and
whose top-k emits physical rows, then dsa_sparse_mla_decode_phys) for 32 requests at
131,072 tokens of context each, FP8 index keys
(132 B/token) and FP8 latents (576 B/token) in a block-packed pool of 65,536
rows, 12 query heads (one TP8 GPU's share).  Inputs are seeded, synthetic and
resident in HBM before timing starts.

Timing: W untimed warmup steps, then K timed steps between device
synchronisations.  A 512 MiB elementwise pass (16-B loads and stores) runs before
every step, outside its HIP events, so that no step finds the previous step's
latents or scores in the 256 MB Infinity Cache.  ms_per_step is the mean of one
event pair around the whole step; wall_ms_per_step is the bracketed wall time
including the scrubs.  stage_us then times each stage on its own (scrub, earlier
stages untimed, one event pair around the stage); the roofline uses the indexer
scan's figure from there.

Metric: algorithmic bytes of the layer-step (sum_b L_b*132 + min(2048, L_b)*576)
divided by the step time, in GB/s, against the 8 TB/s HBM peak.  The roofline
object is the indexer scan (the dominant kernel): its key bytes per launch over
its own mean launch time.  cpu_baseline is the CPU oracle on a bounded sample of
the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|mixed|long|prefill|verify]

--workload mixed (64 requests, MXFP4 index keys, NVFP4 latents) scores the keys against the
indexer query quantised to MXFP4 on native FP4 MFMA; bf16_query_us_per_step times the same
step with the bf16 query.

--workload verify is speculative verification on the same 32 x 131,072-token cache: 8 query
rows per request (DSpark's 7 draft tokens), the indexer reading each key page once for all
8 rows (dsa_indexer_score_verify); its roofline is the bf16 MFMA peak, because 8 rows of
32 x 128 products per 132-byte key outrun HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0

WORKLOADS = {"decode": 1, "long": 2, "mixed": 3, "prefill": 4, "verify": 5}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_paged_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_src, workload):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it still matches the source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(*kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import importlib.util
    # build.py by path: importing it through the package would first load the library
    spec = importlib.util.spec_from_file_location("long_context_sparse_paged_amd_build",
                                                  os.path.join(ROOT, "long_context_sparse_paged_amd", "build.py"))
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)
    B.ensure_built()
    import long_context_sparse_paged_amd as d
    from synth import workloads as W

    cfg_id = WORKLOADS[args.workload]
    wl = W.WORKLOADS[cfg_id]
    ctx = W.workload_ctx(cfg_id)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = wl["topk"]
    t0 = time.time()
    log(f"[bench] building workload {wl['name']} (seed {cfg_id}) on {torch.cuda.get_device_name(0)}")
    cache = W.build_cache(ctx, key_fmt=wl["key_fmt"], lat_fmt=wl["lat_fmt"], seed=cfg_id, device=dev,
                          spare_rows=wl["spare_rows"])
    kb, lb = cache.layout["key_bytes"], cache.layout["lat_bytes"]
    four_call = None
    bf16_query = None
    q_fmt = d.DSA_Q_BF16
    if wl["kind"] == "decode":
        dq = W.decode_queries(len(ctx), wl["heads"], seed=cfg_id, device=dev)
        # MXFP4 keys: the indexer query quantised to MXFP4 and scored on native FP4 MFMA
        q_fmt = d.DSA_Q_MXFP4 if wl["key_fmt"] == 1 else d.DSA_Q_BF16
        qi = dq.q_idx_mxfp4 if q_fmt == d.DSA_Q_MXFP4 else dq.q_idx
        step = d.FusedDecodeStep(cache, qi, dq.w, dq.q_mla, dq.sm_scale, k=k, q_fmt=q_fmt)
        four_call = d.DecodeStep(cache, qi, dq.w, dq.q_mla, dq.sm_scale, k=k, q_fmt=q_fmt)
        if q_fmt == d.DSA_Q_MXFP4:  # for comparison: the same keys scored against the bf16 query
            bf16_query = d.FusedDecodeStep(cache, dq.q_idx, dq.w, dq.q_mla, dq.sm_scale, k=k)
    elif wl["kind"] == "verify":
        vq = W.verify_queries(ctx, wl["rows"], wl["heads"], seed=cfg_id, device=dev)
        step = d.VerifyStep(cache, vq, k=k)
    else:
        pq = W.prefill_queries(wl["prefix"], wl["chunk"], wl["heads"], seed=cfg_id, device=dev)
        # the indexer on FP8 MFMA with the exact band top-k; for comparison the same step with
        # the bf16-MFMA indexer GEMM and the plain top-k (identical indices)
        step = d.PrefillSelectStep(cache, pq, k=k)
        four_call = d.PrefillStep(cache, pq, k=k, q_fmt=d.DSA_Q_FP8_E4M3)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; pool {cache.pool.numel() / 1e9:.2f} GB")

    # cache scrub between steps: a plain elementwise pass (16-B vector loads and stores) over
    # 512 MiB, which evicts the 256 MB MALL; it also serves as the copy of known size that
    # scales the HBM traffic counters
    scrub_src = torch.zeros(1 << 27, dtype=torch.float32, device=dev)
    scrub_dst = torch.empty_like(scrub_src)

    def scrub():
        torch.neg(scrub_src, out=scrub_dst)
    if wl["kind"] == "decode":
        # fused path: dsa_indexer_select (its halves are the score and top-k stages) then
        # attention over physical rows
        stages = [("score", step.score), ("topk", step.topk), ("attend", step.attend)]
        run_step = step.run
    elif wl["kind"] == "prefill":
        # the score half in its two parts, so that "score" is the FP8 GEMM alone
        stages = [("resolve", step.resolve), ("prepare", step.prepare), ("score", step.gemm), ("topk", step.topk),
                  ("attend", step.attend)]
    else:
        stages = [("resolve", step.resolve), ("score", step.score), ("topk", step.topk), ("attend", step.attend)]
    if wl["kind"] != "decode":
        def run_step():
            for _, fn in stages:
                fn()

    for _ in range(args.warmup):
        scrub()
        run_step()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0, "device error flag set"

    # (1) the step: one event pair around the four stages (events between stages would add
    # their own gaps to the step)
    evs = []
    torch.cuda.synchronize()
    tw = time.time()
    for _ in range(args.steps):
        scrub()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run_step()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.time() - tw
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # (2) each stage on its own, for attribution and the roofline: after a scrub, the stages
    # before it run untimed (so its inputs sit where the step leaves them), then an event pair
    # brackets just this stage
    per_stage = {}
    for i, (name, fn) in enumerate(stages):
        evs_i = []
        for _ in range(args.steps):
            scrub()
            for _, g in stages[:i]:
                g()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs_i.append((a, b))
        torch.cuda.synchronize()
        per_stage[name] = float(np.mean([a.elapsed_time(b) for a, b in evs_i]))
    assert int(step.err.item()) == 0, "device error flag set"
    dcp = dcp_merge_timing(d, step, wl, scrub, args.steps) if wl["kind"] == "decode" else None
    four_call_ms = None
    if four_call is not None:  # the same step through the four separate calls, for comparison
        evs_f = []
        for i in range(args.steps + 1):
            scrub()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            four_call.run()
            b.record()
            evs_f.append((a, b))
        torch.cuda.synchronize()
        four_call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs_f[1:]]))
        assert torch.equal(four_call.idx, step.idx), "fused/FP8 and four-call top-k differ"
    bf16_query_ms = None
    if bf16_query is not None:
        evs_q = []
        for i in range(args.steps + 1):
            scrub()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            bf16_query.run()
            b.record()
            evs_q.append((a, b))
        torch.cuda.synchronize()
        bf16_query_ms = float(np.mean([a.elapsed_time(b) for a, b in evs_q[1:]]))

    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "scaling": "weak", "vs_baseline": None,
           "data": "synthetic (seeded; N(0,1) keys/latents/queries quantised to the cache formats)"}
    if wl["kind"] == "decode":
        alg = W.algorithmic_decode_bytes(ctx, kb, lb, k)
        key_bytes = sum(ctx) * kb
        gbs = alg / (step_ms * 1e-3) / 1e9
        score_ms = per_stage["score"]
        ach = key_bytes / (score_ms * 1e-3) / 1e9
        traffic = counter_traffic(["indexer_scan.hip", "dsa_device.hpp"], args.workload)
        out.update({
            "metric": "us/layer-step & HBM GB/s (frac of peak), DSA decode 128K ctx batch 32, one MI355X"
            if cfg_id == 1 else f"us/layer-step & HBM GB/s, DSA decode ({wl['name']}), one MI355X",
            "value": round(gbs, 1), "unit": "GB/s", "higher_is_better": True,
            "ms_per_step": round(step_ms, 4), "us_per_layer_step": round(step_ms * 1e3, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "wall_ms_per_step": round(wall / args.steps * 1e3, 3),
            "algorithmic_bytes": alg, "dtype": "bf16",
            "config": {"workload": wl["name"], "batch": len(ctx), "ctx_total": int(sum(ctx)),
                       "ctx_max": int(max(ctx)), "heads": wl["heads"], "topk": k,
                       "key_format": ["fp8_e4m3+fp32 scale (132 B)", "mxfp4 (68 B)"][wl["key_fmt"]],
                       "latent_format": ["fp8_e4m3 (576 B)", "nvfp4 (352 B)"][wl["lat_fmt"]], "page_tokens": 64,
                       "pool_rows": cache.pool_rows, "scrub_between_steps_bytes": 4 * scrub_src.numel()},
            "stage_us": {n: round(v * 1e3, 2) for n, v in per_stage.items()},
            "path": "fused: dsa_indexer_select (scan via block table, top-k with physical rows)"
                    " -> dsa_sparse_mla_decode_phys",
            "four_call_us_per_step": round(four_call_ms * 1e3, 1),
            "query_format": "mxfp4 (native FP4 MFMA scoring)" if q_fmt == d.DSA_Q_MXFP4 else "bf16",
            "bf16_query_us_per_step": None if bf16_query_ms is None else round(bf16_query_ms * 1e3, 1),
            "dcp_merge": dcp,
            "roofline": {"kernel": "indexer_scan (dsa_indexer_score_pages: pages via the block table)",
                         "bound": "hbm",
                         "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": key_bytes,
                         "traffic": traffic},
        })
    elif wl["kind"] == "verify":
        m = wl["rows"]
        alg = W.algorithmic_verify_bytes(ctx, m, kb, lb, k)
        key_bytes = sum(ctx) * kb
        rl = vq.row_len.cpu().numpy().astype(np.int64)
        flop_idx = int(rl.sum()) * 32 * 128 * 2
        gbs = alg / (step_ms * 1e-3) / 1e9
        score_ms = per_stage["score"]
        tf = flop_idx / (score_ms * 1e-3) / 1e12
        out.update({
            "metric": f"us/layer-step & HBM GB/s, DSA speculative-verify decode ({wl['name']}), one MI355X",
            "value": round(gbs, 1), "unit": "GB/s", "higher_is_better": True,
            "ms_per_step": round(step_ms, 4), "us_per_layer_step": round(step_ms * 1e3, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "wall_ms_per_step": round(wall / args.steps * 1e3, 3),
            "algorithmic_bytes": alg, "dtype": "bf16",
            "config": {"workload": wl["name"], "batch": len(ctx), "rows_per_request": m, "ctx_total": int(sum(ctx)),
                       "heads": wl["heads"], "topk": k, "key_format": "fp8_e4m3+fp32 scale (132 B)",
                       "latent_format": "fp8_e4m3 (576 B)", "page_tokens": 64, "pool_rows": cache.pool_rows,
                       "scrub_between_steps_bytes": 4 * scrub_src.numel()},
            "stage_us": {n: round(v * 1e3, 2) for n, v in per_stage.items()},
            "roofline": {"kernel": "indexer_verify (dsa_indexer_score_verify, bf16 MFMA)", "bound": "mfma",
                         "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flop_per_launch": flop_idx,
                         "key_bytes_per_launch": key_bytes,
                         "key_gbs": round(key_bytes / (score_ms * 1e-3) / 1e9, 1),
                         "traffic": counter_traffic(DOMINANT["verify"][1], args.workload)},
        })
    else:
        rl = pq.row_len.cpu().numpy().astype(np.int64)
        pairs = int(rl.sum())
        flop_idx = pairs * 32 * 128 * 2
        flop_mla = 2 * pq.n_q * wl["heads"] * k * (576 + 512)
        score_ms = per_stage["score"]
        tf = flop_idx / (score_ms * 1e-3) / 1e12
        traffic = counter_traffic(DOMINANT["prefill"][1], args.workload)
        bound = step.bound.double()
        out.update({
            "metric": "us/layer-step & TFLOP/s (frac of MFMA peak), DSA prefill 2K chunk on 150K prefix, one MI355X",
            "value": round((flop_idx + flop_mla) / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "higher_is_better": True, "ms_per_step": round(step_ms, 4), "us_per_layer_step": round(step_ms * 1e3, 1),
            "wall_ms_per_step": round(wall / args.steps * 1e3, 3), "dtype": "fp8 (indexer) / bf16 (attention)",
            "config": {"workload": wl["name"], "rows": pq.n_q, "prefix": wl["prefix"], "heads": wl["heads"],
                       "topk": k, "scored_pairs": pairs, "query_format": "fp8_e4m3 + fp32 scale per (row, head)"},
            "stage_us": {n: round(v * 1e3, 2) for n, v in per_stage.items()},
            "path": "dsa_prefill_score_fp8 (FP8 MFMA) + dsa_prefill_topk_band (exact: band rescored on bf16 MFMA)"
                    " -> dsa_sparse_mla_prefill",
            "four_call_us_per_step": round(four_call_ms * 1e3, 1),
            "four_call_path": "dsa_indexer_score (bf16 MFMA GEMM) + dsa_topk -> dsa_sparse_mla_prefill",
            "row_bound_mean": round(float(bound.mean()), 5),
            "roofline": {"kernel": "indexer_gemm_fp8 (dsa_prefill_gemm_fp8: e4m3 x e4m3 MFMA, with the band "
                                   "top-k's candidate lists)", "bound": "mfma",
                         "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP8_PEAK_TFLOPS, 4), "flop_per_launch": flop_idx, "traffic": traffic},
        })

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cache, step, wl, ctx, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def dcp_merge_timing(d, step, wl, scrub, steps, n_shards=8):
    """The exact top-k merge across n_shards emulated decode-context-parallel shards
    (dsa_dcp_topk) on the step's scores: its time per launch set (HIP events, after a
    scrub), the candidate bytes one row puts on the wire against a merge that sends every
    shard's full top-k as (fp32 score, int32 id), and the rows that needed a resend."""
    import numpy as np
    import torch
    n, ld = step.scores.shape
    k = wl["topk"]
    if ld > 65536 * n_shards:
        return None
    ws = torch.empty(max(d.dsa_dcp_topk_workspace_size(n, k, n_shards), 16), dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, k, dtype=torch.int32, device="cuda")
    rs = torch.zeros(n, dtype=torch.int32, device="cuda")
    step.run()
    evs = []
    for i in range(steps + 1):
        scrub()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        d.dsa_dcp_topk(step.scores, step.row_len, k, n_shards, idx, ws, rs, step.err)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    c = (3 * k + 2 * n_shards - 1) // (2 * n_shards)
    mask = rs.cpu().numpy().astype(np.uint32)
    resent = int(sum(bin(int(m)).count("1") for m in mask))
    sent = n_shards * c * 4
    generic = n_shards * k * 8
    return {"shards": n_shards, "us": round(float(np.mean([a.elapsed_time(b) for a, b in evs[1:]])) * 1e3, 2),
            "candidates_per_shard": c, "candidate_bytes_per_row": sent, "generic_bytes_per_row": generic,
            "traffic_ratio": round(generic / sent, 2), "rows_with_resend": int((mask != 0).sum()),
            "resent_lists": resent}


def cpu_baseline(cache, step, wl, ctx, budget_s):
    """Time the CPU oracle (as it stands) on whole requests / rows of the same workload."""
    import numpy as np

    import oracle
    from synth.workloads import algorithmic_verify_bytes as W_verify_bytes
    t0 = time.time()
    oc = oracle.OracleCache(cache)
    log(f"[bench] host copy for the oracle: {time.time() - t0:.1f}s")
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    kb, lb = cache.layout["key_bytes"], cache.layout["lat_bytes"]
    k = wl["topk"]
    spent, done_bytes, done_units, t_score, t_topk, t_mla = 0.0, 0, 0, 0.0, 0.0, 0.0
    if wl["kind"] == "decode":
        q_idx = step.q_idx.cpu()
        w = step.w.cpu()
        q_mla = step.q_mla.cpu()
        for b in range(len(ctx)):
            L = ctx[b]
            a = time.time()
            s = oracle.indexer_score(oc, q_idx[b:b + 1], step.q_fmt, None, w[b:b + 1], np.array([b], np.int32),
                                     np.array([L], np.int32))
            t1 = time.time()
            idx = oracle.topk(s, np.array([L], np.int32), k)
            t2 = time.time()
            oracle.sparse_mla(oc, idx, q_mla[b:b + 1], 0, None, np.array([b], np.int32), q_mla.shape[1],
                              step.sm_scale)
            t3 = time.time()
            t_score += t1 - a
            t_topk += t2 - t1
            t_mla += t3 - t2
            spent += t3 - a
            done_bytes += L * kb + min(k, L) * lb
            done_units += 1
            if spent >= budget_s:
                break
        return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{done_units} of {len(ctx)} requests (full score + sort + attention each), "
                          f"{spent:.1f}s: score {t_score:.1f}s, top-k {t_topk:.1f}s, attention {t_mla:.1f}s"}
    if wl["kind"] == "verify":
        vq = step.vq
        m = vq.m
        q_idx, w, q_mla = vq.q_idx.cpu(), vq.w.cpu(), vq.q_mla.cpu()
        rl_all = vq.row_len.cpu().numpy()
        for b in range(len(ctx)):
            rows = np.arange(b * m, (b + 1) * m)
            a = time.time()
            s = oracle.indexer_score(oc, q_idx[b * m:(b + 1) * m], 0, None, w[b * m:(b + 1) * m],
                                     np.full(m, b, np.int32), rl_all[rows])
            t1 = time.time()
            idx = oracle.topk(np.nan_to_num(s, nan=0.0), rl_all[rows], k)
            t2 = time.time()
            oracle.sparse_mla(oc, idx, q_mla[b * m:(b + 1) * m], 0, None, np.full(m, b, np.int32), q_mla.shape[1],
                              vq.sm_scale)
            t3 = time.time()
            t_score += t1 - a
            t_topk += t2 - t1
            t_mla += t3 - t2
            spent += t3 - a
            done_bytes += W_verify_bytes([ctx[b]], m, kb, lb, k)
            done_units += 1
            if spent >= budget_s:
                break
        return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{done_units} of {len(ctx)} requests x {m} rows (full score + sort + attention each), "
                          f"{spent:.1f}s: score {t_score:.1f}s, top-k {t_topk:.1f}s, attention {t_mla:.1f}s"}
    pq = step.pq
    rows = pq.n_q
    order = np.random.default_rng(0).permutation(rows)
    qi, qis, wv = pq.q_idx_fp8.cpu(), pq.q_idx_scale.cpu(), pq.w.cpu()
    qm, qms = pq.q_mla_fp8.cpu(), pq.q_mla_scale.cpu()
    rl_all = pq.row_len.cpu().numpy()
    flops = 0
    for r in order:
        a = time.time()
        L = int(rl_all[r])
        s = oracle.indexer_score(oc, qi[r:r + 1], 1, qis[r:r + 1], wv[r:r + 1], np.zeros(1, np.int32),
                                 np.array([L], np.int32))
        t1 = time.time()
        idx = oracle.topk(s, np.array([L], np.int32), k)
        t2 = time.time()
        oracle.sparse_mla(oc, idx, qm[r:r + 1], 1, qms[r:r + 1], np.zeros(1, np.int32), qm.shape[1], pq.sm_scale)
        t3 = time.time()
        t_score += t1 - a
        t_topk += t2 - t1
        t_mla += t3 - t2
        spent += t3 - a
        flops += L * 32 * 128 * 2 + 2 * qm.shape[1] * min(k, L) * (576 + 512)
        done_units += 1
        if spent >= budget_s:
            break
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done_units} of {rows} rows (seeded random order), {spent:.1f}s: score {t_score:.1f}s, "
                      f"top-k {t_topk:.1f}s, attention {t_mla:.1f}s"}


# --------------------------------------------------------------------------- profile summaries
# These turn rocprofv3 output of `bench.py` runs into the short text files kept under profiles/.

def _short_kernel(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("dsa::", "")
    return name.split("(")[0]


def summarize_stats(argv):
    """--summarize-stats <kernel_stats.csv> <out.txt> <title> <command>: the library's kernels."""
    import csv
    src, dst, title, cmd = argv
    rows = [r for r in csv.DictReader(open(src)) if "dsa::" in r["Name"]]
    out = [f"# rocprofv3 kernel statistics -- {title}", "#", "# command (repository root; TMPDIR=/tmp):",
           f"#   {cmd}", "# rows: the library's kernels only (input generation and cache-scrub copies omitted)", "#",
           f"{'kernel':44s} {'calls':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in rows:
        out.append(f"{_short_kernel(r['Name']):44s} {r['Calls']:>5s} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    open(dst, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


# dominant kernel of each workload and the sources its traffic figures depend on
DOMINANT = {w: ("indexer_scan_kernel", ["indexer_scan.hip", "dsa_device.hpp"]) for w in ("decode", "long", "mixed")}
DOMINANT["prefill"] = ("indexer_gemm_fp8_kernel<2>", ["indexer_gemm_fp8.hip", "dsa_device.hpp"])
DOMINANT["verify"] = ("indexer_verify_kernel", ["indexer_verify.hip", "dsa_device.hpp"])


def summarize_pmc(argv):
    """--summarize-pmc <fetch.csv> <write.csv> <workload> <command>: HBM traffic of the dominant kernel.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel are scaled by what the same
    counters read on the bench's cache-scrub copy, whose bytes are known (512 MiB read and
    written), and written to profiles/traffic_<workload>.json beside a .txt summary."""
    import csv
    from collections import defaultdict
    fetch_csv, write_csv, workload, cmd = argv
    kern, src = DOMINANT[workload]
    copy_bytes = 1 << 29

    def per_dispatch(path, counter):
        val, name = defaultdict(float), {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            val[r["Dispatch_Id"]] += float(r["Counter_Value"])
            name[r["Dispatch_Id"]] = r["Kernel_Name"]
        mine = [v for k, v in val.items() if kern in name[k]]
        # the scrub pass (neg over 512 MiB): the largest dispatch outside the library
        copies = [v for k, v in val.items() if "dsa::" not in name[k] and "neg" in name[k].lower()]
        if not mine or not copies:
            raise SystemExit(f"{path}: no {kern} or copy dispatch with {counter}")
        return sum(mine) / len(mine), max(copies), len(mine)

    f_k, f_c, nf = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_k, w_c, nw = per_dispatch(write_csv, "WRITE_SIZE")
    ff, fw = (copy_bytes / 1024) / f_c, (copy_bytes / 1024) / w_c
    traffic = (f_k * ff + w_k * fw) * 1024
    rec = {"kernel": kern, "workload": workload, "source_sha": source_sha(*src),
           "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1), "dispatches": [nf, nw],
           "copy_fetch_kib": round(f_c, 1), "copy_write_kib": round(w_c, 1), "copy_bytes_each_way": copy_bytes,
           "scale_fetch": round(ff, 4), "scale_write": round(fw, 4), "hbm_bytes_per_launch": int(traffic),
           "command": cmd}
    base = os.path.join(ROOT, "profiles", f"traffic_{workload}")
    json.dump(rec, open(base + ".json", "w"), indent=1)
    lines = [f"# HBM traffic of {kern} on workload '{workload}' (rocprofv3 --pmc)", "#",
             "# commands (repository root; TMPDIR=/tmp), one counter per run:", f"#   {cmd}", "#",
             f"FETCH_SIZE per dispatch        {f_k:14.1f} KiB  (mean of {nf} dispatches)",
             f"WRITE_SIZE per dispatch        {w_k:14.1f} KiB  (mean of {nw} dispatches)",
             f"scrub copy (512 MiB each way)  fetch {f_c:.1f} KiB, write {w_c:.1f} KiB",
             f"scale factors                  fetch {ff:.4f}, write {fw:.4f}",
             f"HBM bytes per launch           {traffic / 1e6:14.2f} MB", f"source sha                     {rec['source_sha']}"]
    # every kernel of the library in the same runs, for the stages around the dominant one
    def all_kernels(path, counter):
        val, name = defaultdict(float), {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter and "dsa::" in r["Kernel_Name"]:
                val[r["Dispatch_Id"]] += float(r["Counter_Value"])
                name[r["Dispatch_Id"]] = _short_kernel(r["Kernel_Name"])
        per = defaultdict(list)
        for k, v in val.items():
            per[name[k]].append(v)
        return {n: sum(v) / len(v) for n, v in per.items()}
    fa, wa = all_kernels(fetch_csv, "FETCH_SIZE"), all_kernels(write_csv, "WRITE_SIZE")
    lines += ["", "# every library kernel of the run: HBM MB per launch (same scale factors)",
              f"{'kernel':44s} {'fetch_MB':>10s} {'write_MB':>10s}"]
    for n in sorted(set(fa) | set(wa), key=lambda n: -(fa.get(n, 0) * ff + wa.get(n, 0) * fw)):
        lines.append(f"{n:44s} {fa.get(n, 0) * ff * 1024 / 1e6:10.2f} {wa.get(n, 0) * fw * 1024 / 1e6:10.2f}")
    open(base + ".txt", "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stats":
        summarize_stats(sys.argv[2:])
    elif len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(sys.argv[2:])
    else:
        main()
