"""Pins for the oracle's top-k and its sparse MLA, plus the pages' byte model.

Top-k: brute force (k rounds of argmax with the lower-index tie rule) on
tiny inputs, and the selection invariants.
Attention: with k >= L it must equal dense softmax attention, computed here
as a textbook fp64 logits matrix from an independent decode (torch's
float8_e4m3fn); k = 1, identical rows, sm_scale = 0 and an empty set have
closed forms; the order of idx does not matter.
Byte model (page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持", section
"K3.1 Pro 中的稀疏注意力"; page "vLLM Adds Day-0 Support for Moonshot AI's
Kimi K3.1 Pro", section "Sparse attention targets long-context costs"):
DSA reads L*132 + 2048*576 bytes against dense MLA's L*576, about 23% at
long context.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.helpers import bf16_bits, torch_e4m3_values

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")))


def brute_topk(s, k):
    s = list(map(float, s))
    taken = []
    for _ in range(min(k, len(s))):
        best = None
        for t, v in enumerate(s):
            if t in taken:
                continue
            if best is None or v > s[best]:   # strict: an equal later index never wins
                best = t
        taken.append(best)
    return sorted(taken)


@pytest.mark.parametrize("seed", range(6))
def test_topk_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, k = 37, 9
    vals = rng.integers(-3, 4, size=(4, L)).astype(np.float32)   # many ties on purpose
    vals[1] = np.float32(rng.standard_normal(L))
    vals[2] = 0.0
    vals[2, ::5] = -0.0                                            # -0 ties with +0
    vals[3, 10:] = 7.0
    got = oracle.topk(vals, np.full(4, L, np.int32), k)
    for r in range(4):
        assert got[r].tolist() == brute_topk(vals[r], k)


def test_topk_short_rows_and_padding():
    s = np.arange(12, dtype=np.float32)[None, :].repeat(3, 0)
    got = oracle.topk(s, np.array([12, 3, 0], np.int32), 5)
    assert got[0].tolist() == [7, 8, 9, 10, 11]
    assert got[1].tolist() == [0, 1, 2, -1, -1]
    assert got[2].tolist() == [-1] * 5


def test_topk_invariants_random():
    rng = np.random.default_rng(3)
    L, k = 5000, 2048
    s = rng.standard_normal((3, L)).astype(np.float32)
    rl = np.array([5000, 2048, 4000], np.int32)
    got = oracle.topk(s, rl, k)
    for r in range(3):
        n = min(k, rl[r])
        sel = got[r, :n]
        assert len(set(sel)) == n and (np.diff(sel) > 0).all() and (sel < rl[r]).all()
        rest = np.setdiff1d(np.arange(rl[r]), sel)
        if len(rest):
            assert s[r, sel].min() >= s[r, rest].max()


# ---------------------------------------------------------------- attention

def small_cache(L, lat_fmt=0, seed=0):
    return W.build_cache([L], key_fmt=lat_fmt, lat_fmt=lat_fmt, seed=seed, spare_rows=3)


def dense_reference(cache, q_bits, sm_scale):
    """Textbook dense MLA in fp64 with latents decoded independently (FP8 only)."""
    lp = cache.layout
    L = int(cache.ctx_len[0])
    pool = cache.pool.numpy()
    bt = cache.block_table.numpy()[0]
    codes = np.stack([pool[bt[t // 64], (t % 64) * 576:(t % 64) * 576 + 576] for t in range(L)])
    kv = torch_e4m3_values(codes) * cache.kv_scale                  # [L, 576]
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().numpy()[0]  # [H, 576]
    logits = sm_scale * (q @ kv.T)                                 # [H, L]
    lse = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
    p = np.exp(logits - lse[:, None])
    return p @ kv[:, :512], lse


def run_mla(cache, idx, q_bits, H, sm_scale):
    oc = oracle.OracleCache(cache)
    return oracle.sparse_mla(oc, np.asarray(idx, np.int32), q_bits, 0, None, np.zeros(len(idx), np.int32), H,
                             sm_scale)


def test_full_set_equals_dense_mla():
    L, H = 300, 12
    c = small_cache(L, seed=1)
    q = W.decode_queries(1, H, seed=1)
    qb = bf16_bits(q.q_mla.float().numpy())
    idx = np.arange(2048, dtype=np.int32)
    idx[L:] = -1
    out, lse = run_mla(c, idx[None], qb, H, q.sm_scale)
    ref_o, ref_l = dense_reference(c, qb, q.sm_scale)
    assert np.allclose(out[0], ref_o, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse[0], ref_l, rtol=1e-12, atol=1e-12)


def test_single_token_and_identical_rows():
    L, H = 200, 4
    c = small_cache(L, seed=2)
    oc = oracle.OracleCache(c)
    q = W.decode_queries(1, H, seed=2)
    qb = bf16_bits(q.q_mla.float().numpy())
    qd = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    t = 77
    row = oc.bt[0, t // 64]
    kv = oracle.latent_decode(0, oc.pool[row][(t % 64) * 576:][:576], c.kv_scale)
    out, lse = run_mla(c, np.array([[t]]), qb, H, q.sm_scale)
    assert np.allclose(out[0], np.tile(kv[:512], (H, 1)), rtol=1e-13)
    assert np.allclose(lse[0], q.sm_scale * (qd @ kv), rtol=1e-13)
    # the same token listed k times: o = v, lse = z + ln k
    out5, lse5 = run_mla(c, np.array([[t] * 5 + [-1] * 3]), qb, H, q.sm_scale)
    assert np.allclose(out5[0], out[0], rtol=1e-12)
    assert np.allclose(lse5[0], lse[0] + math.log(5), rtol=1e-12)


def test_zero_softmax_scale_is_mean():
    L, H = 150, 2
    c = small_cache(L, lat_fmt=1, seed=3)
    oc = oracle.OracleCache(c)
    q = W.decode_queries(1, H, seed=3)
    qb = bf16_bits(q.q_mla.float().numpy())
    sel = np.array([3, 10, 64, 149, 100])
    out, lse = run_mla(c, sel[None], qb, H, 0.0)
    kvs = []
    for t in sel:
        row = oc.bt[0, t // 64]
        kvs.append(oracle.latent_decode(1, oc.pool[row][(t % 64) * 352:][:352], c.kv_scale))
    mean = np.mean(np.stack(kvs), 0)[:512]
    assert np.allclose(out[0], np.tile(mean, (H, 1)), rtol=1e-12, atol=1e-15)
    assert np.allclose(lse[0], math.log(5))


def test_order_and_empty_set():
    L, H = 400, 3
    c = small_cache(L, seed=4)
    q = W.decode_queries(1, H, seed=4)
    qb = bf16_bits(q.q_mla.float().numpy())
    idx = np.random.default_rng(0).choice(L, 64, replace=False).astype(np.int32)
    o1, l1 = run_mla(c, idx[None], qb, H, q.sm_scale)
    o2, l2 = run_mla(c, idx[::-1].copy()[None], qb, H, q.sm_scale)
    assert np.allclose(o1, o2, rtol=1e-12) and np.allclose(l1, l2, rtol=1e-13)
    oe, le = run_mla(c, np.full((1, 8), -1, np.int32), qb, H, q.sm_scale)
    assert (oe == 0).all() and np.isneginf(le).all()


def test_out_of_range_index_is_an_error():
    c = small_cache(100, seed=5)
    q = W.decode_queries(1, 2, seed=5)
    with pytest.raises(ValueError):
        run_mla(c, np.array([[5, 100]]), bf16_bits(q.q_mla.float().numpy()), 2, q.sm_scale)


# ---------------------------------------------------------------- byte model

def dsa_bytes(L, k=2048):
    return L * 132 + min(k, L) * 576


def test_byte_model_ratios():
    # about 23% of dense at long context, about a quarter in the TL;DR
    assert round(dsa_bytes(2 ** 20) / (2 ** 20 * 576), 4) == 0.2311
    assert round(dsa_bytes(131072) / (131072 * 576), 4) == 0.2448
    assert round(dsa_bytes(4096) / (4096 * 576), 3) == 0.729
    assert abs(132 / 576 - GOLD["dsa_over_dense_bytes"]["value"]) < 0.005
    assert abs(dsa_bytes(131072) / (131072 * 576) - GOLD["dsa_over_dense_tldr"]["value"]) < 0.01
    # break-even: L*132 + 2048*576 = L*576  =>  L* = 2048*576/444
    Ls = 2048 * 576 / 444
    assert dsa_bytes(int(Ls) + 1) < (int(Ls) + 1) * 576 and dsa_bytes(int(Ls) - 1) > (int(Ls) - 1) * 576


def test_counted_bytes_match_byte_model():
    L = 3000
    c = small_cache(L, seed=6)
    oc = oracle.OracleCache(c)
    q = W.decode_queries(1, 2, seed=6)
    sc, nb_keys = oracle.indexer_score(oc, bf16_bits(q.q_idx.float().numpy()), 0, None, q.w.numpy(),
                                       np.zeros(1, np.int32), np.array([L], np.int32), count_bytes=True)
    idx = oracle.topk(sc, np.array([L], np.int32), 2048)
    _, _, nb_lat = oracle.sparse_mla(oc, idx, bf16_bits(q.q_mla.float().numpy()), 0, None, np.zeros(1, np.int32),
                                     2, q.sm_scale, count_bytes=True)
    assert int(nb_keys[0] + nb_lat[0]) == dsa_bytes(L) == W.algorithmic_decode_bytes([L], 132, 576)
