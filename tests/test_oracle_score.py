"""Pins for the oracle's indexer score.

The pages name the indexer but print no score values, so the score is pinned
by closed forms and special cases that a plausible mistake (dropped weight,
ReLU in the wrong place, scale outside/inside swapped for a negative value,
wrong head or dim index, wrong token address) would break:
  * a hand-computed example,
  * one active head with a unit query: score = ReLU(k[d] * scale) exactly,
  * doubling every key scale doubles every score exactly,
  * ReLU identity: score(q) - score(-q) = sum_j w_j x_j (linear part),
  * linearity in w, non-negativity for w >= 0, zero key -> +0,
  * permuting pool rows together with the block table changes no bit,
  * the FP8 and MXFP4 query modes equal feeding their decoded values.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import workloads as W
from tests.helpers import bf16_bits, fp8_key_row, hand_cache, torch_e4m3_values


def run_score(cache, q_bits, w, q_fmt=0, q_scale=None, row_len=None):
    oc = oracle.OracleCache(cache)
    n_q = q_bits.shape[0]
    rl = np.full(n_q, int(cache.ctx_len[0]), np.int32) if row_len is None else np.asarray(row_len, np.int32)
    return oracle.indexer_score(oc, q_bits, q_fmt, q_scale, np.asarray(w, np.float32),
                                np.zeros(n_q, np.int32), rl)


def test_hand_example():
    # one token: k = [1.0, 2.0, 0, ...] (e4m3 0x38, 0x40), scale 0.5
    # head 0: q = [1, 1]   -> dot 3    -> x = 1.5  -> ReLU 1.5,  w = 0.5 -> 0.75
    # head 1: q = [-1, 0]  -> dot -1   -> x = -0.5 -> ReLU 0,    w = 1   -> 0
    # head 2: q = [0, .25] -> dot 0.5  -> x = 0.25 -> ReLU 0.25, w = 2   -> 0.5
    # score = 1.25
    key = fp8_key_row([0x38, 0x40], 0.5)[None, :]
    q = np.zeros((1, 32, 128), np.float32)
    q[0, 0, :2] = [1, 1]
    q[0, 1, 0] = -1
    q[0, 2, 1] = 0.25
    w = np.zeros((1, 32), np.float32)
    w[0, :3] = [0.5, 1.0, 2.0]
    s = run_score(hand_cache(key, None), bf16_bits(q), w)
    assert s[0, 0] == 1.25


def test_negative_scale_relu_after_scaling():
    # x_j = dot * scale with a negative scale flips which heads pass the ReLU
    key = fp8_key_row([0x38], -2.0)[None, :]
    q = np.zeros((1, 32, 128), np.float32)
    q[0, 0, 0] = 1.0     # dot 1  -> x = -2 -> 0
    q[0, 1, 0] = -1.0    # dot -1 -> x = 2  -> 2
    w = np.zeros((1, 32), np.float32)
    w[0, :2] = [1.0, 3.0]
    s = run_score(hand_cache(key, None), bf16_bits(q), w)
    assert s[0, 0] == 6.0


@pytest.mark.parametrize("d", [0, 5, 64, 127])
def test_unit_query_single_head(d):
    rng = np.random.default_rng(d)
    L = 200
    x = torch.from_numpy(rng.standard_normal((L, 128)).astype(np.float32))
    keys = F.fp8_key_rows(x).numpy()
    q = np.zeros((1, 32, 128), np.float32)
    q[0, 7, d] = 1.0
    w = np.zeros((1, 32), np.float32)
    w[0, 7] = 1.0
    s = run_score(hand_cache(keys, None, perm_seed=3), bf16_bits(q), w)
    kd = torch_e4m3_values(keys[:, d])
    sc = keys[:, 128:132].copy().view(np.float32)[:, 0].astype(np.float64)
    want = np.maximum(kd * sc, 0.0).astype(np.float32)
    assert np.array_equal(s[0, :L], want)


def test_unit_query_mxfp4():
    rng = np.random.default_rng(11)
    L = 100
    keys = F.mxfp4_key_rows(torch.from_numpy(rng.standard_normal((L, 128)).astype(np.float32))).numpy()
    for d in (0, 1, 33, 127):
        q = np.zeros((1, 32, 128), np.float32)
        q[0, 31, d] = 1.0
        w = np.zeros((1, 32), np.float32)
        w[0, 31] = 1.0
        s = run_score(hand_cache(keys, None, key_fmt=1, lat_fmt=1), bf16_bits(q), w)
        nib = (keys[:, d // 2] >> (4 * (d % 2))) & 15
        mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        val = np.where(nib & 8, -1, 1) * mags[nib & 7] * 2.0 ** (keys[:, 64 + d // 32].astype(np.float64) - 127)
        assert np.array_equal(s[0, :L], np.maximum(val, 0).astype(np.float32))


def random_case(L=300, seed=0, key_fmt=0, n_q=2):
    c = W.build_cache([L], key_fmt=key_fmt, lat_fmt=key_fmt, seed=seed, spare_rows=2)
    q = W.decode_queries(n_q, seed=seed)
    return c, bf16_bits(q.q_idx.float().numpy()), q.w.numpy()


def test_scale_doubling_doubles_scores():
    c, q, w = random_case(seed=4)
    s1 = run_score(c, q, w)
    lp = c.layout
    pool = c.pool.clone()
    kv = pool.as_strided((pool.shape[0], 64, 132), (lp["row_stride"], 132, 1), lp["lat_page_bytes"])
    sc = kv[:, :, 128:132].contiguous().view(torch.float32)
    kv[:, :, 128:132] = (sc * 2).view(torch.uint8)
    c2 = W.PagedCache(**{**c.__dict__, "pool": pool})
    s2 = run_score(c2, q, w)
    assert np.array_equal(s2[:, :300], 2 * s1[:, :300])


def test_relu_identity_and_linearity():
    c, q, w = random_case(seed=5)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).float().numpy()
    s_pos = run_score(c, q, w).astype(np.float64)
    s_neg = run_score(c, bf16_bits(-qf), w).astype(np.float64)
    # relu(x) - relu(-x) = x  =>  score(q) - score(-q) = sum_j w_j x_j
    oc = oracle.OracleCache(c)
    lin = np.zeros_like(s_pos)
    for t in range(300):
        row = oc.bt[0, t // 64]
        o = row * oc.layout.row_stride + 64 * 576 + (t % 64) * 132
        k, sc = oracle.key_decode(0, oc.pool.reshape(-1)[o:o + 132])
        lin[:, t] = np.einsum("rj,rjd,d->r", w.astype(np.float64), qf.astype(np.float64), k) * sc
    assert np.allclose(s_pos[:, :300] - s_neg[:, :300], lin[:, :300], rtol=1e-6, atol=1e-6)
    # linearity in w and non-negativity
    w2 = np.roll(w, 3, axis=1)
    s_w2 = run_score(c, q, w2).astype(np.float64)
    s_sum = run_score(c, q, w + w2).astype(np.float64)
    assert np.allclose(s_sum[:, :300], s_pos[:, :300] + s_w2[:, :300], rtol=1e-6)
    assert (s_pos[:, :300] >= 0).all()


def test_zero_key_scores_positive_zero():
    key = fp8_key_row([], 0.0)[None, :].repeat(3, axis=0)
    q = np.random.default_rng(0).standard_normal((1, 32, 128)).astype(np.float32)
    w = np.full((1, 32), 1 / 32, np.float32)
    s = run_score(hand_cache(key, None), bf16_bits(q), w)
    assert (s[0, :3] == 0).all() and not np.signbit(s[0, :3]).any()


def test_page_permutation_invariance():
    c, q, w = random_case(L=520, seed=6)
    s1 = run_score(c, q, w)
    perm = torch.randperm(c.pool_rows, generator=torch.Generator().manual_seed(9))
    inv = torch.argsort(perm)
    pool2 = c.pool[perm]                      # new row i holds old row perm[i]
    bt2 = torch.where(c.block_table >= 0, inv[c.block_table.long().clamp_min(0)].to(torch.int32),
                      c.block_table)
    c2 = W.PagedCache(**{**c.__dict__, "pool": pool2, "block_table": bt2})
    s2 = run_score(c2, q, w)
    assert np.array_equal(s1[:, :520], s2[:, :520])


def test_fp8_query_mode_matches_decoded_bf16():
    """FP8 query mode: code * scale per (row, head) -- same as feeding those values exactly."""
    c, _, w = random_case(L=150, seed=7)
    p = W.prefill_queries(prefix=100, chunk=3, n_heads=12, seed=7)
    s8 = run_score(c, p.q_idx_fp8.numpy(), p.w.numpy(), q_fmt=1, q_scale=p.q_idx_scale.numpy(),
                   row_len=[101, 102, 103])
    # the same query values, exactly, as doubles: a head scale only multiplies
    vals = torch_e4m3_values(p.q_idx_fp8.numpy()) * p.q_idx_scale.numpy()[..., None]
    oc = oracle.OracleCache(c)
    for r in range(3):
        for t in (0, 50, 100 + r):
            row = oc.bt[0, t // 64]
            o = row * oc.layout.row_stride + 64 * 576 + (t % 64) * 132
            k, sc = oracle.key_decode(0, oc.pool.reshape(-1)[o:o + 132])
            x = vals[r] @ k * sc
            want = np.float32(np.sum(p.w.numpy()[r].astype(np.float64) * np.maximum(x, 0)))
            assert abs(s8[r, t] - want) <= 1e-6 * abs(want) + 1e-30
        assert np.isnan(s8[r, 101 + r:]).all()   # causal: nothing written past the position


def mxfp4_values(rows):
    """[..., 68] MXFP4 rows -> [..., 128] float64 values, decoded here from the OCP MX
    definition (e2m1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, sign bit 3, E8M0 bias 127)."""
    rows = np.asarray(rows)
    d = np.arange(128)
    nib = (rows[..., d // 2] >> (4 * (d % 2))) & 15
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return np.where(nib & 8, -1, 1) * mags[nib & 7] * 2.0 ** (rows[..., 64 + d // 32].astype(np.float64) - 127)


def test_mxfp4_query_mode_matches_decoded_bf16():
    """MXFP4 query mode: the 68-byte rows decode to e2m1 x 2^(e-127) -- values that bf16 holds
    exactly, so feeding the decoded values as bf16 must give the same scores bit for bit."""
    c = W.build_cache([300], key_fmt=1, lat_fmt=1, seed=21, spare_rows=2)
    dq = W.decode_queries(2, seed=21)
    q4 = dq.q_idx_mxfp4.numpy()
    vals = mxfp4_values(q4)
    assert np.array_equal(bf16_bits(vals.astype(np.float32)).view(np.uint16).astype(np.uint32) << 16,
                          vals.astype(np.float32).view(np.uint32))  # exact in bf16
    s4 = run_score(c, q4, dq.w.numpy(), q_fmt=2)
    sb = run_score(c, bf16_bits(vals.astype(np.float32)), dq.w.numpy(), q_fmt=0)
    assert np.array_equal(s4.view(np.uint32), sb.view(np.uint32))
    # and the quantised query is close to the bf16 one it came from (MX rounding)
    qb = dq.q_idx.float().numpy()
    assert np.abs(vals - qb).max() <= 0.26 * np.abs(qb).max()


def test_unit_query_mxfp4_query_mode():
    """One nonzero MXFP4 query element (code 1.5 in block 2, scale 2^-3): x = 0.1875 k[d]."""
    rng = np.random.default_rng(12)
    L = 80
    keys = F.mxfp4_key_rows(torch.from_numpy(rng.standard_normal((L, 128)).astype(np.float32))).numpy()
    d = 71                                   # block 2, odd element: high nibble of byte 35
    q4 = np.zeros((1, 32, 68), np.uint8)
    q4[0, 5, 64:68] = 127                    # unit scales elsewhere
    q4[0, 5, 64 + 2] = 124                   # 2^-3
    q4[0, 5, d // 2] = 0x3 << 4              # e2m1 code 3 = 1.5
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = 2.0
    s = run_score(hand_cache(keys, None, key_fmt=1, lat_fmt=1), q4, w, q_fmt=2)
    kd = mxfp4_values(keys)[:, d]
    want = (2.0 * np.maximum(0.1875 * kd, 0.0)).astype(np.float32)
    assert np.array_equal(s[0, :L], want)


def test_bytes_counted_equal_keys_read():
    c, q, w = random_case(L=777, seed=8, key_fmt=1)
    oc = oracle.OracleCache(c)
    _, nb = oracle.indexer_score(oc, q, 0, None, w, np.zeros(2, np.int32), np.array([777, 5], np.int32),
                                 count_bytes=True)
    assert list(nb) == [777 * 68, 5 * 68]
