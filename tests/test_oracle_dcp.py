"""Pins for the oracle of the exact top-k merge across decode-context-parallel shards.

Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持", section "流量减少 10× 的精确 top-k
合并": shards pick candidates from BF16 scores, the global top-2048 is selected
from the gathered candidates, and a shard that held more of it than it sent
resends.  The oracle returns the protocol's outcome from its definition (one
full sort); these tests pin it to things other than itself:

- BF16 rounding against torch's float32 -> bfloat16 conversion (round to
  nearest even), including constructed halfway cases;
- the kept set against numpy's lexsort on torch-rounded values;
- the kept set does not depend on the number of shards;
- the resend mask: closed forms (one shard never resends; a score that falls
  with the token index spreads the top-k evenly; a row whose best tokens all
  sit on one shard flags exactly that shard) and brute force per shard on
  small rows.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def lexsort_topk(s, length, k):
    """The min(k, len) first tokens of (BF16 value desc, index asc), ascending."""
    v = torch_bf16(s[:length])
    order = np.lexsort((np.arange(length), -v))
    keep = min(k, length)
    out = np.full(k, -1, np.int32)
    out[:keep] = np.sort(order[:keep])
    return out


def brute_resend(s, length, k, n_shards):
    """Shard r flagged iff it holds more than c tokens and its c-th best is kept."""
    c = -(-3 * k // (2 * n_shards))
    v = torch_bf16(s[:length])
    kept = set(np.lexsort((np.arange(length), -v))[:min(k, length)].tolist())
    mask = 0
    for r in range(n_shards):
        toks = sorted(range(r, length, n_shards), key=lambda t: (-v[t], t))
        if len(toks) > c and toks[c - 1] in kept:
            mask |= 1 << r
    return mask


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000),
                        rng.uniform(0, 1, 500)]).astype(np.float32)
    # halfway cases: the 16 dropped bits are exactly 0x8000, kept mantissa odd and even
    bits = (rng.integers(0x0080, 0x7F00, 400).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, bits.view(np.float32), -bits.view(np.float32)])
    ref = torch_bf16(x)
    got = np.array([oracle.bf16_round(float(v)) for v in x])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("quant", [None, 64.0])  # quantised scores: many BF16 ties
def test_kept_set_is_the_bf16_order_topk(quant):
    rng = np.random.default_rng(11)
    L, k = 3000, 256
    s = rng.standard_normal((5, L)).astype(np.float32)
    if quant:
        s = (np.round(s * quant) / quant).astype(np.float32)
    rl = np.array([L, 2999, 257, 256, 0], np.int32)
    idx, _ = oracle.dcp_topk(s, rl, k, 8)
    for r in range(5):
        assert np.array_equal(idx[r], lexsort_topk(s[r], rl[r], k))


def test_kept_set_does_not_depend_on_shards():
    rng = np.random.default_rng(12)
    s = (np.round(rng.standard_normal((3, 4000)) * 32) / 32).astype(np.float32)
    rl = np.array([4000, 1234, 4000], np.int32)
    ref, _ = oracle.dcp_topk(s, rl, 512, 1)
    for w in (2, 3, 5, 8):
        idx, _ = oracle.dcp_topk(s, rl, 512, w)
        assert np.array_equal(idx, ref)


def test_resend_closed_forms():
    k, w = 256, 8
    # one shard sends ceil(1.5 k) > k candidates: never flagged
    s = np.random.default_rng(1).standard_normal((1, 5000)).astype(np.float32)
    assert oracle.dcp_topk(s, np.array([5000], np.int32), k, 1)[1][0] == 0
    # score falling with the index (ties go to the lower index too): the top-k is tokens
    # 0..k-1, k / W per shard < c, so nobody is flagged
    L = 4096
    s = np.arange(L, 0, -1, dtype=np.float32)[None, :]
    idx, rs = oracle.dcp_topk(s, np.array([L], np.int32), k, w)
    assert np.array_equal(idx[0], np.arange(k)) and rs[0] == 0
    # every shard-3 token outscores the rest: the top-k is shard 3's first k tokens, and
    # shard 3's c-th token is among them
    s = np.where(np.arange(L) % w == 3, 1.0, 0.5).astype(np.float32)[None, :]
    idx, rs = oracle.dcp_topk(s, np.array([L], np.int32), k, w)
    assert np.array_equal(idx[0], 3 + w * np.arange(k)) and rs[0] == 1 << 3
    # every shard holds exactly c = 1 token (k = 1, W = 8, three tokens): shards that sent all
    # their tokens are never flagged, even when their last one is kept
    s3 = np.array([[0.1, 0.5, 0.9]], np.float32)
    idx, rs = oracle.dcp_topk(s3, np.array([3], np.int32), 1, w)
    assert idx[0][0] == 2 and rs[0] == 0
    # fewer tokens than k: everything kept, nobody flagged
    idx, rs = oracle.dcp_topk(s, np.array([100], np.int32), k, w)
    assert np.array_equal(idx[0][:100], np.arange(100)) and (idx[0][100:] == -1).all() and rs[0] == 0


@pytest.mark.parametrize("n_shards", [2, 3, 8])
def test_resend_brute_force(n_shards):
    rng = np.random.default_rng(20 + n_shards)
    k = 50  # 1.5 k / W is fractional for W = 8 and 2: c's rounding matters
    rows = []
    for r in range(12):
        L = int(rng.integers(40, 700))
        s = rng.standard_normal(700).astype(np.float32)
        if r % 3 == 1:  # skew: one shard's tokens boosted
            s[(np.arange(700) % n_shards) == r % n_shards] += 2.0
        if r % 3 == 2:  # coarse values: BF16 ties across shards
            s = (np.round(s * 4) / 4).astype(np.float32)
        rows.append((s, L))
    S = np.stack([s for s, _ in rows])
    rl = np.array([L for _, L in rows], np.int32)
    idx, rs = oracle.dcp_topk(S, rl, k, n_shards)
    for r, (s, L) in enumerate(rows):
        assert rs[r] == brute_resend(s, L, k, n_shards), r
        assert np.array_equal(idx[r], lexsort_topk(s, L, k))
    assert rs.any()  # the skewed rows exercise the flag
