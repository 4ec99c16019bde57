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
  sit on one shard flags exactly that shard), constructed skew rows where the
  protocol's detectable rule flags shards that hold none of the true top-k
  (masks derived by hand), and a brute force of the protocol on small rows;
- the output after the resend round: the plain top-k in the BF16 order.
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
    """The protocol played out shard by shard: each shard sends its c best tokens (all of
    them when it holds at most c); shard r is flagged iff it held more than c and its
    last sent token is among the min(k, len) best of everything sent."""
    c = -(-3 * k // (2 * n_shards))
    v = torch_bf16(s[:length])
    sent, last = [], {}
    for r in range(n_shards):
        toks = list(range(r, length, n_shards))
        toks.sort(key=lambda t: (-v[t], t))
        mine = toks[:c]
        sent += mine
        if len(toks) > c:
            last[r] = mine[-1]
    sent.sort(key=lambda t: (-v[t], t))
    top = set(sent[:min(k, length)])
    return sum(1 << r for r, t in last.items() if t in top)


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


def skew_row(W, n_top, second, n_second, L):
    """Shard 0's first n_top tokens score 10, each shard in `second` has its first n_second
    tokens at 5, everything else scores 1."""
    s = np.ones(L, np.float32)
    t = np.arange(L)
    sh, i = t % W, t // W
    s[(sh == 0) & (i < n_top)] = 10.0
    s[np.isin(sh, second) & (i < n_second)] = 5.0
    return s


@pytest.mark.parametrize("W,second,expect", [(8, [1, 2, 3, 4], 0b11111), (3, [1], 0b011)])
def test_resend_flags_what_the_candidates_show(W, second, expect):
    """k = 2048, c = ceil(1.5 k / W) (384 at W = 8, 1024 at W = 3).  Shard 0 holds 3000
    tokens at 10, more than k, so the true top-k is shard 0's first 2048 tokens alone.  The
    candidates show less: shard 0's c at 10, then c per shard at 5 for shards 1..4 (W = 8:
    4 x 384 = 1536; W = 3: shard 1's 1024, shard 2 holds none at 5).  At W = 8 the union's
    2048 best are 384 + 1536 at 10 and 5 and 128 at 1, so the last sent token of shards 0..4
    is kept and shards 5..7's (at 1) are not: 0b11111.  At W = 3 the union's 2048 best are
    shard 0's 1024 and shard 1's 1024: 0b011.  After the resend the output is shard 0's
    first 2048 tokens either way."""
    k = 2048
    c = -(-3 * k // (2 * W))
    L = 4000 * W
    s = skew_row(W, 3000, second, c, L)[None, :]
    idx, rs = oracle.dcp_topk(s, np.array([L], np.int32), k, W)
    assert rs[0] == expect
    assert rs[0] == brute_resend(s[0], L, k, W)
    assert np.array_equal(idx[0], W * np.arange(k))
