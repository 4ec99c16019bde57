"""GPU parity of dsa_prefill_select: the prefill indexer on FP8 MFMA with its exact top-k.

The claim under test: idx equals, bit for bit, dsa_topk of dsa_indexer_score's FP8 scores (the
bf16-MFMA GEMM, itself pinned to the oracle in test_gpu_prefill.py), and every FP8-MFMA score
lies within its row bound E_r = delta sum_g U_rg M_bg of that GEMM's score.  The FP8 MFMA's
rounding is measured against the per-token form of the bound, sum_g U_rg A_tg: on the
workload's data, on inputs chosen to stress it (products over many binades, sums that cancel),
and on a hand-built near-worst case (in every group of 8 dims one large product and seven just
below its truncation step), which must land between 1/2 and 1 of the 3.5 * 2^-13 the model
allows (7 * 2^-13 on each head's dot product, halved by the split ReLU: only the |x| half is
scored in FP8).  U, A and M are recomputed from the codes with torch's float8_e4m3fn decode, in fp64.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import workloads as W
from tests.helpers import fp8_key_row, hand_cache, topk_set_ok
from tests.test_gpu_decode import check_scores, log

pytestmark = pytest.mark.gpu

DELTA = 5.5 * 2.0 ** -13       # the library's delta
MODEL = 3.5 * 2.0 ** -13       # the measured truncation model's worst case, halved by the split ReLU


@pytest.fixture(scope="module")
def d(gpu):
    from tests.helpers import ensure_lib
    ensure_lib()
    import long_context_sparse_paged_amd as d
    return d


def key_rows(cache, b):
    """uint8 [ctx_len[b], 132]: request b's key rows, gathered through the block table."""
    lp = cache.layout
    rs, ls, kb, lb = lp["row_stride"], lp["layer_stride"], lp["key_bytes"], lp["lat_bytes"]
    rows = cache.pool.shape[0]
    view = cache.pool.as_strided((rows, W.PAGE, kb), (rs, kb, 1), cache.layer * ls + W.PAGE * lb)
    L = int(cache.ctx_len[b])
    t = torch.arange(L, device=cache.pool.device)
    return view[cache.block_table[b].long()[t // W.PAGE], t % W.PAGE]


def a_tg(cache, b):
    """fp64 [ctx_len[b], 16]: |scale_t| * max over each group of 8 dims of |e4m3 value of k_t|."""
    kr = key_rows(cache, b)
    vals = kr[:, :128].contiguous().view(torch.float8_e4m3fn).double()
    scale = kr[:, 128:132].contiguous().view(torch.float32).double()[:, 0]
    return scale.abs()[:, None] * vals.abs().view(-1, 16, 8).amax(dim=2)


def u_rg(codes, qs, w):
    """fp64 [n_q, 16]: sum_j w_j |qs_j| max over each group of 8 dims of |code value|."""
    v = codes.contiguous().view(torch.float8_e4m3fn).double()
    return (w.double() * qs.double().abs())[:, :, None].mul(v.abs().view(v.shape[0], 32, 16, 8).amax(dim=3)).sum(dim=1)


class Case:
    """One prefill problem run both ways: the four-call FP8 path (dsa_indexer_score's bf16-MFMA
    GEMM + dsa_topk) and dsa_prefill_select."""

    def __init__(self, d, cache, codes, qs, w, q_req, row_len, k=2048):
        dev = "cuda"
        self.cache, self.k = cache, k
        self.codes, self.qs, self.w = codes.to(dev), qs.to(dev).float(), w.to(dev).float()
        self.q_req = torch.as_tensor(q_req, dtype=torch.int32).to(dev)
        self.row_len = torch.as_tensor(row_len, dtype=torch.int32).to(dev)
        n_q = self.row_len.shape[0]
        n_req, mp = cache.block_table.shape
        ld = max(int(cache.ctx_len.max()), 1)
        layout = d.dsa_layout_make(64, cache.layout["n_layers"], 0, 0, cache.layout["extra_row_bytes"])
        lat_off = torch.empty(n_req, mp, dtype=torch.int64, device=dev)
        self.key_off = torch.empty_like(lat_off)
        self.err_ref = torch.zeros(1, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        d.dsa_resolve_pages(layout, cache.layer, cache.block_table, cache.n_pages, cache.pool_rows, lat_off,
                            self.key_off, self.err_ref)
        # reference: bf16-MFMA GEMM scores and dsa_topk
        self.s_ref = torch.full((n_q, ld), float("nan"), device=dev)
        self.idx_ref = torch.full((n_q, k), -7, dtype=torch.int32, device=dev)
        ws = torch.empty(d.dsa_indexer_score_workspace_size(n_q, d.DSA_Q_FP8_E4M3), dtype=torch.uint8, device=dev)
        d.dsa_indexer_score(layout, cache.pool, self.key_off, n_req, self.codes, d.DSA_Q_FP8_E4M3, self.qs, self.w,
                            self.q_req, self.row_len, self.s_ref, ws, self.err_ref)
        wt = torch.empty(max(d.dsa_topk_workspace_size(n_q, ld, k), 16), dtype=torch.uint8, device=dev)
        d.dsa_topk(self.s_ref, self.row_len, k, self.idx_ref, wt, self.err_ref)
        del ws, wt
        # FP8 MFMA + band
        self.s = torch.full((n_q, ld), float("nan"), device=dev)
        self.idx = torch.full((n_q, k), -7, dtype=torch.int32, device=dev)
        self.bound = torch.full((n_q,), float("nan"), device=dev)
        self.ws = torch.empty(d.dsa_prefill_select_workspace_size(n_q, ld, n_req, mp, k), dtype=torch.uint8,
                              device=dev)
        self.layout = layout
        self.d = d
        self.select()
        torch.cuda.synchronize()

    def select(self):
        c = self.cache
        self.d.dsa_prefill_select(self.layout, c.pool, self.key_off, c.block_table.shape[0], c.ctx_len, self.codes,
                                  self.qs, self.w, self.q_req, self.row_len, self.k, self.s, self.idx, self.ws,
                                  self.bound, self.err)

    def check(self, lo=0.0):
        """idx bit-exact; bound = E_r; every score within E_r, and within
        delta sum_g U_rg A_tg, of the GEMM's.  Returns the largest |s^ - s| / sum_g U_rg A_tg."""
        assert int(self.err_ref.item()) == 0 and int(self.err.item()) == 0, (self.err_ref.item(), self.err.item())
        assert torch.equal(self.idx, self.idx_ref)
        u = u_rg(self.codes, self.qs, self.w)
        rl = self.row_len.cpu().numpy()
        qr = self.q_req.cpu().numpy()
        worst = 0.0
        for b in range(self.cache.block_table.shape[0]):
            rows = np.nonzero(qr == b)[0]
            if len(rows) == 0:
                continue
            at = a_tg(self.cache, b)
            mb = at.max(dim=0).values if at.shape[0] else torch.zeros(16, dtype=torch.float64, device=u.device)
            rt = torch.as_tensor(rows, device=u.device)
            want = DELTA * (u[rt] * mb).sum(dim=1)
            got = self.bound[rt].double()
            assert torch.allclose(got, want, rtol=1e-4, atol=0.0), (got[:4], want[:4])
            for r in rows:
                L = int(rl[r])
                if L == 0:
                    continue
                diff = (self.s[r, :L].double() - self.s_ref[r, :L].double()).abs()
                assert bool((diff <= self.bound[r].double()).all())
                denom = at[:L] @ u[r]
                assert bool((diff[denom == 0] == 0).all())
                ratio = diff[denom > 0] / denom[denom > 0]
                if ratio.numel():
                    worst = max(worst, float(ratio.max()))
        log(f"[measure] max |s8 - s_bf16| / sum_g U_rg A_tg = {worst:.3e} = {worst / MODEL:.3f} of the model's "
            f"3.5*2^-13 (delta {DELTA:.3e})")
        assert worst <= MODEL * 1.01
        assert worst >= lo * MODEL
        return worst


def prefill_case(d, prefix, chunk, seed, k=2048, key_hook=None, q_gen=None):
    log(f"[case] prefill select prefix={prefix} chunk={chunk} seed={seed} k={k}")
    cache = W.build_cache([prefix + chunk], seed=seed, device="cuda", spare_rows=2, key_hook=key_hook)
    if q_gen is None:
        pq = W.prefill_queries(prefix, chunk, 12, seed=seed, device="cuda")
        codes, qs, w = pq.q_idx_fp8, pq.q_idx_scale, pq.w
    else:
        codes, qs, w = q_gen(chunk)
    row_len = np.arange(prefix + 1, prefix + chunk + 1, dtype=np.int32)
    return Case(d, cache, codes, qs, w, np.zeros(chunk, np.int32), row_len, k=k)


def test_select_equals_four_call_path(d):
    """Long rows (candidate lists written by the GEMM from a threshold drawn from sampled tiles,
    then the band's passes), several row blocks, a ragged last block."""
    c = prefill_case(d, 30000, 100, seed=11)
    c.check()


def test_select_short_rows_and_keep_all(d):
    """Rows shorter than k keep everything (no band); rows of up to 12288 tokens are selected whole."""
    c = prefill_case(d, 1500, 70, seed=12)
    c.check()
    c = prefill_case(d, 9000, 40, seed=13, k=4096)
    c.check()


def test_select_rows_of_several_requests(d):
    """Rows of one 32-row tile from different requests, interleaved; negative query scales."""
    ctx = [15000, 700, 21000, 5000]
    cache = W.build_cache(ctx, seed=14, device="cuda", spare_rows=2)
    rng = np.random.default_rng(14)
    n_q = 77
    q_req = rng.integers(0, len(ctx), size=n_q).astype(np.int32)
    row_len = np.array([rng.integers(1, ctx[b] + 1) for b in q_req], np.int32)
    row_len[:4] = [ctx[q_req[i]] for i in range(4)]
    q = torch.randn(n_q, 32, 128, generator=torch.Generator().manual_seed(14))
    codes, qs = F.fp8_rowhead_quant(q)
    qs[::5, 3] *= -1.0
    w = torch.rand(n_q, 32, generator=torch.Generator().manual_seed(15)) / 32
    log("[case] prefill select, rows of 4 requests interleaved")
    c = Case(d, cache, codes, qs, w, q_req, row_len)
    c.check()


def heavy_tail_keys(seed):
    def hook(t0, x):
        g = torch.Generator(device=x.device).manual_seed(seed * 1000 + t0)
        return x * torch.exp(1.5 * torch.randn(x.shape, generator=g, device=x.device))
    return hook


def heavy_tail_queries(seed):
    def gen(n):
        g = torch.Generator().manual_seed(seed)
        q = torch.randn(n, 32, 128, generator=g) * torch.exp(1.5 * torch.randn(n, 32, 128, generator=g))
        codes, qs = F.fp8_rowhead_quant(q)
        w = torch.rand(n, 32, generator=g) / 32
        return codes, qs, w
    return gen


def cancelling_keys(seed):
    """Keys whose two 64-dim halves are equal: against queries whose halves are opposite, the
    first K-step's sum is cancelled by the second's, so x is (exactly) 0 but sum|p| is not."""
    def hook(t0, x):
        x = x.clone()
        x[:, 64:] = x[:, :64]
        return x
    return hook


def cancelling_queries(seed):
    def gen(n):
        g = torch.Generator().manual_seed(seed)
        q = torch.randn(n, 32, 128, generator=g)
        q[:, ::2, 64:] = -q[:, ::2, :64]   # even heads cancel, odd heads do not
        codes, qs = F.fp8_rowhead_quant(q)
        w = torch.rand(n, 32, generator=g) / 32
        return codes, qs, w
    return gen


@pytest.mark.parametrize("kind", ["gaussian", "heavy_tail", "cancelling"])
def test_fp8_mfma_rounding_within_bound(d, kind):
    """Measures the FP8 MFMA's rounding against delta A_t B_r (and the exactness of the top-k)
    on the workload's Gaussian data, heavy-tailed codes (products over ~35 binades) and sums
    that cancel."""
    if kind == "gaussian":
        c = prefill_case(d, 40000, 64, seed=21)
    elif kind == "heavy_tail":
        c = prefill_case(d, 40000, 64, seed=22, key_hook=heavy_tail_keys(22), q_gen=heavy_tail_queries(22))
    else:
        c = prefill_case(d, 40000, 64, seed=23, key_hook=cancelling_keys(23), q_gen=cancelling_queries(23))
    c.check()


def test_fp8_mfma_rounding_near_worst_case(d):
    """Hand-built keys (every code 1.0, scales spread over [0.5, 1.5]) against queries whose every
    group of 8 dims holds one 256 and seven 1.875 * 2^-6, just under the 2^-5 truncation step:
    each group loses 7 * 0.94 steps, 0.94 of the model's bound.  (All heads alike and positive,
    so the linear half of the split ReLU is large and exact, and the |x| half carries the loss.)"""
    L = 20000
    rng = np.random.default_rng(71)
    one = torch.full((128,), 1.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = rng.uniform(0.5, 1.5, size=L).astype(np.float32)
    keys = np.stack([fp8_key_row(one, float(sc)) for sc in scales])
    hc = hand_cache(keys, None, perm_seed=71)
    cache = W.PagedCache(layout=hc.layout, layer=0, pool=hc.pool.cuda(), block_table=hc.block_table.cuda(),
                         n_pages=hc.n_pages.cuda(), ctx_len=hc.ctx_len.cuda(), kv_scale=1.0, seed=-1)
    n_q = 48
    v = np.full(128, 1.875 * 2.0 ** -6, np.float32)
    v[::8] = 256.0
    row = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = row.repeat(n_q, 32, 1)
    qs = torch.ones(n_q, 32)
    w = torch.from_numpy(rng.uniform(0.0, 1.0, size=(n_q, 32)).astype(np.float32)) / 32
    log("[case] prefill select, near-worst-case FP8 truncation")
    c = Case(d, cache, codes, qs, w, np.zeros(n_q, np.int32), np.full(n_q, L, np.int32))
    c.check(lo=0.5)


def test_select_band_overflow_rescores_row(d):
    """Thousands of identical keys at the threshold: the band overflows its 2048 entries, the
    row is rescored exactly in place and selected from there (the lower indices win the ties)."""
    V = torch.randn(128, generator=torch.Generator().manual_seed(31))

    def hook(t0, x):
        t = torch.arange(t0, t0 + x.shape[0], device=x.device)
        m = (t % 7 == 3) & (t < 35000)
        x = x.clone()
        x[m] = 3.0 * V.to(x.device)   # one key of about 3x the usual norm, repeated 5000 times
        return x
    c = prefill_case(d, 35000, 33, seed=31, key_hook=hook)
    c.check()
    # the rows whose band overflowed now hold exact scores: bit-equal to the GEMM's
    rl = c.row_len.cpu().numpy()
    n_exact = 0
    for r in range(len(rl)):
        L = int(rl[r])
        if torch.equal(c.s[r, :L].view(torch.int32), c.s_ref[r, :L].view(torch.int32)):
            n_exact += 1
    log(f"[measure] rows rescored in place: {n_exact} of {len(rl)}")
    assert n_exact > 0


def test_select_matches_oracle(d):
    """Against the oracle (fp64 scores): bit-exact on the GEMM's scores is shown above; here the
    selection is within the 1e-5 tie window of the oracle's top-k."""
    c = prefill_case(d, 14000, 40, seed=41)
    c.check()
    oc = oracle.OracleCache(c.cache)
    rl = c.row_len.cpu().numpy()
    ref = oracle.indexer_score(oc, c.codes, 1, c.qs, c.w, c.q_req, rl, ld=c.s.shape[1])
    check_scores(c.s_ref.cpu().numpy(), ref, rl)
    topk_set_ok(ref, oracle.topk(np.nan_to_num(ref), rl, 2048), c.idx.cpu().numpy(), rl, 2048)


def test_select_repeat_is_deterministic(d):
    c = prefill_case(d, 20000, 50, seed=51)
    i0, s0 = c.idx.clone(), c.s.clone()
    c.select()
    torch.cuda.synchronize()
    assert torch.equal(c.idx, i0)
    rl = c.row_len.cpu().numpy()
    for r, L in enumerate(rl):
        assert torch.equal(c.s[r, :L].view(torch.int32), s0[r, :L].view(torch.int32))


def test_select_row_past_ctx_len_flags(d):
    """A row_len past its request's ctx_len flags DSA_DEVERR_ROW_LEN (memory-safe, no trap)."""
    cache = W.build_cache([3000], seed=61, device="cuda", spare_rows=2)
    pq = W.prefill_queries(2990, 10, 12, seed=61, device="cuda")
    rl = pq.row_len.clone()
    rl[3] = 3001
    log("[case] prefill select, row_len past ctx_len")
    dev = "cuda"
    layout = d.dsa_layout_make(64, 1, 0, 0, 0)
    lat_off = torch.empty(1, cache.block_table.shape[1], dtype=torch.int64, device=dev)
    key_off = torch.empty_like(lat_off)
    d.dsa_resolve_pages(layout, 0, cache.block_table, cache.n_pages, cache.pool_rows, lat_off, key_off)
    s = torch.empty(10, 3001, device=dev)
    idx = torch.empty(10, 2048, dtype=torch.int32, device=dev)
    ws = torch.empty(d.dsa_prefill_select_workspace_size(10, 3001, 1, key_off.shape[1], 2048), dtype=torch.uint8,
                     device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    d.dsa_prefill_select(layout, cache.pool, key_off, 1, cache.ctx_len, pq.q_idx_fp8, pq.q_idx_scale, pq.w,
                         pq.q_req, rl, 2048, s, idx, ws, None, err)
    torch.cuda.synchronize()
    assert int(err.item()) & d.DSA_DEVERR_ROW_LEN


def test_halves_equal_select(d):
    """dsa_prefill_score_fp8 then dsa_prefill_topk_band on one workspace: the same scores, bound
    and indices as dsa_prefill_select, bit for bit."""
    c = prefill_case(d, 26000, 45, seed=81)
    c.check()
    cache = c.cache
    s2 = torch.full_like(c.s, float("nan"))
    i2 = torch.full_like(c.idx, -7)
    b2 = torch.full_like(c.bound, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty_like(c.ws)
    n_req = cache.block_table.shape[0]
    d.dsa_prefill_score_fp8(c.layout, cache.pool, c.key_off, n_req, cache.ctx_len, c.codes, c.qs, c.w, c.q_req,
                            c.row_len, c.k, s2, ws, b2, err)
    d.dsa_prefill_topk_band(c.layout, cache.pool, c.key_off, n_req, c.q_req, c.row_len, c.k, s2, i2, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(i2, c.idx)
    assert torch.equal(b2.view(torch.int32), c.bound.view(torch.int32))
    rl = c.row_len.cpu().numpy()
    for r, L in enumerate(rl):
        assert torch.equal(s2[r, :L].view(torch.int32), c.s[r, :L].view(torch.int32))


def test_select_long_rows_sample_and_collect(d):
    """Rows past 2^18 tokens: the GEMM does not write candidate lists and the band top-k samples
    and collects from the score matrix instead; the same exactness."""
    c = prefill_case(d, 290000, 40, seed=91)
    c.check()


@pytest.mark.parametrize("k", [1, 7, 4096])
def test_select_k_extremes_long_rows(d, k):
    """k = 1, 7 and 4096 on rows long enough for the GEMM-written candidate lists."""
    c = prefill_case(d, 24000, 35, seed=100 + k, k=k)
    c.check()


def test_score_parts_equal_score_half(d):
    """dsa_prefill_prepare_fp8 then dsa_prefill_gemm_fp8 (then the band top-k): the same as the
    one call, bit for bit."""
    c = prefill_case(d, 27000, 36, seed=82)
    cache = c.cache
    s2 = torch.full_like(c.s, float("nan"))
    i2 = torch.full_like(c.idx, -7)
    b2 = torch.full_like(c.bound, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty_like(c.ws)
    n_req = cache.block_table.shape[0]
    args = (c.layout, cache.pool, c.key_off, n_req, cache.ctx_len, c.codes, c.qs, c.w, c.q_req, c.row_len, c.k, s2, ws,
            b2, err)
    d.dsa_prefill_prepare_fp8(*args)
    d.dsa_prefill_gemm_fp8(*args)
    d.dsa_prefill_topk_band(c.layout, cache.pool, c.key_off, n_req, c.q_req, c.row_len, c.k, s2, i2, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(i2, c.idx)
    assert torch.equal(b2.view(torch.int32), c.bound.view(torch.int32))
    for r, L in enumerate(c.row_len.cpu().numpy()):
        assert torch.equal(s2[r, :L].view(torch.int32), c.s[r, :L].view(torch.int32))
