"""Seeded synthetic workloads for the DSA step (decode batches and a prefill chunk).

Everything here is input construction: random draws, quantisation to the
cache formats (``synth.formats``) and placement of rows into a block-packed
pool behind a random block table.  No part of the method's arithmetic lives
here.

Block-packed pool (one contiguous row per cache block, every DSA layer's pages
in it, after the page titled "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持",
section "面向三种状态的 KV 缓存"):

    row r, layer l:  [latent page: page_size * lat_bytes][key page: page_size * key_bytes]
    layer_stride = align256(page_size*lat_bytes + page_size*key_bytes)
    row_stride   = align256(n_layers*layer_stride + extra_row_bytes)

Unused bytes (spare rows, other layers, slots past a request's length) hold
0xFF, which decodes to NaN in every format used here (e4m3 0xFF, E8M0 0xFF,
fp32 0xFFFFFFFF), so a read of the wrong bytes shows up as a NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import formats as F

PAGE = 64
IDX_HEADS = 32
IDX_DIM = 128
LAT_DIM = 576
V_DIM = 512
POISON = 0xFF


def align256(x: int) -> int:
    return (x + 255) // 256 * 256


def layout_params(key_fmt: int, lat_fmt: int, n_layers: int = 1,
                  page_size: int = PAGE, extra_row_bytes: int = 0) -> dict:
    kb, lb = F.KEY_BYTES[key_fmt], F.LAT_BYTES[lat_fmt]
    layer_stride = align256(page_size * lb + page_size * kb)
    row_stride = align256(n_layers * layer_stride + extra_row_bytes)
    return dict(page_size=page_size, n_layers=n_layers, key_fmt=key_fmt, lat_fmt=lat_fmt,
                key_bytes=kb, lat_bytes=lb, lat_page_bytes=page_size * lb,
                key_page_bytes=page_size * kb, layer_stride=layer_stride,
                extra_row_bytes=extra_row_bytes, row_stride=row_stride)


@dataclass
class PagedCache:
    """One layer's latents and index keys for a batch of requests, in a block-packed pool."""
    layout: dict
    layer: int
    pool: torch.Tensor          # uint8 [pool_rows, row_stride]
    block_table: torch.Tensor   # int32 [n_req, max_pages]  (unused entries = -1)
    n_pages: torch.Tensor       # int32 [n_req]
    ctx_len: torch.Tensor       # int32 [n_req]
    kv_scale: float
    seed: int
    recipe: dict = field(default_factory=dict)

    @property
    def pool_rows(self) -> int:
        return self.pool.shape[0]

    @property
    def n_req(self) -> int:
        return self.block_table.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(rows: int, cols: int, seed: int, device) -> torch.Tensor:
    return torch.randn(rows, cols, generator=_gen(seed, device), device=device, dtype=torch.float32)


def build_cache(ctx_lens, key_fmt: int = 0, lat_fmt: int = 0, seed: int = 0,
                device="cpu", n_layers: int = 1, layer: int = 0, spare_rows: int = 0,
                extra_row_bytes: int = 0, max_pages: int | None = None,
                key_hook=None, chunk_tokens: int = 1 << 18) -> PagedCache:
    """Build a pool holding ``len(ctx_lens)`` requests' keys and latents at ``layer``.

    Keys ~ N(0,1) per dim, quantised per token (FP8: absmax/448 scale; MXFP4:
    OCP MX block scales).  Latents ~ N(0,1), one per-tensor kv_scale =
    absmax/448 over the whole layer.  Pages go to a random permutation of
    the pool's rows; ``spare_rows`` extra rows stay poisoned.
    ``key_hook(t0, x)`` may edit the float keys of tokens t0.. before
    quantisation (tie tests duplicate or zero rows this way).
    """
    ctx = [int(c) for c in ctx_lens]
    lp = layout_params(key_fmt, lat_fmt, n_layers, PAGE, extra_row_bytes)
    pages = [(c + PAGE - 1) // PAGE for c in ctx]
    total_pages = sum(pages)
    mp = max(pages + [1]) if max_pages is None else int(max_pages)
    assert mp >= max(pages + [0])
    pool_rows = total_pages + int(spare_rows)
    rs, ls = lp["row_stride"], lp["layer_stride"]
    kb, lb = lp["key_bytes"], lp["lat_bytes"]

    perm = torch.randperm(pool_rows, generator=_gen(seed * 7919 + 1, device), device=device)
    pool = torch.full((pool_rows, rs), POISON, dtype=torch.uint8, device=device)
    bt = torch.full((len(ctx), mp), -1, dtype=torch.int32, device=device)
    page_base = np.concatenate([[0], np.cumsum(pages)]).astype(np.int64)
    for b, npg in enumerate(pages):
        if npg:
            bt[b, :npg] = perm[page_base[b]:page_base[b] + npg].to(torch.int32)

    lat_view = pool.as_strided((pool_rows, PAGE, lb), (rs, lb, 1), layer * ls)
    key_view = pool.as_strided((pool_rows, PAGE, kb), (rs, kb, 1), layer * ls + PAGE * lb)

    # token t of request b has global number tok_base[b] + t (request-major)
    tok_base = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    n_tok = int(tok_base[-1])
    # map a global token range to (pool row, slot)
    req_of_tok_starts = torch.tensor(tok_base[:-1], device=device)
    page_base_t = torch.tensor(page_base[:-1], device=device)
    ctx_t = torch.tensor(ctx, device=device, dtype=torch.int64)

    def rows_slots(t0: int, t1: int):
        gt = torch.arange(t0, t1, device=device, dtype=torch.int64)
        b = torch.searchsorted(req_of_tok_starts, gt, right=True) - 1
        # skip empty requests sharing a start: searchsorted(right) picks the last start <= gt
        t = gt - req_of_tok_starts[b]
        assert bool((t < ctx_t[b]).all())
        row = perm[page_base_t[b] + t // PAGE]
        return row, t % PAGE

    # latents: pass 1 for the per-tensor absmax, pass 2 to quantise (regenerated from seeds)
    chunks = [(t0, min(n_tok, t0 + chunk_tokens)) for t0 in range(0, n_tok, chunk_tokens)]
    amax = 0.0
    for ci, (t0, t1) in enumerate(chunks):
        amax = max(amax, float(_normal(t1 - t0, LAT_DIM, seed * 1000003 + 2 * ci + 1, device).abs().max()))
    kv_scale = float(np.float32(amax / F.E4M3_MAX)) if amax > 0 else 1.0
    for ci, (t0, t1) in enumerate(chunks):
        row, slot = rows_slots(t0, t1)
        xl = _normal(t1 - t0, LAT_DIM, seed * 1000003 + 2 * ci + 1, device)
        enc = F.fp8_latent_rows(xl, kv_scale) if lat_fmt == 0 else F.nvfp4_latent_rows(xl, kv_scale)
        lat_view[row, slot] = enc
        del xl, enc
        xk = _normal(t1 - t0, IDX_DIM, seed * 1000003 + 2 * ci + 2, device)
        if key_hook is not None:
            xk = key_hook(t0, xk)
        enc = F.fp8_key_rows(xk) if key_fmt == 0 else F.mxfp4_key_rows(xk)
        key_view[row, slot] = enc
        del xk, enc

    return PagedCache(layout=lp, layer=layer, pool=pool, block_table=bt,
                      n_pages=torch.tensor(pages, dtype=torch.int32, device=device),
                      ctx_len=torch.tensor(ctx, dtype=torch.int32, device=device),
                      kv_scale=kv_scale, seed=seed,
                      recipe=dict(ctx=ctx, key_fmt=key_fmt, lat_fmt=lat_fmt, n_layers=n_layers,
                                  layer=layer, spare_rows=spare_rows))


@dataclass
class DecodeQueries:
    q_idx: torch.Tensor   # bf16 [B, 32, 128]
    w: torch.Tensor       # fp32 [B, 32]
    q_mla: torch.Tensor   # bf16 [B, H, 576]
    sm_scale: float
    q_idx_mxfp4: torch.Tensor = None  # uint8 [B, 32, 68]: q_idx quantised to MXFP4 (OCP MX rule)


def decode_queries(n_req: int, n_heads: int = 12, seed: int = 0, device="cpu") -> DecodeQueries:
    """Indexer query bf16 ~ N(0,1), head weights ~ U(0,1)/32, MLA query bf16 ~ N(0,1)."""
    g = _gen(seed * 31337 + 5, device)
    q_idx = torch.randn(n_req, IDX_HEADS, IDX_DIM, generator=g, device=device).to(torch.bfloat16)
    w = torch.rand(n_req, IDX_HEADS, generator=g, device=device) / IDX_HEADS
    q_mla = torch.randn(n_req, n_heads, LAT_DIM, generator=g, device=device).to(torch.bfloat16)
    q4 = F.mxfp4_key_rows(q_idx.reshape(-1, IDX_DIM)).view(n_req, IDX_HEADS, F.KEY_BYTES[1]).contiguous()
    return DecodeQueries(q_idx=q_idx, w=w.float().contiguous(), q_mla=q_mla,
                         sm_scale=float(np.float32(1.0 / math.sqrt(LAT_DIM))), q_idx_mxfp4=q4)


@dataclass
class PrefillQueries:
    n_q: int
    q_req: torch.Tensor        # int32 [n_q]
    row_len: torch.Tensor      # int32 [n_q]   (causal: position + 1)
    q_idx_bf16: torch.Tensor   # bf16 [n_q, 32, 128]
    q_idx_fp8: torch.Tensor    # uint8 [n_q, 32, 128]
    q_idx_scale: torch.Tensor  # fp32 [n_q, 32]
    w: torch.Tensor            # fp32 [n_q, 32]
    q_mla_bf16: torch.Tensor   # bf16 [n_q, H, 576]
    q_mla_fp8: torch.Tensor    # uint8 [n_q, H, 576]
    q_mla_scale: torch.Tensor  # fp32 [n_q, H]
    sm_scale: float


def prefill_queries(prefix: int, chunk: int, n_heads: int = 96, seed: int = 0, device="cpu",
                    req: int = 0) -> PrefillQueries:
    """A prefill chunk of ``chunk`` new tokens at positions prefix..prefix+chunk-1.

    Queries are drawn bf16 ~ N(0,1); the FP8 query mode consumes their e4m3
    codes with one absmax/448 scale per (row, head).
    """
    g = _gen(seed * 7727 + 11, device)
    q_idx = torch.randn(chunk, IDX_HEADS, IDX_DIM, generator=g, device=device).to(torch.bfloat16)
    w = torch.rand(chunk, IDX_HEADS, generator=g, device=device) / IDX_HEADS
    q_mla = torch.randn(chunk, n_heads, LAT_DIM, generator=g, device=device).to(torch.bfloat16)
    qi8, qis = F.fp8_rowhead_quant(q_idx.float())
    qm8, qms = F.fp8_rowhead_quant(q_mla.float())
    pos = torch.arange(prefix, prefix + chunk, device=device, dtype=torch.int32)
    return PrefillQueries(n_q=chunk, q_req=torch.full((chunk,), req, dtype=torch.int32, device=device),
                          row_len=(pos + 1).to(torch.int32), q_idx_bf16=q_idx, q_idx_fp8=qi8,
                          q_idx_scale=qis, w=w.float().contiguous(), q_mla_bf16=q_mla,
                          q_mla_fp8=qm8, q_mla_scale=qms,
                          sm_scale=float(np.float32(1.0 / math.sqrt(LAT_DIM))))


@dataclass
class VerifyQueries:
    """Speculative verification: m query rows per request (the last accepted token and m-1
    drafts) at the request's last m positions; row i of request b is row b*m + i."""
    m: int
    q_req: torch.Tensor   # int32 [B*m]
    row_len: torch.Tensor  # int32 [B*m]  causal: L_b - m + 1 + i
    q_idx: torch.Tensor   # bf16 [B*m, 32, 128]
    w: torch.Tensor       # fp32 [B*m, 32]
    q_mla: torch.Tensor   # bf16 [B*m, H, 576]
    sm_scale: float


def verify_queries(ctx_lens, m: int, n_heads: int = 12, seed: int = 0, device="cpu") -> VerifyQueries:
    """Indexer query bf16 ~ N(0,1), head weights ~ U(0,1)/32, MLA query bf16 ~ N(0,1), per row."""
    ctx = [int(c) for c in ctx_lens]
    n = len(ctx) * m
    g = _gen(seed * 40503 + 17, device)
    q_idx = torch.randn(n, IDX_HEADS, IDX_DIM, generator=g, device=device).to(torch.bfloat16)
    w = torch.rand(n, IDX_HEADS, generator=g, device=device) / IDX_HEADS
    q_mla = torch.randn(n, n_heads, LAT_DIM, generator=g, device=device).to(torch.bfloat16)
    rl = [max(0, L - m + 1 + i) for L in ctx for i in range(m)]
    return VerifyQueries(m=m, q_req=torch.arange(n, dtype=torch.int32, device=device) // m,
                         row_len=torch.tensor(rl, dtype=torch.int32, device=device), q_idx=q_idx,
                         w=w.float().contiguous(), q_mla=q_mla,
                         sm_scale=float(np.float32(1.0 / math.sqrt(LAT_DIM))))


def loguniform_lengths(n: int, lo: int, hi: int, seed: int) -> list[int]:
    """Context lengths round(exp(U[ln lo, ln hi])), seeded."""
    rng = np.random.default_rng(seed)
    return [int(round(math.exp(v))) for v in rng.uniform(math.log(lo), math.log(hi), size=n)]


# The five workloads.  Sizes follow the decode/prefill shapes of the pages'
# measurements: "batch 32 at 128K" (page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持",
# section "流量减少 10× 的精确 top-k 合并"), a 1M-token window, a mixed batch of
# 64 with MXFP4 keys / NVFP4 latents (sections "KV 缓存占用" and
# "量化：原生 MXFP4 索引器"; recipe page, section "NVFP4 KV cache"), and the
# 2K append to a ~150K prefix (section "预填充：按 token 而非按头分片注意力").
WORKLOADS = {
    0: dict(name="tiny-decode-b1-4k", kind="decode", ctx=[4096], heads=12, key_fmt=0, lat_fmt=0,
            spare_rows=64, topk=2048),
    1: dict(name="decode-b32-128k-fp8", kind="decode", ctx=[131072] * 32, heads=12, key_fmt=0,
            lat_fmt=0, spare_rows=0, topk=2048),
    2: dict(name="decode-b8-1m-fp8", kind="decode", ctx=[1048576] * 8, heads=12, key_fmt=0,
            lat_fmt=0, spare_rows=0, topk=2048),
    3: dict(name="decode-b64-mixed-mxfp4-nvfp4", kind="decode", ctx="loguniform", heads=12,
            key_fmt=1, lat_fmt=1, spare_rows=0, topk=2048, n=64, lo=4096, hi=524288),
    4: dict(name="prefill-2k-on-150k-fp8", kind="prefill", prefix=153600, chunk=2048, heads=96,
            key_fmt=0, lat_fmt=0, spare_rows=0, topk=2048),
    # speculative verification: DSpark's 7 draft tokens, i.e. 8 query rows per request
    # (section "低延迟解码：融合的 DSA 解码路径"), each key read once for all 8 rows
    # (section "量化：原生 MXFP4 索引器"), on the batch-32 / 128K decode shape
    5: dict(name="verify-b32x8-128k-fp8", kind="verify", ctx=[131072] * 32, rows=8, heads=12, key_fmt=0,
            lat_fmt=0, spare_rows=0, topk=2048),
}


def workload_ctx(cfg_id: int, seed: int | None = None) -> list[int]:
    w = WORKLOADS[cfg_id]
    s = cfg_id if seed is None else seed
    if w["kind"] == "prefill":
        return [w["prefix"] + w["chunk"]]
    if w["ctx"] == "loguniform":
        return loguniform_lengths(w["n"], w["lo"], w["hi"], s)
    return list(w["ctx"])


def algorithmic_verify_bytes(ctx_lens, m: int, key_bytes: int, lat_bytes: int, k: int = 2048) -> int:
    """Verify step with key reuse: each request's keys once, plus every row's selected latents
    (row i of a request at context L has L - m + 1 + i tokens)."""
    return int(sum(int(L) * key_bytes + sum(min(k, max(0, int(L) - m + 1 + i)) * lat_bytes for i in range(m))
                   for L in ctx_lens))


def algorithmic_decode_bytes(ctx_lens, key_bytes: int, lat_bytes: int, k: int = 2048) -> int:
    """Cache bytes the method must move per decode layer-step: sum_b L_b*key + min(k,L_b)*lat."""
    return int(sum(int(L) * key_bytes + min(k, int(L)) * lat_bytes for L in ctx_lens))
