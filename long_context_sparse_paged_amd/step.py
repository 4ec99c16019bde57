"""One DSA layer-step, as a sequence of the C entry points.

``DecodeStep`` / ``PrefillStep`` own the device buffers a step needs (page
offsets, scores, selected indices, outputs, workspaces) and call
dsa_resolve_pages -> dsa_indexer_score -> dsa_topk -> dsa_sparse_mla_* on one
stream; ``PrefillSelectStep`` scores and selects a prefill chunk in one call,
dsa_prefill_select (FP8 MFMA, exact top-k); ``VerifyStep`` does the same for speculative verification, with
dsa_indexer_score_verify reading each key page once for all rows of a request.
``FusedDecodeStep`` is the fused decode path: dsa_indexer_select (scores with
pages found through the block table, exact top-k and physical rows) ->
dsa_sparse_mla_decode_phys.
No arithmetic happens here.
"""
from __future__ import annotations

import torch

from . import (DSA_Q_BF16, DSA_Q_FP8_E4M3, dsa_indexer_score, dsa_indexer_score_pages, dsa_indexer_score_verify,
               dsa_indexer_score_workspace_size, dsa_indexer_select, dsa_indexer_select_workspace_size,
               dsa_layout_make, dsa_prefill_gemm_fp8, dsa_prefill_prepare_fp8, dsa_prefill_score_fp8,
               dsa_prefill_select, dsa_prefill_select_workspace_size, dsa_prefill_topk_band, dsa_resolve_pages,
               dsa_sparse_mla_decode, dsa_sparse_mla_decode_phys, dsa_sparse_mla_decode_workspace_size,
               dsa_sparse_mla_prefill, dsa_sparse_mla_prefill_workspace_size, dsa_topk, dsa_topk_pages,
               dsa_topk_workspace_size)


def _layout_of(cache):
    lp = cache.layout
    return dsa_layout_make(lp["page_size"], lp["n_layers"], lp["key_fmt"], lp["lat_fmt"], lp["extra_row_bytes"])


class _Base:
    def __init__(self, cache, k: int, n_rows: int, ld: int, device):
        self.cache = cache
        self.layout = _layout_of(cache)
        self.k = k
        self.device = device
        n_req, max_pages = cache.block_table.shape
        self.lat_off = torch.empty(n_req, max_pages, dtype=torch.int64, device=device)
        self.key_off = torch.empty(n_req, max_pages, dtype=torch.int64, device=device)
        self.scores = torch.empty(n_rows, max(ld, 1), dtype=torch.float32, device=device)
        self.idx = torch.empty(n_rows, k, dtype=torch.int32, device=device)
        self.ws_topk = torch.empty(max(dsa_topk_workspace_size(n_rows, max(ld, 1), k), 16), dtype=torch.uint8,
                                   device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)

    def resolve(self, stream=None):
        c = self.cache
        dsa_resolve_pages(self.layout, c.layer, c.block_table, c.n_pages, c.pool_rows, self.lat_off, self.key_off,
                          self.err, stream)

    def topk(self, stream=None):
        dsa_topk(self.scores, self.row_len, self.k, self.idx, self.ws_topk, self.err, stream)


class DecodeStep(_Base):
    """Decode: one query row per request (row_len = context length).  q_fmt DSA_Q_MXFP4 takes
    q_idx as [B, 32, 68] MXFP4 rows (MXFP4 keys: native FP4 scoring)."""

    def __init__(self, cache, q_idx, w, q_mla, sm_scale: float, k: int = 2048, device="cuda",
                 q_fmt: int = DSA_Q_BF16):
        n_req = cache.block_table.shape[0]
        ld = int(cache.ctx_len.max().item()) if n_req else 1
        super().__init__(cache, k, n_req, ld, device)
        self.q_idx, self.w, self.q_mla = q_idx, w, q_mla
        self.q_fmt = q_fmt
        self.sm_scale = sm_scale
        self.n_heads = q_mla.shape[1]
        self.q_req = torch.arange(n_req, dtype=torch.int32, device=device)
        self.row_len = cache.ctx_len
        self.out = torch.empty(n_req, self.n_heads, 512, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(n_req, self.n_heads, dtype=torch.float32, device=device)
        nb = dsa_sparse_mla_decode_workspace_size(n_req, self.n_heads, k)
        self.ws_mla = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None

    def score(self, stream=None):
        c = self.cache
        dsa_indexer_score(self.layout, c.pool, self.key_off, c.n_req, self.q_idx, self.q_fmt, None, self.w,
                          self.q_req, self.row_len, self.scores, None, self.err, stream)

    def attend(self, stream=None):
        c = self.cache
        dsa_sparse_mla_decode(self.layout, c.pool, self.lat_off, c.ctx_len, self.idx, self.k, self.q_mla,
                              self.sm_scale, c.kv_scale, self.out, self.lse, self.ws_mla, self.err, stream)

    def run(self, stream=None):
        self.resolve(stream)
        self.score(stream)
        self.topk(stream)
        self.attend(stream)


class PrefillStep(_Base):
    """Prefill chunk: rows at consecutive positions of one request (row_len = position + 1)."""

    def __init__(self, cache, pq, k: int = 2048, q_fmt: int = DSA_Q_FP8_E4M3, device="cuda"):
        ld = int(cache.ctx_len.max().item())
        super().__init__(cache, k, pq.n_q, ld, device)
        self.pq = pq
        self.q_fmt = q_fmt
        self.n_heads = pq.q_mla_bf16.shape[1]
        self.row_len = pq.row_len
        self.out = torch.empty(pq.n_q, self.n_heads, 512, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(pq.n_q, self.n_heads, dtype=torch.float32, device=device)
        nb = dsa_sparse_mla_prefill_workspace_size(pq.n_q, self.n_heads, k)
        self.ws_mla = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None
        nb = dsa_indexer_score_workspace_size(pq.n_q, q_fmt)
        self.ws_score = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None

    def score(self, stream=None):
        c, pq = self.cache, self.pq
        if self.q_fmt == DSA_Q_FP8_E4M3:
            q, qs = pq.q_idx_fp8, pq.q_idx_scale
        else:
            q, qs = pq.q_idx_bf16, None
        dsa_indexer_score(self.layout, c.pool, self.key_off, c.n_req, q, self.q_fmt, qs, pq.w, pq.q_req, pq.row_len,
                          self.scores, self.ws_score, self.err, stream)

    def attend(self, stream=None):
        c, pq = self.cache, self.pq
        if self.q_fmt == DSA_Q_FP8_E4M3:
            q, qs = pq.q_mla_fp8, pq.q_mla_scale
        else:
            q, qs = pq.q_mla_bf16, None
        dsa_sparse_mla_prefill(self.layout, c.pool, self.lat_off, c.n_req, c.ctx_len, self.idx, self.k, q, self.q_fmt,
                               qs, pq.q_req, pq.sm_scale, c.kv_scale, self.out, self.lse, self.ws_mla, self.err,
                               stream)

    def run(self, stream=None):
        self.resolve(stream)
        self.score(stream)
        self.topk(stream)
        self.attend(stream)


class VerifyStep(_Base):
    """Speculative verification: m query rows per request (row b*m + i at position L_b - m + i,
    row_len = L_b - m + 1 + i); the indexer reads each key page once for all m rows, then every
    row gets its own top-k and attention."""

    def __init__(self, cache, vq, k: int = 2048, device="cuda"):
        n_req = cache.block_table.shape[0]
        ld = int(cache.ctx_len.max().item()) if n_req else 1
        super().__init__(cache, k, n_req * vq.m, ld, device)
        self.vq = vq
        self.m = vq.m
        self.n_heads = vq.q_mla.shape[1]
        self.row_len = vq.row_len
        self.out = torch.empty(n_req * vq.m, self.n_heads, 512, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(n_req * vq.m, self.n_heads, dtype=torch.float32, device=device)
        nb = dsa_sparse_mla_prefill_workspace_size(n_req * vq.m, self.n_heads, k)
        self.ws_mla = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None

    def score(self, stream=None):
        c, vq = self.cache, self.vq
        dsa_indexer_score_verify(self.layout, c.pool, self.key_off, c.n_req, vq.m, vq.q_idx, vq.w, vq.row_len,
                                 self.scores, self.err, stream)

    def attend(self, stream=None):
        c, vq = self.cache, self.vq
        dsa_sparse_mla_prefill(self.layout, c.pool, self.lat_off, c.n_req, c.ctx_len, self.idx, self.k, vq.q_mla,
                               DSA_Q_BF16, None, vq.q_req, vq.sm_scale, c.kv_scale, self.out, self.lse, self.ws_mla,
                               self.err, stream)

    def run(self, stream=None):
        self.resolve(stream)
        self.score(stream)
        self.topk(stream)
        self.attend(stream)


class FusedDecodeStep:
    """Fused decode: the scan reads pages through the block table (no resolve launch), the
    top-k writes each kept token's physical row beside its index, and attention reads those
    rows directly.  The same results as DecodeStep (bit for bit)."""

    def __init__(self, cache, q_idx, w, q_mla, sm_scale: float, k: int = 2048, device="cuda",
                 q_fmt: int = DSA_Q_BF16):
        self.cache = cache
        self.layout = _layout_of(cache)
        self.k = k
        self.q_fmt = q_fmt
        n_req = cache.block_table.shape[0]
        ld = int(cache.ctx_len.max().item()) if n_req else 1
        ld = (ld + 3) // 4 * 4  # score rows start on 16 B (vector loads and stores)
        self.q_idx, self.w, self.q_mla = q_idx, w, q_mla
        self.sm_scale = sm_scale
        self.n_heads = q_mla.shape[1]
        self.q_req = torch.arange(n_req, dtype=torch.int32, device=device)
        self.row_len = cache.ctx_len
        self.scores = torch.empty(n_req, ld, dtype=torch.float32, device=device)
        self.idx = torch.empty(n_req, k, dtype=torch.int32, device=device)
        self.phys = torch.empty(n_req, k, dtype=torch.int32, device=device)
        self.ws_sel = torch.empty(max(dsa_indexer_select_workspace_size(n_req, ld), 256), dtype=torch.uint8,
                                  device=device)
        self.out = torch.empty(n_req, self.n_heads, 512, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(n_req, self.n_heads, dtype=torch.float32, device=device)
        nb = dsa_sparse_mla_decode_workspace_size(n_req, self.n_heads, k)
        self.ws_mla = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None
        self.err = torch.zeros(1, dtype=torch.int32, device=device)

    def select(self, stream=None):
        c = self.cache
        dsa_indexer_select(self.layout, c.layer, c.pool, c.block_table, c.n_req, self.q_idx, self.w, self.q_req,
                           self.row_len, self.k, self.scores, self.idx, self.phys, self.ws_sel, self.err, stream,
                           q_fmt=self.q_fmt)

    def score(self, stream=None):
        """The select's first half alone (the scan)."""
        c = self.cache
        dsa_indexer_score_pages(self.layout, c.layer, c.pool, c.block_table, c.n_req, self.q_idx, self.w, self.q_req,
                                self.row_len, self.scores, self.err, stream, q_fmt=self.q_fmt)

    def topk(self, stream=None):
        """The select's second half alone (needs score() first)."""
        c = self.cache
        dsa_topk_pages(self.layout, c.pool, c.block_table, c.n_req, self.q_req, self.scores, self.row_len, self.k,
                       self.ws_sel, self.idx, self.phys, self.err, stream)

    def attend(self, stream=None):
        c = self.cache
        dsa_sparse_mla_decode_phys(self.layout, c.layer, c.pool, self.phys, self.k, self.q_mla, self.sm_scale,
                                   c.kv_scale, self.out, self.lse, self.ws_mla, self.err, stream)

    def run(self, stream=None):
        self.select(stream)
        self.attend(stream)


class PrefillSelectStep(PrefillStep):
    """Prefill chunk with the indexer on FP8 MFMA: dsa_resolve_pages -> dsa_prefill_select
    (approximate scores, exact top-k) -> dsa_sparse_mla_prefill.  FP8 queries only."""

    def __init__(self, cache, pq, k: int = 2048, device="cuda"):
        super().__init__(cache, pq, k=k, q_fmt=DSA_Q_FP8_E4M3, device=device)
        self.ws_score = None
        self.ws_topk = None
        n_req, max_pages = cache.block_table.shape
        nb = dsa_prefill_select_workspace_size(pq.n_q, self.scores.shape[1], n_req, max_pages, k)
        self.ws_select = torch.empty(nb, dtype=torch.uint8, device=device)
        self.bound = torch.empty(pq.n_q, dtype=torch.float32, device=device)

    def select(self, stream=None):
        c, pq = self.cache, self.pq
        dsa_prefill_select(self.layout, c.pool, self.key_off, c.n_req, c.ctx_len, pq.q_idx_fp8, pq.q_idx_scale, pq.w,
                           pq.q_req, pq.row_len, self.k, self.scores, self.idx, self.ws_select, self.bound, self.err,
                           stream)

    def _score_args(self):
        c, pq = self.cache, self.pq
        return (self.layout, c.pool, self.key_off, c.n_req, c.ctx_len, pq.q_idx_fp8, pq.q_idx_scale, pq.w, pq.q_req,
                pq.row_len, self.k, self.scores, self.ws_select, self.bound, self.err)

    def score(self, stream=None):
        """First half of select(): the FP8 MFMA scores and their bound."""
        dsa_prefill_score_fp8(*self._score_args(), stream)

    def prepare(self, stream=None):
        """score()'s first part: pre-pass, key bound, sampled tiles and thresholds."""
        dsa_prefill_prepare_fp8(*self._score_args(), stream)

    def gemm(self, stream=None):
        """score()'s second part: the full FP8 GEMM."""
        dsa_prefill_gemm_fp8(*self._score_args(), stream)

    def topk(self, stream=None):
        """Second half of select(): the exact top-k (band rescored)."""
        c, pq = self.cache, self.pq
        dsa_prefill_topk_band(self.layout, c.pool, self.key_off, c.n_req, pq.q_req, pq.row_len, self.k, self.scores,
                              self.idx, self.ws_select, self.err, stream)

    def run(self, stream=None):
        self.resolve(stream)
        self.select(stream)
        self.attend(stream)
