"""Pins for the block-packed layout, the page resolver and the sizes printed on the pages."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")))


def g(name):
    return GOLD[name]["value"]


def test_row_widths_match_pages():
    fp8 = oracle.layout_make(64, 1, 0, 0)
    fp4 = oracle.layout_make(64, 1, 1, 1)
    assert fp8.key_bytes == g("fp8_key_bytes") and fp8.lat_bytes == g("fp8_latent_bytes")
    assert fp4.key_bytes == g("mxfp4_key_bytes") and fp4.lat_bytes == g("nvfp4_latent_bytes")
    # the two per-token widths are not multiples of each other (the packing problem)
    assert 576 % 132 and 352 % 68


def test_ratios_printed_on_pages():
    # MXFP4 keys: 1 - 68/132 = 48.5% less index cache
    assert round(1 - 68 / 132, 3) == g("mxfp4_index_cache_cut")
    # NVFP4 latents: (576+132)/(352+132) = 1.46, "about 1.5x"
    assert abs((576 + 132) / (352 + 132) - g("nvfp4_capacity_gain")) < 0.05
    # both FP4: (576+132)/(352+68) = 1.69, "1.7x"
    assert round((576 + 132) / (352 + 68), 1) == g("both_fp4_capacity_gain")
    # 1M tokens = 2^20: 3.04M tokens are 2.9 one-M requests only if 1M = 2^20
    assert round(g("tp8_fp8_tokens") / 2 ** 20, 1) == g("tp8_concurrent_1m")
    # FP8 latents plus keys for 2^20 tokens: 742,391,808 B, "about 0.7 GB"
    b = 2 ** 20 * (576 + 132)
    assert b == 742_391_808 and round(b / 1e9, 1) == g("dcp_workspace_gb_per_1m_fp8")


def test_layout_strides_closed_form():
    # 64*576 + 64*132 = 45312 = 177*256; 64*352 + 64*68 = 26880 = 105*256
    L = oracle.layout_make(64, 24, 0, 0, 1000)
    assert L.layer_stride == 45312 and L.row_stride == (24 * 45312 + 1000 + 255) // 256 * 256
    L = oracle.layout_make(64, 3, 1, 1, 0)
    assert L.layer_stride == 26880 and L.row_stride == 3 * 26880
    L = oracle.layout_make(64, 1, 0, 1, 0)   # NVFP4 latents with FP8 keys
    assert L.layer_stride == (64 * 352 + 64 * 132 + 255) // 256 * 256
    for kf in (0, 1):
        for lf in (0, 1):
            for nl, ex in ((1, 0), (24, 4096), (3, 17)):
                assert oracle.layout_make(64, nl, kf, lf, ex).as_dict() == {
                    k: v for k, v in W.layout_params(kf, lf, nl, 64, ex).items()
                    if k in oracle.OrLayout().as_dict()}


def test_resolve_closed_form():
    c = W.build_cache([700, 64, 1, 300], key_fmt=0, lat_fmt=1, seed=5, spare_rows=9, n_layers=3, layer=2)
    oc = oracle.OracleCache(c)
    rc, lat, key = oracle.resolve_pages(oc, off_ld=20)
    assert rc == oracle.OK
    L = oc.layout
    for b in range(oc.n_req):
        for p in range(20):
            if p < oc.n_pages[b]:
                row = oc.bt[b, p]
                assert lat[b, p] == row * L.row_stride + 2 * L.layer_stride
                assert key[b, p] == lat[b, p] + 64 * 352
            elif p < oc.bt.shape[1]:
                assert lat[b, p] == -1 and key[b, p] == -1
            else:   # columns past the block table's width are left alone
                assert lat[b, p] == -2 and key[b, p] == -2


def test_resolve_flags_bad_block():
    c = W.build_cache([200], seed=1)
    oc = oracle.OracleCache(c)
    oc.bt[0, 1] = oc.pool_rows      # one past the end
    rc, lat, key = oracle.resolve_pages(oc)
    assert rc == oracle.ERR_RANGE and lat[0, 1] == -1 and lat[0, 0] >= 0


def test_pool_places_tokens_where_the_layout_says():
    """Generator placement agrees with the oracle's address rule (token -> row, slot)."""
    c = W.build_cache([130], key_fmt=0, lat_fmt=0, seed=2, spare_rows=3, n_layers=2, layer=1)
    oc = oracle.OracleCache(c)
    L = oc.layout
    # every used key slot decodes to finite values; unused slot 130 % 64 = 2.. of page 2 is poison
    for t in range(130):
        row = oc.bt[0, t // 64]
        o = row * L.row_stride + L.layer_stride + 64 * 576 + (t % 64) * 132
        k, s = oracle.key_decode(0, oc.pool[row].reshape(-1)[o - row * L.row_stride:][:132])
        assert np.isfinite(k).all() and np.isfinite(s)
    row = oc.bt[0, 2]
    o = L.layer_stride + 64 * 576 + 2 * 132
    k, s = oracle.key_decode(0, oc.pool[row][o:o + 132])
    assert np.isnan(s)
