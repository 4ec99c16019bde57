"""Pins for the oracle's number-format decoders and the generator's encoders.

The oracle's decoders are checked against (a) values fixed by the public
specifications (OCP OFP8 E4M3; OCP MX v1.0 E2M1 / E8M0), written out here as
constants, and (b) an independent decoder: torch's float8_e4m3fn type.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from tests.helpers import torch_e4m3_values


# OCP OFP8 (E4M3) fixed points: code -> value.
E4M3_POINTS = {
    0x00: 0.0, 0x80: -0.0,
    0x01: 2.0 ** -9,            # smallest subnormal
    0x07: 0.875 * 2.0 ** -6,    # largest subnormal
    0x08: 2.0 ** -6,            # smallest normal
    0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0xB8: -1.0,
    0x7E: 448.0,                # largest finite
    0xFE: -448.0,
}
# OCP MX E2M1: the eight magnitudes, in code order.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_fixed_points():
    for code, v in E4M3_POINTS.items():
        got = oracle.e4m3(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(code)


def test_e4m3_nan_codes():
    assert math.isnan(oracle.e4m3(0x7F)) and math.isnan(oracle.e4m3(0xFF))
    # no other code is NaN or infinite (E4M3FN has no infinities)
    for c in range(256):
        if c not in (0x7F, 0xFF):
            assert math.isfinite(oracle.e4m3(c)), hex(c)


def test_e4m3_all_codes_vs_torch():
    ref = torch_e4m3_values(np.arange(256))
    for c in range(256):
        got = oracle.e4m3(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == ref[c], hex(c)


def test_e2m1_all_codes():
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        want = -mag if c & 8 else mag
        assert oracle.e2m1(c) == want, c


def test_e8m0_codes():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0
    assert oracle.e8m0(126) == 0.5
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def test_bf16_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b, r in zip(bits, ref):
        got = oracle.bf16(int(b))
        assert (math.isnan(got) and math.isnan(r)) or got == r


# --- generator encoders: round to nearest, so |decode(encode(x)) - x| <= half a step ---

def test_e2m1_encoder_is_nearest_even():
    xs = np.linspace(-7, 7, 2801, dtype=np.float32)
    codes = F.e2m1_codes(torch.from_numpy(xs)).numpy()
    grid = np.array(E2M1_MAGNITUDES)
    for x, c in zip(xs, codes):
        v = oracle.e2m1(int(c))
        a = min(abs(float(x)), 6.0)
        d = np.abs(grid - a)
        best = grid[d == d.min()]
        if len(best) == 2:   # tie: the even mantissa (code index even) wins
            best = [b for b in best if E2M1_MAGNITUDES.index(b) % 2 == 0]
        assert abs(v) == best[0], (x, v)


def test_fp8_key_rows_round_trip():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(1))
    rows = F.fp8_key_rows(x).numpy()
    for t in range(64):
        k, s = oracle.key_decode(0, rows[t])
        amax = float(x[t].abs().max())
        assert s == np.float32(amax / 448.0)
        # e4m3 has 3 mantissa bits: relative step <= 2^-3 in the normal range
        err = np.abs(k * s - x[t].double().numpy())
        assert (err <= np.maximum(np.abs(x[t].double().numpy()) * 2 ** -4, s * 2 ** -10) + 1e-12).all()


def test_mxfp4_key_rows_round_trip():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(2))
    rows = F.mxfp4_key_rows(x).numpy()
    for t in range(64):
        k, s = oracle.key_decode(1, rows[t])
        assert s == 1.0
        xv = x[t].double().numpy()
        for blk in range(4):
            e8 = int(rows[t, 64 + blk])
            scale = 2.0 ** (e8 - 127)
            sl = slice(32 * blk, 32 * blk + 32)
            # largest element maps into [4, 8) before rounding (OCP MX shared-exponent rule)
            assert 4.0 <= np.abs(xv[sl]).max() / scale < 8.0
            # elements: nearest e2m1 step (max step 2 at the top of the range), saturating at 6
            assert (np.abs(k[sl] - np.clip(xv[sl], -6 * scale, 6 * scale)) <= 1.0 * scale + 1e-12).all()


def test_nvfp4_latent_rows_round_trip():
    x = torch.randn(32, 576, generator=torch.Generator().manual_seed(3))
    kv_scale = float(np.float32(float(x.abs().max()) / 448.0))
    rows = F.nvfp4_latent_rows(x, kv_scale).numpy()
    for t in range(32):
        kv = oracle.latent_decode(1, rows[t], kv_scale)
        xv = x[t].double().numpy()
        # rope dims: e4m3 of x/kv_scale
        assert (np.abs(kv[512:] - xv[512:]) <= np.abs(xv[512:]) * 2 ** -4 + kv_scale * 2 ** -10).all()
        # no-rope dims: within one e2m1 step of the block's scale
        for blk in range(32):
            sl = slice(16 * blk, 16 * blk + 16)
            bsc = oracle.e4m3(int(rows[t, 256 + blk])) * kv_scale
            assert (np.abs(kv[sl] - xv[sl]) <= 1.0 * bsc + 0.07 * np.abs(xv[sl]).max() + 1e-12).all()


def test_fp8_latent_rows_round_trip():
    x = torch.randn(16, 576, generator=torch.Generator().manual_seed(4))
    kv_scale = float(np.float32(float(x.abs().max()) / 448.0))
    rows = F.fp8_latent_rows(x, kv_scale).numpy()
    for t in range(16):
        kv = oracle.latent_decode(0, rows[t], kv_scale)
        xv = x[t].double().numpy()
        assert (np.abs(kv - xv) <= np.abs(xv) * 2 ** -4 + kv_scale * 2 ** -10).all()


@pytest.mark.parametrize("key_fmt,lat_fmt", [(0, 0), (1, 1)])
def test_poison_decodes_to_nan(key_fmt, lat_fmt):
    """0xFF filler (spare rows, unused slots) decodes to NaN in every format."""
    k, s = oracle.key_decode(key_fmt, np.full(132, 0xFF, np.uint8))
    assert math.isnan(s * k.sum())
    kv = oracle.latent_decode(lat_fmt, np.full(576, 0xFF, np.uint8), 1.0)
    assert np.isnan(kv).all()
