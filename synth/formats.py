"""Encoders that turn real-valued synthetic data into the cache's byte formats.

This module only *produces* inputs.  It holds none of the arithmetic of the
sparse-attention step itself (no decoding of cache rows, no scoring, no
selection, no attention).  The HIP library and the CPU oracle both consume the
bytes written here, and neither imports the other.

Formats (public specifications):
  * e4m3  -- OCP 8-bit floating point, E4M3FN: bias 7, max 448, no infinities.
  * e2m1  -- OCP Microscaling (MX) v1.0 FP4 element: {0, .5, 1, 1.5, 2, 3, 4, 6}.
  * E8M0  -- OCP MX shared scale, 2^(e-127).
  * NVFP4 -- 16-element blocks of e2m1 with an e4m3 block scale.

Rounding is round-to-nearest-even everywhere, with saturation to the largest
finite magnitude (the rule the generator states; it is not part of parity).
"""
from __future__ import annotations

import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0

KEY_BYTES = {0: 132, 1: 68}    # FP8 e4m3 + fp32 scale ; MXFP4 (64 B codes + 4 E8M0)
LAT_BYTES = {0: 576, 1: 352}   # FP8 e4m3 ; NVFP4 (256 B e2m1 + 32 e4m3 scales + 64 e4m3 rope)


def e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """e4m3 codes of ``x`` (RNE, saturating at +-448), as uint8."""
    return x.float().clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def e4m3_value_of_codes(c: torch.Tensor) -> torch.Tensor:
    """Real value of e4m3 codes through torch's own float8 type.

    Used only to learn the value a block scale rounded to, so that the
    generator can encode elements against it.
    """
    return c.view(torch.float8_e4m3fn).float()


def e2m1_codes(x: torch.Tensor) -> torch.Tensor:
    """e2m1 nibble codes (0..15, bit 3 = sign) of ``x``: RNE, saturating at 6.

    The magnitude code is the number of representable magnitudes that ``|x|``
    rounds above; each comparison is strict or not so that a tie goes to the
    neighbour with the even mantissa bit.
    """
    a = x.float().abs()
    mag = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8)
           + (a > 1.25).to(torch.uint8) + (a >= 1.75).to(torch.uint8)
           + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
           + (a > 5.0).to(torch.uint8))
    neg = (x < 0) & (mag > 0)
    return mag | (neg.to(torch.uint8) << 3)


def _pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """Pack [..., 2n] nibble codes into [..., n] bytes, element 2i in the low nibble."""
    return codes[..., 0::2] | (codes[..., 1::2] << 4)


def _floor_log2(a: torch.Tensor) -> torch.Tensor:
    """floor(log2(a)) for a > 0, exactly (via frexp: a = m * 2^e, m in [0.5, 1))."""
    _, e = torch.frexp(a)
    return e.to(torch.int32) - 1


def fp8_key_rows(x: torch.Tensor) -> torch.Tensor:
    """[n,128] floats -> [n,132] bytes: 128 e4m3 codes then the fp32 scale (LE).

    Per-token absmax scaling: scale = absmax/448, codes = e4m3(x/scale).
    """
    n = x.shape[0]
    x = x.float()
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = e4m3_codes(x / scale[:, None])
    sbytes = scale.contiguous().view(torch.uint8).view(n, 4)
    return torch.cat([codes, sbytes], dim=1)


def mxfp4_key_rows(x: torch.Tensor) -> torch.Tensor:
    """[n,128] floats -> [n,68] bytes: 64 B of e2m1 pairs, then 4 E8M0 scales.

    OCP MX scale selection: the shared exponent of each 32-element block is
    floor(log2(absmax)) - 2 (2 = largest exponent of e2m1), so the largest
    element lands in [4, 8) before rounding and saturation.
    """
    n = x.shape[0]
    xb = x.float().view(n, 4, 32)
    amax = xb.abs().amax(dim=2)
    e = torch.where(amax > 0, _floor_log2(amax.clamp_min(1e-30)) - 2,
                    torch.zeros_like(amax, dtype=torch.int32))
    e = e.clamp(-126, 127)
    scale = torch.pow(torch.tensor(2.0, device=x.device), e.float())
    codes = e2m1_codes(xb / scale[..., None]).view(n, 128)
    biased = (e + 127).to(torch.uint8)
    return torch.cat([_pack_nibbles(codes), biased], dim=1)


def fp8_latent_rows(x: torch.Tensor, kv_scale: float) -> torch.Tensor:
    """[n,576] floats -> [n,576] e4m3 codes of x/kv_scale."""
    return e4m3_codes(x.float() / kv_scale)


def nvfp4_latent_rows(x: torch.Tensor, kv_scale: float) -> torch.Tensor:
    """[n,576] floats -> [n,352] bytes.

    Bytes 0..255: e2m1 codes of dims 0..511 (element 2i in the low nibble);
    bytes 256..287: e4m3 block scales, one per 16 dims of 0..511;
    bytes 288..351: e4m3 codes of the rope dims 512..575.
    A value is code * block_scale * kv_scale (rope: code * kv_scale).
    """
    n = x.shape[0]
    x = x.float()
    nope = x[:, :512].reshape(n, 32, 16)
    bamax = nope.abs().amax(dim=2)
    bs_codes = e4m3_codes(bamax / (E2M1_MAX * kv_scale))
    bs = e4m3_value_of_codes(bs_codes) * kv_scale
    safe = torch.where(bs > 0, bs, torch.ones_like(bs))
    q = torch.where(bs[..., None] > 0, nope / safe[..., None], torch.zeros_like(nope))
    codes = e2m1_codes(q).view(n, 512)
    rope = e4m3_codes(x[:, 512:] / kv_scale)
    return torch.cat([_pack_nibbles(codes), bs_codes, rope], dim=1)


def fp8_rowhead_quant(x: torch.Tensor):
    """Quantise [..., D] to e4m3 with one fp32 absmax scale per leading index.

    Returns (codes uint8 [..., D], scale float32 [...]).  Used for the FP8
    query mode: the oracle and the kernels both consume these codes/scales.
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    return e4m3_codes(x / scale[..., None]), scale.contiguous()
