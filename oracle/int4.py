"""Group-32 symmetric absmax int4 codec of the latent cache (oracle; test infrastructure only).

The Paper-Notes ACL2025 page on MHA2MLA (section 关键设计, "compatible with KV-cache
quantisation") states that the latent c_kv can be quantised to 4 bits on top of the
low-rank compression; it fixes no format.  The format here, per token and per group
of 32 consecutive latent dims:

    a    = max |x|                         (x are fp32 values)
    s    = fp16_rne(a / 7)                 (a / 7 an IEEE fp32 division; an infinite s saturates to 65504)
    code = clamp(rint_half_even(x / s), -7, 7)   (x / s an IEEE fp32 division); s == 0 gives codes 0
    byte i of the group = (code[2i] & 0xF) | (code[2i+1] & 0xF) << 4     (two's-complement nibbles)
    dequant = fp32(code) * fp32(s)         (exact in fp32)

Codes are integers decided in fp32, so this module computes in numpy float32 / float16,
whose element-wise division and conversions are IEEE correctly rounded (round to nearest even).
"""

from __future__ import annotations

import numpy as np

GROUP = 32
QMAX = 7


def int4_scale(absmax):
    """Group scale from the group's fp32 absmax: fp16_rne(absmax / 7), the division in IEEE fp32, an infinite
    result saturated to 65504.  Returns float16."""
    a = np.asarray(absmax, dtype=np.float32)
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(QMAX)).astype(np.float16)
    return np.where(np.isinf(s16), np.float16(65504.0), s16).astype(np.float16)


def int4_codes(x, s16):
    """Codes of fp32 values x [..., 32] under their group's fp16 scale s16 [...]: clamp(rint_half_even(x / s),
    -7, 7) with an IEEE fp32 division; a zero scale gives zero codes.  Returns int8."""
    g = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    nz = np.broadcast_to(s32 > 0, g.shape)
    q = np.divide(g, np.where(s32 > 0, s32, np.float32(1.0)), dtype=np.float32)
    return np.where(nz, np.clip(np.rint(q), -QMAX, QMAX), 0).astype(np.int8)


def quantize_int4_g32(x):
    """x: fp32 array [..., n*32].  Returns (codes int8 [..., n*32] in [-7, 7], scales float16 [..., n])."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    g = x.reshape(-1, GROUP)
    s16 = int4_scale(np.max(np.abs(g), axis=1))
    codes = int4_codes(g, s16)
    return codes.reshape(shp), s16.reshape(shp[:-1] + (shp[-1] // GROUP,))


def pack_nibbles(codes):
    """int8 codes [..., 2m] -> uint8 [..., m], low nibble = even element."""
    c = np.asarray(codes).astype(np.int16)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """uint8 [..., m] -> int8 codes [..., 2m] (sign-extended nibbles)."""
    p = np.asarray(packed).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_int4(codes, scales):
    """fp32(code) * fp32(scale) per group, returned as fp64 (exact)."""
    c = np.asarray(codes, dtype=np.float32)
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    shp = c.shape
    g = c.reshape(-1, GROUP) * s.reshape(-1, 1)
    return g.reshape(shp).astype(np.float64)


def windowed_latent_int4(rows_bf16, W):
    """The latent rows that attention reads for one sequence of an int4 cache that keeps a window of recent bf16
    rows (the README page's quantised-cache evaluation keeps the most recent tokens unquantised): rows older
    than the last min(L, W) are replaced by the int4 codec of their bf16 values, the window's rows stay.

    rows_bf16: [L, d_kv] values already on the bf16 grid.  Returns (rows [L, d_kv] fp64, codes
    [L - min(L, W), d_kv], scales [L - min(L, W), d_kv/32])."""
    x = np.asarray(rows_bf16, dtype=np.float32)
    L = x.shape[0]
    nq = L - min(L, W)
    codes, scales = quantize_int4_g32(x[:nq])
    out = x.astype(np.float64)
    if nq > 0:
        out[:nq] = dequant_int4(codes, scales)
    return out, codes, scales
