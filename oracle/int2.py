"""Group-32 affine 2-bit codec of the latent cache with a window of recent bf16 rows (oracle; test
infrastructure only).

The Paper-Notes ACL2025 page on MHA2MLA (key designs, compatibility with KV-cache quantisation) says the
latent c_kv composes with 4-bit or 2-bit KV-cache quantisation; the GitHub README page's quantised-cache
evaluation runs an HQQ backend that keeps the most recent 128 tokens unquantised (its residual length).
Neither page fixes a 2-bit format.  The reading here, per token and per group of 32 consecutive latent
dims of the token's bf16 row x (values held in fp32):

    z    = fp16_rne(min x)                       (an infinite z saturates to +-65504)
    s    = fp16_rne(max(max x - z, 0) / 3)       (fp32 subtraction, IEEE fp32 division; saturating)
    code = 0 if s == 0 else clamp(rint_half_even((x - z) / s), 0, 3)   (fp32 subtraction and division)
    byte i of the group = code[4i] | code[4i+1] << 2 | code[4i+2] << 4 | code[4i+3] << 6
    dequant = fp32_rne(z + code * s)             (one rounding: the exact sum, as a fused multiply-add)

Window W >= 0: once a sequence holds L tokens, its last min(L, W) positions are bf16 rows and every
older position is codes.  A row is quantised from its bf16 value when it leaves the window, or at once
when it is appended already outside it; slot `pos mod W` of a ring of W rows holds position pos.

Codes are integers decided in fp32, so the codec computes in numpy float32 / float16, whose element-wise
operations and conversions are IEEE correctly rounded (round to nearest even).
"""

from __future__ import annotations

import numpy as np

GROUP = 32
LEVELS = 3  # codes 0..3
FP16_MAX = np.float16(65504.0)


def _sat16(v32):
    with np.errstate(over="ignore"):  # out-of-range values become +-inf, then saturate
        v16 = np.asarray(v32, dtype=np.float32).astype(np.float16)
    return np.where(np.isinf(v16), np.copysign(FP16_MAX, v16), v16).astype(np.float16)


def int2_offset(group_min):
    """Group offset z = fp16_rne(min x) of the group's fp32 minimum (saturating).  Returns float16."""
    return _sat16(group_min)


def int2_scale(group_max, z16):
    """Group scale s = fp16_rne(max(max x - z, 0) / 3) from the group's fp32 maximum and its fp16 offset (fp32
    subtraction, IEEE fp32 division, saturating).  Returns float16."""
    z32 = np.asarray(z16, dtype=np.float16).astype(np.float32)
    span = np.maximum(np.asarray(group_max, dtype=np.float32) - z32, np.float32(0.0))
    return _sat16(span / np.float32(LEVELS))


def int2_codes(x, s16, z16):
    """Codes of fp32 values x [..., 32] under their group's (s, z): clamp(rint_half_even((x - z) / s), 0, 3)
    in fp32 (subtraction, IEEE division); a zero scale gives zero codes.  Returns uint8."""
    g = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    z32 = np.asarray(z16, dtype=np.float16).astype(np.float32)[..., None]
    q = np.divide(g - z32, np.where(s32 > 0, s32, np.float32(1.0)), dtype=np.float32)
    return np.where(np.broadcast_to(s32 > 0, g.shape), np.clip(np.rint(q), 0, LEVELS), 0).astype(np.uint8)


def quantize_int2_g32(x):
    """x: fp32 array [..., n*32].  Returns (codes uint8 [..., n*32] in 0..3, meta float16 [..., n, 2] = (s, z))."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    g = x.reshape(-1, GROUP)
    z16 = int2_offset(np.min(g, axis=1))
    s16 = int2_scale(np.max(g, axis=1), z16)
    codes = int2_codes(g, s16, z16)
    meta = np.stack([s16, z16], axis=1)
    return codes.reshape(shp), meta.reshape(shp[:-1] + (shp[-1] // GROUP, 2))


def pack_crumbs(codes):
    """uint8 codes [..., 4m] in 0..3 -> uint8 [..., m]; element 4i + j at bits 2j, 2j+1 of byte i."""
    c = np.asarray(codes).astype(np.uint16)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_crumbs(packed):
    """uint8 [..., m] -> codes [..., 4m]."""
    p = np.asarray(packed).astype(np.uint16)
    out = np.empty(p.shape[:-1] + (4 * p.shape[-1],), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (p >> (2 * j)) & 3
    return out


def dequant_int2(codes, meta):
    """fp32_rne(z + code * s) per element, returned as fp64 (the fp32 values exactly)."""
    c = np.asarray(codes, dtype=np.float64)
    m = np.asarray(meta, dtype=np.float16).astype(np.float64)
    shp = c.shape
    g = c.reshape(-1, GROUP)
    s = m.reshape(-1, 2)[:, 0:1]
    z = m.reshape(-1, 2)[:, 1:2]
    exact = z + g * s  # exact in fp64: both terms lie on the fp16 grid
    return exact.astype(np.float32).astype(np.float64).reshape(shp)


def window_len(L, W):
    """Number of bf16 rows of a sequence of L tokens under window W."""
    return min(L, W)


def windowed_latent(rows_bf16, W):
    """The latent rows that attention reads for one sequence of L = len(rows_bf16) tokens.

    rows_bf16: [L, d_kv] values already on the bf16 grid (fp64 or fp32).  Rows older than the last
    min(L, W) are replaced by the dequantised 2-bit codes of their bf16 values.
    Returns (rows [L, d_kv] fp64, codes [L - min(L, W), d_kv], meta [L - min(L, W), d_kv/32, 2])."""
    x = np.asarray(rows_bf16, dtype=np.float32)
    L = x.shape[0]
    nq = L - window_len(L, W)
    codes, meta = quantize_int2_g32(x[:nq]) if nq > 0 else (np.zeros((0, x.shape[1]), np.uint8),
                                                              np.zeros((0, x.shape[1] // GROUP, 2), np.float16))
    out = x.astype(np.float64)
    if nq > 0:
        out[:nq] = dequant_int2(codes, meta)
    return out, codes, meta


def ring_positions(L, W):
    """Position held by each of the W ring slots after L tokens (-1: slot not yet used or stale)."""
    pos = np.full(W, -1, dtype=np.int64)
    for p in range(L - window_len(L, W), L):
        pos[p % W] = p
    return pos
