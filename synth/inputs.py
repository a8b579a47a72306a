"""Configurations, seeded random streams and device-dtype rounding.

Stream layout (numpy PCG64 seeded from a SeedSequence with an explicit spawn key):

* layer weights, keyed by shape family (tiny -> 0, mid -> 2, llama -> 1):
  spawn key (0,) W_q, (1,) W_k, (2,) W_v, each [d_model, n_heads*d_head] ~ N(0,1)*0.02;
  spawn key (3,) calibration activations X_cal [n_calib, d_model] ~ N(0,1);
  spawn keys (4,), (5,) the structured layer and its X_cal, (6,) evaluation activations
  (structured_layer_weights, eval_x).
* per-configuration inputs, entropy 100 + config index:
  spawn key (0,) per-sequence context lengths (variable-length configs only);
  spawn key (1, b) the activations x_b [L_b, d_model] ~ N(0,1) of sequence b.

Every tensor that crosses to the GPU is rounded to the device dtype here
(fp64 -> fp32 by IEEE round-to-nearest-even, then fp32 -> bf16 by RNE on the
bit pattern), and both sides consume exactly those rounded values.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# Shape families: (d_model, n_heads, d_head, weight-stream seed).
FAMILIES = {
    "tiny": (576, 9, 64, 0),  # SmolLM-135M-shaped layer
    "llama": (4096, 32, 128, 1),  # Llama-2-7B-shaped layer
    "mid": (1024, 32, 128, 2),  # Llama head shapes with a narrower model width (fast tests)
    "odd": (640, 5, 128, 3),  # Llama head dim, a head count that is not a multiple of 8 (tests)
    "head80": (640, 4, 80, 7),  # a head dim of five 16-wide blocks (tests)
}


@dataclass(frozen=True)
class Config:
    name: str
    index: int  # input-stream key (100 + index)
    family: str
    r_pairs: int
    d_kv: int
    dtype: str  # "f32" or "bf16": activations, weights and cache values
    cache_fmt: str  # "dense" or "int4_g32"
    mode: str  # "decode" or "prefill"
    batch: int
    context: int = 0  # fixed context (decode) or sequence length (prefill)
    ctx_range: Optional[Tuple[int, int]] = None  # inclusive range for variable lengths
    theta: float = 1e4
    n_calib: int = 64

    @property
    def d_model(self) -> int:
        return FAMILIES[self.family][0]

    @property
    def n_heads(self) -> int:
        return FAMILIES[self.family][1]

    @property
    def d_head(self) -> int:
        return FAMILIES[self.family][2]

    @property
    def family_seed(self) -> int:
        return FAMILIES[self.family][3]


CONFIGS = [
    Config("tiny_f32_decode", 0, "tiny", 4, 32, "f32", "dense", "decode", 1, 256),
    Config("llama_bf16_decode", 1, "llama", 4, 512, "bf16", "dense", "decode", 32, 4096),
    Config("llama_bf16_prefill", 2, "llama", 4, 512, "bf16", "dense", "prefill", 4, 4096),
    Config("llama_bf16_longctx_decode", 3, "llama", 2, 256, "bf16", "dense", "decode", 8, 0, (8192, 32768)),
    Config("llama_int4_decode", 4, "llama", 4, 512, "bf16", "int4_g32", "decode", 64, 8192),
]


def scaled(cfg: Config, **changes) -> Config:
    """A copy of `cfg` with some fields replaced (smaller batch, context, family ...)."""
    return dataclasses.replace(cfg, **changes)


def _gen(entropy: int, key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy, spawn_key=key)))


def layer_weights(family: str):
    """W_q, W_k, W_v [d_model, n_heads*d_head] ~ N(0, 0.02^2) and X_cal [64, d_model] ~ N(0,1), fp64."""
    d, n_h, d_h, seed = FAMILIES[family]
    w = [_gen(seed, (i,)).standard_normal((d, n_h * d_h)) * 0.02 for i in range(3)]
    x_cal = _gen(seed, (3,)).standard_normal((64, d))
    return w[0], w[1], w[2], x_cal


# Grouped-query shape families: (d_model, n_heads, n_kv_heads, d_head, weight-stream seed).
GQA_FAMILIES = {
    "gqa_mid": (1024, 32, 8, 128, 5),  # Llama head shapes, 8 KV heads, narrow model width (tests)
    "llama3": (4096, 32, 8, 128, 6),  # Llama-3-8B-shaped attention layer
}


def gqa_layer_weights(family: str):
    """W_q [d, n_heads*d_head], W_k, W_v [d, n_kv*d_head] ~ N(0, 0.02^2) and X_cal [64, d] ~ N(0, 1), fp64
    (stream keys (0,) .. (3,) of the family's seed, as layer_weights)."""
    d, n_h, n_kv, d_h, seed = GQA_FAMILIES[family]
    wq = _gen(seed, (0,)).standard_normal((d, n_h * d_h)) * 0.02
    wk = _gen(seed, (1,)).standard_normal((d, n_kv * d_h)) * 0.02
    wv = _gen(seed, (2,)).standard_normal((d, n_kv * d_h)) * 0.02
    x_cal = _gen(seed, (3,)).standard_normal((64, d))
    return wq, wk, wv, x_cal


def structured_layer_weights(family: str):
    """W_q, W_k, W_v [d_model, n_heads*d_head] and X_cal [64, d_model] (fp64) with two kinds of structure
    that i.i.d. weights lack (stream keys (4,) for the weights, (5,) for X_cal of the family's seed):

    * a shared input subspace: each W = A diag(s) G_W + 0.05 N_W with one A [d, d/4] ~ N(0, 1/d) for all
      three, s_i = exp(-3 i / (d/4)), and G_W, N_W ~ N(0, 1) of their own;
    * a frequency band per head: the q and k columns of subspace p (dims 2p, 2p+1) of head h are scaled by
      0.25 + 2 exp(-((p - c_h) / w)^2 / 2), c_h ~ uniform over the d_head/2 subspaces, w = d_head/32.
    Each W is then scaled to an entry RMS of 0.02."""
    d, n_h, d_h, seed = FAMILIES[family]
    g = _gen(seed, (4,))
    rho = d // 4
    a = g.standard_normal((d, rho)) / np.sqrt(d)
    spec = np.exp(-3.0 * np.arange(rho) / rho)
    ws = []
    for _ in range(3):
        ws.append((a * spec) @ g.standard_normal((rho, n_h * d_h)) + 0.05 * g.standard_normal((d, n_h * d_h)) / np.sqrt(d))
    n_pairs = d_h // 2
    centre = g.integers(0, n_pairs, size=n_h)
    p = np.arange(n_pairs)
    gain = 0.25 + 2.0 * np.exp(-0.5 * ((p[None, :] - centre[:, None]) / (d_h / 32)) ** 2)  # [n_h, n_pairs]
    col_gain = np.repeat(gain, 2, axis=1).reshape(n_h * d_h)
    ws[0] = ws[0] * col_gain
    ws[1] = ws[1] * col_gain
    ws = [w * (0.02 / np.sqrt(np.mean(w * w))) for w in ws]
    x_cal = _gen(seed, (5,)).standard_normal((64, d))
    return ws[0], ws[1], ws[2], x_cal


def eval_x(family: str, length: int) -> np.ndarray:
    """Evaluation activations [length, d_model] ~ N(0, 1), fp64 (stream key (6,) of the family's seed)."""
    d = FAMILIES[family][0]
    return _gen(FAMILIES[family][3], (6,)).standard_normal((length, d))


def seq_lens(cfg: Config) -> np.ndarray:
    """Per-sequence context lengths (int64): fixed, or uniform over cfg.ctx_range inclusive."""
    if cfg.ctx_range is None:
        return np.full(cfg.batch, cfg.context, dtype=np.int64)
    lo, hi = cfg.ctx_range
    return _gen(100 + cfg.index, (0,)).integers(lo, hi, size=cfg.batch, endpoint=True)


def context_x(cfg: Config, b: int, length: int) -> np.ndarray:
    """Activations x_b [length, d_model] ~ N(0,1) of sequence b, already rounded to the device dtype
    and returned as fp64 (exact)."""
    x = _gen(100 + cfg.index, (1, b)).standard_normal((length, cfg.d_model), dtype=np.float32)
    return round_to_device(x, cfg.dtype)


def query_rows(x_rows: np.ndarray, w_q: np.ndarray, dtype: str) -> np.ndarray:
    """Raw (pre-RoPE) queries q = x . W_q for the given activation rows, rounded to the device dtype.

    The query projection sits upstream of the method (q is an input of decode and prefill); it is
    computed in fp32 for bf16 configurations and in fp64 for fp32 ones, then rounded."""
    if dtype == "f32":
        q = x_rows @ w_q
    else:
        q = x_rows.astype(np.float32) @ w_q.astype(np.float32)
    return round_to_device(q, dtype)


# ---------------------------------------------------------------- rounding

def bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns (uint16) of `a`: fp64 -> fp32 (RNE) -> bf16 (RNE on the bits).  Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bit patterns."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_device(a, dtype: str) -> np.ndarray:
    """Values of `a` after rounding to the device dtype, returned exactly as fp64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bits_to_f64(bf16_bits(a))
    if dtype == "f16":
        return np.asarray(np.asarray(a, dtype=np.float32), dtype=np.float16).astype(np.float64)
    raise ValueError(dtype)
