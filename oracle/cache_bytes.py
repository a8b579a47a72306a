"""KV-cache bytes per token per layer (oracle; test infrastructure only).

Plain MHA caches keys and values of every head, 2 * n_heads * d_head elements per
token (Paper-Notes ACL2025 page on MHA2MLA, section 研究背景与动机, cache size
O(2 l n_h d_h)).  The latent cache holds d_kv latent elements plus 2r RoPE key
elements per head (section 关键设计); a group-quantised latent also stores one
fp16 scale per group.
"""

from __future__ import annotations


def mha_bytes_per_token(n_heads, d_head, elem_bytes=2):
    return 2 * n_heads * d_head * elem_bytes


def cache_bytes_per_token(n_heads, r_pairs, d_kv, latent_bits=16, rope_bytes=2, group=32, scale_bytes=0):
    """Latent-cache bytes per token: d_kv latent values at latent_bits each, n_heads*2r RoPE key values,
    and (for a grouped quantised latent) scale_bytes per group of `group` latent values."""
    latent = d_kv * latent_bits / 8
    scales = (d_kv // group) * scale_bytes if scale_bytes else 0
    return latent + n_heads * 2 * r_pairs * rope_bytes + scales


def reduction_pct(cache_bytes, mha_bytes):
    return 100.0 * (1.0 - cache_bytes / mha_bytes)
