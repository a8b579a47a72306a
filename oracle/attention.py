"""Latent-cache append and attention over the latent cache (oracle; test infrastructure only).

Follows the Paper-Notes ACL2025 page on MHA2MLA, section 关键设计 ("key designs"):
the cache holds the latent c_kv = x . W_dkv shared by all heads plus, per head,
the keys of the retained RoPE subspaces; K_nope and V of a head are recovered
from c_kv through that head's up-projections W_uk and W_uv, and the RoPE part
is computed separately because it cannot be merged into the matrices.

RoPE: subspace p = dims (2p, 2p+1) of a head is rotated by the angle
pos * theta^(-2p/d_head) (the standard RoFormer rotation; the page names the
2-D subspaces and their distinct frequencies but not the formula).

attend_ref is the UNABSORBED definition: it rebuilds K and V of every head in
the original head-dimension order and applies plain causal softmax attention
with the 1/sqrt(d_head) scale.  absorbed_decode_ref is a separate function
written in the absorbed form only to pin that the two agree.
"""

from __future__ import annotations

import numpy as np

from .convert import split_dims


def rope_rotate(a, b, phi):
    """Rotate the 2-vector (a, b) by angle phi: (a cos phi - b sin phi, a sin phi + b cos phi)."""
    c, s = np.cos(phi), np.sin(phi)
    return a * c - b * s, a * s + b * c


def _freq(p, d_head, theta):
    return theta ** (-2.0 * p / d_head)


def append_ref(x, w_dkv, w_krope, pair_idx, positions, d_head, theta):
    """Cache rows for activations x [T, d] at the given absolute positions.

    c_kv [T, d_kv] = x . W_dkv.  k_rope [T, n_heads, 2r]: for head h and slot j the pre-RoPE pair
    (x . W_krope)[h, j, 0:2] rotated at position pos_t with the frequency of subspace pair_idx[h, j]."""
    n_heads, r = pair_idx.shape
    t = x.shape[0]
    c_kv = x @ w_dkv
    kpre = (x @ w_krope).reshape(t, n_heads, r, 2)
    k_rope = np.zeros((t, n_heads, r, 2))
    pos = np.asarray(positions, dtype=np.float64)
    for h in range(n_heads):
        for j in range(r):
            phi = pos * _freq(int(pair_idx[h, j]), d_head, theta)
            a, b = rope_rotate(kpre[:, h, j, 0], kpre[:, h, j, 1], phi)
            k_rope[:, h, j, 0] = a
            k_rope[:, h, j, 1] = b
    return c_kv, k_rope.reshape(t, n_heads, 2 * r)


def reconstruct_head(c_kv, k_rope, w_uk, w_uv, pair_idx, h, d_head):
    """Full keys and values of head h, [N, d_head] each, in the original head-dimension order.

    K[:, nope(h)] = c_kv . W_uk[h], K[:, rope(h)] = k_rope[:, h], V = c_kv . W_uv[h]."""
    rope, nope = split_dims(pair_idx, d_head)
    n = c_kv.shape[0]
    k = np.zeros((n, d_head))
    if nope[h]:
        k[:, nope[h]] = c_kv @ w_uk[h]
    k[:, rope[h]] = k_rope[:, h, :]
    v = c_kv @ w_uv[h]
    return k, v


def _rope_query(q_h, q_pos, pair_idx_h, d_head, theta):
    """Rotate only the retained subspaces of per-position query rows q_h [M, d_head]."""
    out = np.array(q_h, dtype=np.float64, copy=True)
    pos = np.asarray(q_pos, dtype=np.float64)
    for p in pair_idx_h:
        p = int(p)
        phi = pos * _freq(p, d_head, theta)
        out[:, 2 * p], out[:, 2 * p + 1] = rope_rotate(q_h[:, 2 * p], q_h[:, 2 * p + 1], phi)
    return out


def attend_ref(q, q_pos, c_kv, k_rope, key_pos, w_uk, w_uv, pair_idx, d_head, theta):
    """Causal attention of query rows q [M, n_heads, d_head] (raw, pre-RoPE) at positions q_pos over
    cached keys at positions key_pos.  Key n is visible to query m iff key_pos[n] <= q_pos[m].

    Returns out [M, n_heads, d_head]: per-head attention outputs (before the output projection)."""
    m_rows, n_heads, _ = q.shape
    key_pos = np.asarray(key_pos)
    q_pos = np.asarray(q_pos)
    out = np.zeros((m_rows, n_heads, d_head))
    visible = key_pos[None, :] <= q_pos[:, None]
    for h in range(n_heads):
        k, v = reconstruct_head(c_kv, k_rope, w_uk, w_uv, pair_idx, h, d_head)
        qh = _rope_query(q[:, h, :], q_pos, pair_idx[h], d_head, theta)
        s = (qh @ k.T) / np.sqrt(d_head)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v
    return out


def decode_ref(q, c_kv, k_rope, w_uk, w_uv, pair_idx, d_head, theta):
    """Decode for one sequence of L cached tokens: the query q [n_heads, d_head] is the token at
    position L-1 (already appended) and attends to positions 0..L-1."""
    length = c_kv.shape[0]
    out = attend_ref(q[None], [length - 1], c_kv, k_rope, np.arange(length), w_uk, w_uv, pair_idx, d_head, theta)
    return out[0]


def prefill_ref(q, c_kv, k_rope, w_uk, w_uv, pair_idx, d_head, theta, rows=None):
    """Causal prefill for one sequence starting at position 0: q [S, n_heads, d_head].
    `rows` optionally restricts the computed query positions (returns [len(rows), n_heads, d_head])."""
    s_len = q.shape[0]
    rows = np.arange(s_len) if rows is None else np.asarray(rows)
    return attend_ref(q[rows], rows, c_kv, k_rope, np.arange(s_len), w_uk, w_uv, pair_idx, d_head, theta)


def absorbed_decode_ref(q, c_kv, k_rope, w_uk, w_uv, pair_idx, d_head, theta):
    """Decode in the absorbed form (W_uk folded into the query, W_uv applied after the weighted sum
    of latents).  Same arguments and result as decode_ref; kept only to pin that the algebra holds."""
    rope, nope = split_dims(pair_idx, d_head)
    length = c_kv.shape[0]
    n_heads = q.shape[0]
    out = np.zeros((n_heads, d_head))
    for h in range(n_heads):
        qr = _rope_query(q[None, h, :], [length - 1], pair_idx[h], d_head, theta)[0]
        q_lat = w_uk[h] @ qr[nope[h]] if nope[h] else np.zeros(c_kv.shape[1])
        s = (c_kv @ q_lat + k_rope[:, h, :] @ qr[rope[h]]) / np.sqrt(d_head)
        p = np.exp(s - s.max())
        o_lat = (p @ c_kv) / p.sum()
        out[h] = o_lat @ w_uv[h]
    return out
