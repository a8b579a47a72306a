"""Offline MHA -> MLA conversion of one layer (host, fp64 numpy).

Implements the two steps of the MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计):
  * contribution-aware partial RoPE: per head, keep the r subspaces [2p, 2p+1] with the largest
    2-norm score ||q^[2p,2p+1]|| * ||k^[2p,2p+1]|| (averaged over calibration tokens; ties to the
    lower index), the other subspaces become NoPE dimensions;
  * joint low-rank approximation: the best rank-d_kv approximation of [W_k,nope | W_v] (all heads'
    NoPE key columns, then all value columns); W_dkv spans its top-d_kv left singular subspace
    (orthonormal columns) and the up-projections are W_dkv^T [W_k,nope | W_v] split per head.

The subspace is found from the eigen-decomposition of the smaller Gram matrix, which gives the same
truncated factorisation as an SVD up to the signs of the basis vectors.  This runs once per layer,
outside the inference path.
"""

from __future__ import annotations

import numpy as np


def pair_scores(x_cal, w_q, w_k, n_heads, d_head):
    """[n_heads, d_head/2] scores: mean pair norm of q times mean pair norm of k over calibration tokens."""
    t = x_cal.shape[0]
    qn = np.hypot(*np.moveaxis((x_cal @ w_q).reshape(t, n_heads, d_head // 2, 2), -1, 0))
    kn = np.hypot(*np.moveaxis((x_cal @ w_k).reshape(t, n_heads, d_head // 2, 2), -1, 0))
    return qn.mean(axis=0) * kn.mean(axis=0)


def top_pairs(scores, r):
    """Per head the r best subspaces (largest score, ties to the lower index), ascending, int32."""
    n_heads, n_pairs = scores.shape
    idx = np.arange(n_pairs)
    out = np.empty((n_heads, r), dtype=np.int32)
    for h in range(n_heads):
        order = np.lexsort((idx, -scores[h]))
        out[h] = np.sort(order[:r])
    return out


def low_rank_factors(m, rank):
    """Orthonormal basis u [rows, rank] of the top-`rank` left singular subspace of m and the
    singular values (descending), via the Gram matrix's symmetric eigen-decomposition."""
    rows, cols = m.shape
    if rows <= cols:
        w, v = np.linalg.eigh(m @ m.T)
        order = np.argsort(w)[::-1]
        sig = np.sqrt(np.clip(w[order], 0.0, None))
        u = v[:, order[:rank]]
    else:
        w, v = np.linalg.eigh(m.T @ m)
        order = np.argsort(w)[::-1]
        sig = np.sqrt(np.clip(w[order], 0.0, None))
        u = (m @ v[:, order[:rank]]) / sig[:rank]
    return u, sig


def convert_layer(w_q, w_k, w_v, x_cal, n_heads, d_head, r, d_kv):
    """Returns the converted layer in math layouts:
    pair_idx [n_h, r], w_dkv [d, d_kv], w_krope [d, n_h*2r], w_uk [n_h, d_kv, d_h-2r], w_uv [n_h, d_kv, d_h],
    sigma (all singular values of [W_k,nope | W_v])."""
    pair_idx = top_pairs(pair_scores(x_cal, w_q, w_k, n_heads, d_head), r)
    d = w_k.shape[0]
    wk = w_k.reshape(d, n_heads, d_head // 2, 2)
    keep = np.zeros((n_heads, d_head // 2), dtype=bool)
    for h in range(n_heads):
        keep[h, pair_idx[h]] = True
    w_krope = np.stack([wk[:, h, pair_idx[h], :] for h in range(n_heads)], axis=1).reshape(d, n_heads * 2 * r)
    w_knope = np.stack([wk[:, h, ~keep[h], :].reshape(d, -1) for h in range(n_heads)], axis=1).reshape(d, -1)
    m = np.hstack([w_knope, w_v])
    u, sig = low_rank_factors(m, d_kv)
    z = u.T @ m
    dn = d_head - 2 * r
    w_uk = z[:, : n_heads * dn].reshape(d_kv, n_heads, dn).transpose(1, 0, 2)
    w_uv = z[:, n_heads * dn:].reshape(d_kv, n_heads, d_head).transpose(1, 0, 2)
    return dict(pair_idx=pair_idx, w_dkv=u, w_krope=w_krope, w_uk=np.ascontiguousarray(w_uk),
                w_uv=np.ascontiguousarray(w_uv), sigma=sig)
