"""Offline MHA -> MLA conversion of one layer (host, fp64 numpy).

Implements the two steps of the MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计):
  * contribution-aware partial RoPE: per head, keep the r subspaces [2p, 2p+1] with the largest
    2-norm score ||q^[2p,2p+1]|| * ||k^[2p,2p+1]|| (averaged over calibration tokens; ties to the
    lower index), the other subspaces become NoPE dimensions;
  * joint low-rank approximation: the best rank-d_kv approximation of [W_k,nope | W_v] (all heads'
    NoPE key columns, then all value columns); W_dkv spans its top-d_kv left singular subspace
    (orthonormal columns) and the up-projections are W_dkv^T [W_k,nope | W_v] split per head.

The pages' ablation variants are options of convert_layer: the fixed partial-RoPE strategies S_high,
S_low and S_uniform (kept_pairs), and SVD_split at the same latent width; n_kv_heads converts a
grouped-query source layer (the pages convert Llama3-8B, a GQA model).

The subspace is found from the eigen-decomposition of the smaller Gram matrix, which gives the same
truncated factorisation as an SVD up to the signs of the basis vectors.  This runs once per layer,
outside the inference path.
"""

from __future__ import annotations

import numpy as np


def pair_scores(x_cal, w_q, w_k, n_heads, d_head, n_kv=None):
    """[n_kv, d_head/2] scores: mean pair norm of q times mean pair norm of k over calibration tokens; with
    grouped-query keys (n_kv < n_heads) the q factor is averaged over the n_heads / n_kv heads of a group."""
    n_kv = n_heads if n_kv is None else n_kv
    t = x_cal.shape[0]
    qn = np.hypot(*np.moveaxis((x_cal @ w_q).reshape(t, n_heads, d_head // 2, 2), -1, 0)).mean(axis=0)
    kn = np.hypot(*np.moveaxis((x_cal @ w_k).reshape(t, n_kv, d_head // 2, 2), -1, 0)).mean(axis=0)
    return qn.reshape(n_kv, n_heads // n_kv, d_head // 2).mean(axis=1) * kn


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


def kept_pairs(strategy, scores, r):
    """Kept RoPE subspaces [n_h, r] (ascending, int32) under one of the partial-RoPE strategies the pages
    compare (README strategy list; ablation table of the Paper-Notes page).  Subspace p turns at
    frequency theta^(-2p/d_h), decreasing in p:
      "2-norm"  -- head-wise top-r by score (the method's own choice),
      "high"    -- the r highest frequencies, p = 0 .. r-1, for every head,
      "low"     -- the r lowest, p = d_h/2 - r .. d_h/2 - 1,
      "uniform" -- every (d_h/2)/r-th subspace from p = 0, p_k = floor(k d_h / (2r))."""
    n_heads, n_pairs = scores.shape
    if strategy == "2-norm":
        return top_pairs(scores, r)
    table = {
        "high": np.arange(r),
        "low": np.arange(n_pairs - r, n_pairs),
        "uniform": np.arange(r) * n_pairs // max(r, 1),
    }
    if strategy not in table:
        raise ValueError(f"unknown partial-RoPE strategy {strategy!r}; expected one of 2-norm, high, low, uniform")
    return np.broadcast_to(table[strategy].astype(np.int32), (n_heads, r)).copy()


def _factor(w_k, w_v, pair_idx, n_kv, d_head, d_kv, svd):
    """Kept RoPE columns and the low-rank factors of one layer whose keys and values have n_kv heads."""
    r = pair_idx.shape[1]
    d = w_k.shape[0]
    wk = w_k.reshape(d, n_kv, d_head // 2, 2)
    keep = np.zeros((n_kv, d_head // 2), dtype=bool)
    for h in range(n_kv):
        keep[h, pair_idx[h]] = True
    w_krope = np.stack([wk[:, h, pair_idx[h], :] for h in range(n_kv)], axis=1).reshape(d, n_kv * 2 * r)
    w_knope = np.stack([wk[:, h, ~keep[h], :].reshape(d, -1) for h in range(n_kv)], axis=1).reshape(d, -1)
    dn = d_head - 2 * r
    out = dict(w_krope=w_krope)
    if svd == "joint":
        m = np.hstack([w_knope, w_v])
        u, sig = low_rank_factors(m, d_kv)
        z = u.T @ m
        w_uk = z[:, : n_kv * dn].reshape(d_kv, n_kv, dn).transpose(1, 0, 2)
        w_uv = z[:, n_kv * dn:].reshape(d_kv, n_kv, d_head).transpose(1, 0, 2)
        out.update(w_dkv=u, sigma=sig)
    elif svd == "split":
        rk = d_kv // 2
        if rk > min(w_knope.shape) or d_kv - rk > min(w_v.shape):
            raise ValueError("svd='split': d_kv/2 exceeds the rank W_k,nope or W_v can have")
        uk, sig_k = low_rank_factors(w_knope, rk)
        uv, sig_v = low_rank_factors(w_v, d_kv - rk)
        w_uk = np.zeros((n_kv, d_kv, dn))
        w_uv = np.zeros((n_kv, d_kv, d_head))
        w_uk[:, :rk, :] = (uk.T @ w_knope).reshape(rk, n_kv, dn).transpose(1, 0, 2)
        w_uv[:, rk:, :] = (uv.T @ w_v).reshape(d_kv - rk, n_kv, d_head).transpose(1, 0, 2)
        out.update(w_dkv=np.hstack([uk, uv]), sigma_k=sig_k, sigma_v=sig_v)
    else:
        raise ValueError(f"unknown SVD variant {svd!r}; expected joint or split")
    out.update(w_uk=np.ascontiguousarray(w_uk), w_uv=np.ascontiguousarray(w_uv))
    return out


def convert_layer(w_q, w_k, w_v, x_cal, n_heads, d_head, r, d_kv, strategy="2-norm", svd="joint", n_kv_heads=None,
                  compact_rope=False):
    """Returns the converted layer in math layouts:
    pair_idx [n_h, r], w_dkv [d, d_kv], w_krope [d, n_h*2r], w_uk [n_h, d_kv, d_h-2r], w_uv [n_h, d_kv, d_h],
    and the singular values: sigma (all of [W_k,nope | W_v]) for the joint SVD, sigma_k / sigma_v (of W_k,nope
    and of W_v) for the split one.

    svd="joint" is the method's joint low-rank step.  svd="split" is the SVD_split ablation at the same latent
    width: the first d_kv/2 latent dims span the top left singular subspace of W_k,nope alone and the other
    d_kv - d_kv/2 that of W_v alone, so W_uk is zero on the value half and W_uv on the key half; the
    result is an ordinary MLA layer that the attention kernels run unchanged.

    n_kv_heads < n_heads converts a grouped-query layer (w_k, w_v [d, n_kv*d_h]; query head h reads KV head
    h // (n_heads / n_kv)): subspaces are kept per KV head by the group's mean score, the low-rank step runs
    over the n_kv heads' columns, and the result is expanded per query head (each head takes its group's
    kept subspaces, RoPE key columns and up-projections; the per-group factors are under `group_*`).  With
    compact_rope the RoPE part stays per KV head instead: pair_idx [n_kv, r] and w_krope [d, n_kv*2r], the
    layout of a cache that stores each group's RoPE keys once (LayerShape.rope_heads = n_kv)."""
    n_kv = n_heads if n_kv_heads is None else int(n_kv_heads)
    if n_kv <= 0 or n_heads % n_kv:
        raise ValueError("n_kv_heads must divide n_heads")
    scores = pair_scores(x_cal, w_q, w_k, n_heads, d_head, n_kv)
    pair_idx = kept_pairs(strategy, scores, r)
    f = _factor(w_k, w_v, pair_idx, n_kv, d_head, d_kv, svd)
    if n_kv == n_heads:
        f.update(pair_idx=pair_idx, scores=scores)
        return f
    grp = np.arange(n_heads) // (n_heads // n_kv)
    d = w_k.shape[0]
    out = dict(f)
    out.update(pair_idx=pair_idx[grp], scores=scores, group_pair_idx=pair_idx,
               w_krope=f["w_krope"].reshape(d, n_kv, 2 * r)[:, grp, :].reshape(d, n_heads * 2 * r),
               w_uk=np.ascontiguousarray(f["w_uk"][grp]), w_uv=np.ascontiguousarray(f["w_uv"][grp]),
               group_w_uk=f["w_uk"], group_w_uv=f["w_uv"], group_w_krope=f["w_krope"])
    if compact_rope:
        out.update(pair_idx=pair_idx, w_krope=f["w_krope"])
    return out
