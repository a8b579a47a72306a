"""MHA -> MLA conversion of one attention layer (oracle; test infrastructure only).

Follows the Paper-Notes ACL2025 page on MHA2MLA, section 关键设计 ("key designs"):

1. Contribution-aware partial-RoPE.  RoPE splits q and k of a head into d_h/2
   two-dimensional subspaces [2k, 2k+1], each rotated at its own frequency.  The
   contribution of subspace k to the attention score is bounded (Cauchy-Schwarz)
   by ||q^[2k,2k+1]|| * ||k^[2k,2k+1]||; each head keeps RoPE on its top-r
   subspaces and the rest become NoPE dimensions.
2. Joint SVD.  The NoPE key projections of all heads and the value projections
   are concatenated, [W_k,nope ; W_v], and given a truncated SVD U S V^T.
   W_dkv = U_trunc is the down-projection to the latent c_kv, and S V^T is split
   per head into the up-projections W_uk and W_uv.

The ablation variants of the pages (partial-RoPE strategies S_high / S_low / S_uniform, and SVD_split
at the same latent width) are select_pairs_by and split_svd_layer.  Grouped-query source layers (the
pages convert Llama3-8B, a GQA model, as well as MHA ones) are convert_gqa_layer.

Readings where the page leaves a step open (each also listed in the design notes):
* scores aggregate over calibration tokens as the product of the mean pair norms,
  which is exactly the mean of the bound over every (query token, key token) pair;
* ties in the score go to the lower pair index; kept pairs are stored ascending;
* the concatenation is by columns: all heads' K_nope blocks, then all heads' V blocks;
* Sigma goes to the up-projections, so W_dkv has orthonormal columns.
"""

from __future__ import annotations

import numpy as np


def calibration_qk(x_cal, w_q, w_k, n_heads, d_head):
    """Per-head queries and keys of the calibration tokens, [T, n_heads, d_head], without RoPE.

    RoPE rotates each 2-D subspace, which leaves its 2-norm unchanged, so the pair norms
    (and hence the scores) are the same with or without it."""
    t = x_cal.shape[0]
    q = (x_cal @ w_q).reshape(t, n_heads, d_head)
    k = (x_cal @ w_k).reshape(t, n_heads, d_head)
    return q, k


def pair_scores(q, k):
    """2-norm contribution score s[h, p] of subspace p = dims (2p, 2p+1) of head h.

    s[h,p] = mean_t ||q_t^[2p,2p+1]|| * mean_t ||k_t^[2p,2p+1]||, the mean over all token pairs
    (m, n) of the Cauchy-Schwarz bound ||q_m^p|| * ||k_n^p||."""
    t, n_heads, d_head = q.shape
    n_pairs = d_head // 2
    s = np.zeros((n_heads, n_pairs))
    for h in range(n_heads):
        for p in range(n_pairs):
            qn = np.sqrt(q[:, h, 2 * p] ** 2 + q[:, h, 2 * p + 1] ** 2)
            kn = np.sqrt(k[:, h, 2 * p] ** 2 + k[:, h, 2 * p + 1] ** 2)
            s[h, p] = qn.mean() * kn.mean()
    return s


def select_pairs(scores, r):
    """Head-wise top-r subspaces by score (ties: lower index first), stored ascending, int32 [n_heads, r]."""
    n_heads, n_pairs = scores.shape
    out = np.zeros((n_heads, r), dtype=np.int32)
    for h in range(n_heads):
        order = sorted(range(n_pairs), key=lambda p: (-scores[h, p], p))
        out[h] = sorted(order[:r])
    return out


def select_pairs_by(strategy, scores, r):
    """Kept RoPE subspaces of every head under the partial-RoPE strategies the pages compare
    (README strategy list: S_high, S_uniform, S_2-norm, S_low; ablation table of the Paper-Notes page).

    Subspace p rotates at frequency theta^(-2p/d_h), which falls with p, so S_high keeps p = 0..r-1 and
    S_low keeps the last r.  S_uniform keeps r subspaces evenly spaced from p = 0 with stride (d_h/2)/r
    (reading: the page does not fix the offset).  S_2-norm is the head-wise top-r of the scores.
    All strategies but S_2-norm give every head the same subspaces.  int32 [n_heads, r], ascending."""
    n_heads, n_pairs = scores.shape
    if strategy == "2-norm":
        return select_pairs(scores, r)
    if strategy == "high":
        idx = list(range(r))
    elif strategy == "low":
        idx = list(range(n_pairs - r, n_pairs))
    elif strategy == "uniform":
        idx = [(k * n_pairs) // r for k in range(r)]
    else:
        raise ValueError(f"unknown partial-RoPE strategy {strategy!r}")
    return np.array([idx] * n_heads, dtype=np.int32)


def split_dims(pair_idx, d_head):
    """Per head: (rope dims, nope dims), both in ascending original order.

    rope(h) lists dims 2p, 2p+1 for p in pair_idx[h] (in slot order j = 0..r-1), nope(h) the rest."""
    rope, nope = [], []
    for h in range(pair_idx.shape[0]):
        rd = []
        for p in pair_idx[h]:
            rd += [2 * int(p), 2 * int(p) + 1]
        rope.append(rd)
        nope.append([i for i in range(d_head) if i not in set(rd)])
    return rope, nope


def _nope_and_rope_columns(w_k, pair_idx, n_heads, d_head):
    rope, nope = split_dims(pair_idx, d_head)
    w_knope = np.concatenate([w_k[:, [h * d_head + i for i in nope[h]]] for h in range(n_heads)], axis=1)
    w_krope = np.concatenate([w_k[:, [h * d_head + i for i in rope[h]]] for h in range(n_heads)], axis=1)
    return w_knope, w_krope


def joint_svd(w_k, w_v, pair_idx, n_heads, d_head, d_kv):
    """Truncated joint SVD of M = [W_k,nope | W_v] (columns: K_nope blocks of all heads, then V blocks).

    Returns W_dkv [d, d_kv], W_uk [n_heads, d_kv, d_head-2r], W_uv [n_heads, d_kv, d_head],
    W_krope [d, n_heads*2r] (kept RoPE columns of W_k packed (head, slot, 2)) and all singular values."""
    r = pair_idx.shape[1]
    dn = d_head - 2 * r
    w_knope, w_krope = _nope_and_rope_columns(w_k, pair_idx, n_heads, d_head)
    m = np.concatenate([w_knope, w_v], axis=1)
    u, sig, vt = np.linalg.svd(m, full_matrices=False)
    w_dkv = u[:, :d_kv]
    z = sig[:d_kv, None] * vt[:d_kv]
    w_uk = np.stack([z[:, h * dn:(h + 1) * dn] for h in range(n_heads)])
    off = n_heads * dn
    w_uv = np.stack([z[:, off + h * d_head: off + (h + 1) * d_head] for h in range(n_heads)])
    return dict(w_dkv=w_dkv, w_uk=w_uk, w_uv=w_uv, w_krope=w_krope, sigma=sig, m=m)


def split_svd(w_k, w_v, pair_idx, n_heads, d_head, rank_k, rank_v):
    """SVD_split baseline: separate truncated SVDs of W_k,nope (rank_k) and W_v (rank_v).

    Returns the two rank-truncated approximations (used to check that the joint SVD at the same
    total latent width is never worse)."""
    w_knope, _ = _nope_and_rope_columns(w_k, pair_idx, n_heads, d_head)

    def trunc(a, rank):
        u, s, vt = np.linalg.svd(a, full_matrices=False)
        return (u[:, :rank] * s[:rank]) @ vt[:rank]

    return trunc(w_knope, rank_k), trunc(w_v, rank_v), w_knope


def split_svd_layer(w_k, w_v, pair_idx, n_heads, d_head, d_kv):
    """SVD_split as an MLA layer of the same latent width (the pages' SVD ablation: separate SVDs of
    the NoPE keys and of the values, same cache size).  Reading: the latent is split evenly, d_kv/2
    dims from the truncated SVD of W_k,nope and d_kv - d_kv/2 from that of W_v:
        W_dkv = [U_k | U_v],  W_uk,h = [S_k V_k^T restricted to head h ; 0],  W_uv,h = [0 ; S_v V_v^T of head h],
    so keys read only the first half of c_kv and values only the second.  Same layouts as joint_svd."""
    r = pair_idx.shape[1]
    dn = d_head - 2 * r
    rk = d_kv // 2
    rv = d_kv - rk
    w_knope, w_krope = _nope_and_rope_columns(w_k, pair_idx, n_heads, d_head)
    if rk > min(w_knope.shape) or rv > min(w_v.shape):
        raise ValueError("SVD_split: d_kv/2 exceeds the rank W_k,nope or W_v can have")
    uk, sk, vtk = np.linalg.svd(w_knope, full_matrices=False)
    uv, sv, vtv = np.linalg.svd(w_v, full_matrices=False)
    w_dkv = np.concatenate([uk[:, :rk], uv[:, :rv]], axis=1)
    zk = sk[:rk, None] * vtk[:rk]
    zv = sv[:rv, None] * vtv[:rv]
    w_uk = np.stack([np.concatenate([zk[:, h * dn:(h + 1) * dn], np.zeros((rv, dn))]) for h in range(n_heads)])
    w_uv = np.stack([np.concatenate([np.zeros((rk, d_head)), zv[:, h * d_head:(h + 1) * d_head]]) for h in range(n_heads)])
    return dict(w_dkv=w_dkv, w_uk=w_uk, w_uv=w_uv, w_krope=w_krope, sigma_k=sk, sigma_v=sv,
                m=np.concatenate([w_knope, w_v], axis=1))


def group_of(h, n_heads, n_kv):
    """KV head (group) that query head h reads in a grouped-query layer: n_heads / n_kv consecutive heads each."""
    return h // (n_heads // n_kv)


def gqa_pair_scores(q, k, n_heads, n_kv):
    """[n_kv, d_head/2] scores of a grouped-query layer: for KV head g and subspace p, the mean over the query
    heads h of the group of the 2-norm score of (h, p) against the group's keys (q [T, n_heads, d_h],
    k [T, n_kv, d_h]).  Reading: the kept subspaces are cached once per KV head, so they are chosen per
    group, by the mean of the Cauchy-Schwarz bounds of the heads that read them."""
    t, _, d_head = q.shape
    n_pairs = d_head // 2
    s = np.zeros((n_kv, n_pairs))
    for g in range(n_kv):
        heads = [h for h in range(n_heads) if group_of(h, n_heads, n_kv) == g]
        for p in range(n_pairs):
            kn = np.sqrt(k[:, g, 2 * p] ** 2 + k[:, g, 2 * p + 1] ** 2).mean()
            acc = 0.0
            for h in heads:
                acc += np.sqrt(q[:, h, 2 * p] ** 2 + q[:, h, 2 * p + 1] ** 2).mean() * kn
            s[g, p] = acc / len(heads)
    return s


def convert_gqa_layer(w_q, w_k, w_v, x_cal, n_heads, n_kv, d_head, r, d_kv):
    """Conversion of a grouped-query layer (n_kv KV heads, each read by n_heads / n_kv query heads).

    Per KV head: top-r subspaces by gqa_pair_scores; joint SVD of [W_k,nope | W_v] over the n_kv KV heads
    (n_kv (d_h - 2r) + n_kv d_h columns).  The result is given per query head, in the layouts of
    convert_layer, so that it is an ordinary MLA layer: query head h takes its group's kept subspaces,
    RoPE key columns and up-projections (pair_idx [n_heads, r], w_krope [d, n_heads*2r] with each group's
    columns repeated for its heads, w_uk [n_heads, d_kv, d_h-2r], w_uv [n_heads, d_kv, d_h]).  The per-group
    factors are returned too (`group_*`)."""
    t = x_cal.shape[0]
    q = (x_cal @ w_q).reshape(t, n_heads, d_head)
    k = (x_cal @ w_k).reshape(t, n_kv, d_head)
    scores = gqa_pair_scores(q, k, n_heads, n_kv)
    gidx = select_pairs(scores, r)
    j = joint_svd(w_k, w_v, gidx, n_kv, d_head, d_kv)
    grp = [group_of(h, n_heads, n_kv) for h in range(n_heads)]
    two_r = 2 * r
    w_krope = np.concatenate([j["w_krope"][:, g * two_r:(g + 1) * two_r] for g in grp], axis=1)
    return dict(pair_idx=gidx[grp], w_dkv=j["w_dkv"], w_krope=w_krope, w_uk=j["w_uk"][grp], w_uv=j["w_uv"][grp],
                sigma=j["sigma"], m=j["m"], scores=scores, group_pair_idx=gidx, group_w_uk=j["w_uk"],
                group_w_uv=j["w_uv"], group_w_krope=j["w_krope"])


def convert_layer(w_q, w_k, w_v, x_cal, n_heads, d_head, r, d_kv, strategy="2-norm", svd="joint"):
    """Full conversion: calibration -> scores -> kept subspaces (S_2-norm by default, see
    select_pairs_by) -> joint SVD (or SVD_split, see split_svd_layer)."""
    q, k = calibration_qk(x_cal, w_q, w_k, n_heads, d_head)
    scores = pair_scores(q, k)
    pair_idx = select_pairs_by(strategy, scores, r)
    if svd == "joint":
        out = joint_svd(w_k, w_v, pair_idx, n_heads, d_head, d_kv)
    elif svd == "split":
        out = split_svd_layer(w_k, w_v, pair_idx, n_heads, d_head, d_kv)
    else:
        raise ValueError(f"unknown SVD variant {svd!r}")
    out.update(pair_idx=pair_idx, scores=scores)
    return out
