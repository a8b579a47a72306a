"""Conversion errors along the pages' ablation axes (oracle; test infrastructure only).

The Paper-Notes ACL2025 page on MHA2MLA (ablation tables) ranks the partial-RoPE strategies S_high,
S_low, S_uniform and S_2-norm, and SVD_split against SVD_joint, by the perplexity a converted model
recovers after fine-tuning.  Without training data or weights, the comparable quantities are the
errors that the conversion itself makes, before any fine-tuning, on a seeded layer:

* dropped score   -- share of a head's summed 2-norm scores (the Cauchy-Schwarz bounds of the
                     key-designs section) that falls on subspaces losing RoPE, mean over heads;
* partial-RoPE    -- causal attention with RoPE on the kept subspaces only, at full rank, against
                     full-RoPE MHA (relative L2 of the per-head outputs);
* K/V fit         -- ||M - W_dkv Z||_F / ||M||_F for M = [W_k,nope | W_v] and Z the up-projections;
* end to end      -- the converted layer's attention (latent cache, unabsorbed) against full-RoPE MHA.

Run as `python -m oracle.ablation [--family llama] [--r 4] [--d-kv 512] [--tokens 512] [--iid]`
from the repository root; it prints one table row per (strategy, SVD variant).  `--gqa llama3` measures a
grouped-query source layer instead (synth.GQA_FAMILIES; the reference is its own grouped-query attention,
the conversion convert_gqa_layer), for the 2-norm strategy and the joint SVD.
"""

from __future__ import annotations

import argparse
import time

import numpy as np

from .attention import append_ref, prefill_ref, rope_rotate
from .convert import (calibration_qk, convert_gqa_layer, convert_layer, group_of, pair_scores,
                      select_pairs_by)

STRATEGIES = ("2-norm", "high", "uniform", "low")
SVDS = ("joint", "split")


def mha_ref(x, w_q, w_k, w_v, n_heads, d_head, theta, kept=None):
    """Causal multi-head attention of tokens x [T, d] at positions 0..T-1 with RoPE on the subspaces
    kept[h] of head h (every subspace when kept is None), scale 1/sqrt(d_head).  [T, n_heads, d_head]."""
    t = x.shape[0]
    pos = np.arange(t, dtype=np.float64)
    out = np.zeros((t, n_heads, d_head))
    causal = np.tril(np.ones((t, t), dtype=bool))
    for h in range(n_heads):
        cols = slice(h * d_head, (h + 1) * d_head)
        q, k, v = x @ w_q[:, cols], x @ w_k[:, cols], x @ w_v[:, cols]
        pairs = range(d_head // 2) if kept is None else kept[h]
        for p in pairs:
            p = int(p)
            phi = pos * theta ** (-2.0 * p / d_head)
            q[:, 2 * p], q[:, 2 * p + 1] = rope_rotate(q[:, 2 * p], q[:, 2 * p + 1], phi)
            k[:, 2 * p], k[:, 2 * p + 1] = rope_rotate(k[:, 2 * p], k[:, 2 * p + 1], phi)
        s = np.where(causal, (q @ k.T) / np.sqrt(d_head), -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out


def gqa_ref(x, w_q, w_k, w_v, n_heads, n_kv, d_head, theta, kept=None):
    """Grouped-query attention: mha_ref with each query head reading its group's K and V columns (kept[g]:
    the RoPE subspaces of KV head g, all when None)."""
    grp = [group_of(h, n_heads, n_kv) for h in range(n_heads)]

    def expand(w):
        return np.concatenate([w[:, g * d_head:(g + 1) * d_head] for g in grp], axis=1)

    kept_h = None if kept is None else [kept[g] for g in grp]
    return mha_ref(x, w_q, expand(w_k), expand(w_v), n_heads, d_head, theta, kept=kept_h)


def gqa_rows(w_q, w_k, w_v, x_cal, x_eval, n_heads, n_kv, d_head, r, d_kv, theta=1e4):
    """The four errors for the grouped-query conversion (2-norm subspaces per KV head, joint SVD)."""
    full = gqa_ref(x_eval, w_q, w_k, w_v, n_heads, n_kv, d_head, theta)
    conv = convert_gqa_layer(w_q, w_k, w_v, x_cal, n_heads, n_kv, d_head, r, d_kv)
    kept = conv["group_pair_idx"]
    m = conv["m"]
    z = np.concatenate([np.concatenate(list(conv["group_w_uk"]), axis=1),
                        np.concatenate(list(conv["group_w_uv"]), axis=1)], axis=1)
    return [dict(strategy="2-norm", svd="joint", dropped_score=dropped_score(conv["scores"], kept),
                 partial_rope_err=rel_l2(gqa_ref(x_eval, w_q, w_k, w_v, n_heads, n_kv, d_head, theta, kept=kept), full),
                 kv_fit_err=float(np.linalg.norm(m - conv["w_dkv"] @ z) / np.linalg.norm(m)),
                 end_to_end_err=rel_l2(converted_ref(x_eval, w_q, conv, d_head, theta), full))]


def converted_ref(x, w_q, conv, d_head, theta):
    """Attention of the converted layer over its own latent cache of x (positions 0..T-1)."""
    t = x.shape[0]
    n_heads = conv["pair_idx"].shape[0]
    c_kv, k_rope = append_ref(x, conv["w_dkv"], conv["w_krope"], conv["pair_idx"], np.arange(t), d_head, theta)
    q = (x @ w_q).reshape(t, n_heads, d_head)
    return prefill_ref(q, c_kv, k_rope, conv["w_uk"], conv["w_uv"], conv["pair_idx"], d_head, theta)


def dropped_score(scores, pair_idx):
    """Mean over heads of the share of the head's summed scores on subspaces that are not kept."""
    shares = []
    for h in range(scores.shape[0]):
        total = scores[h].sum()
        shares.append((total - scores[h, list(pair_idx[h])].sum()) / total)
    return float(np.mean(shares))


def kv_fit_error(conv, n_heads):
    """||M - W_dkv [W_uk,1 .. W_uk,n | W_uv,1 .. W_uv,n]||_F / ||M||_F (M as the conversion built it)."""
    z = np.concatenate([np.concatenate(list(conv["w_uk"]), axis=1), np.concatenate(list(conv["w_uv"]), axis=1)], axis=1)
    m = conv["m"]
    return float(np.linalg.norm(m - conv["w_dkv"] @ z) / np.linalg.norm(m))


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def ablation_rows(w_q, w_k, w_v, x_cal, x_eval, n_heads, d_head, r, d_kv, theta=1e4,
                  strategies=STRATEGIES, svds=SVDS):
    """One dict per (strategy, SVD variant) with the four errors above."""
    full = mha_ref(x_eval, w_q, w_k, w_v, n_heads, d_head, theta)
    scores = pair_scores(*calibration_qk(x_cal, w_q, w_k, n_heads, d_head))
    rows = []
    for strategy in strategies:
        kept = select_pairs_by(strategy, scores, r)
        partial = rel_l2(mha_ref(x_eval, w_q, w_k, w_v, n_heads, d_head, theta, kept=kept), full)
        for svd in svds:
            conv = convert_layer(w_q, w_k, w_v, x_cal, n_heads, d_head, r, d_kv, strategy=strategy, svd=svd)
            rows.append(dict(strategy=strategy, svd=svd, dropped_score=dropped_score(scores, kept),
                             partial_rope_err=partial, kv_fit_err=kv_fit_error(conv, n_heads),
                             end_to_end_err=rel_l2(converted_ref(x_eval, w_q, conv, d_head, theta), full)))
    return rows


def main(argv=None):
    import synth  # seeded inputs, only when run as a script

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--family", default="llama")
    ap.add_argument("--r", type=int, default=4)
    ap.add_argument("--d-kv", type=int, default=512)
    ap.add_argument("--tokens", type=int, default=512)
    ap.add_argument("--iid", action="store_true", help="i.i.d. N(0, 0.02^2) weights instead of the structured layer")
    ap.add_argument("--gqa", default=None, help="a grouped-query family of synth.GQA_FAMILIES (i.i.d. weights)")
    args = ap.parse_args(argv)
    t0 = time.time()
    if args.gqa:
        d, n_h, n_kv, d_h, _ = synth.GQA_FAMILIES[args.gqa]
        wq, wk, wv, xc = synth.gqa_layer_weights(args.gqa)
        x = np.random.default_rng(0).standard_normal((args.tokens, d))
        rows = gqa_rows(wq, wk, wv, xc, x, n_h, n_kv, d_h, args.r, args.d_kv)
        print(f"grouped-query family {args.gqa} (d={d}, n_h={n_h}, n_kv={n_kv}, d_h={d_h}), r={args.r}, "
              f"d_kv={args.d_kv}, {args.tokens} tokens, {time.time() - t0:.0f} s")
    else:
        d, n_h, d_h, _ = synth.FAMILIES[args.family]
        wq, wk, wv, xc = (synth.layer_weights if args.iid else synth.structured_layer_weights)(args.family)
        x = synth.eval_x(args.family, args.tokens)
        rows = ablation_rows(wq, wk, wv, xc, x, n_h, d_h, args.r, args.d_kv)
        print(f"family {args.family} (d={d}, n_h={n_h}, d_h={d_h}), r={args.r}, d_kv={args.d_kv}, "
              f"{args.tokens} tokens, {'iid' if args.iid else 'structured'} weights, {time.time() - t0:.0f} s")
    print("| strategy | SVD | dropped score | partial-RoPE err | K/V fit err | end-to-end err |")
    print("|---|---|---|---|---|---|")
    for row in rows:
        print(f"| {row['strategy']} | {row['svd']} | {row['dropped_score']:.4f} | {row['partial_rope_err']:.4f} | "
              f"{row['kv_fit_err']:.4f} | {row['end_to_end_err']:.4f} |")


if __name__ == "__main__":
    main()
