"""Paged latent cache and multi-query decode (oracle; test infrastructure only).

The MHA2MLA GitHub README page (TO-DO list) names FlashMLA, a paged-cache MLA decoder, with KV-cache
quantisation as the direction for serving converted models.  A paged cache only changes where a sequence's rows
are stored, and multi-query decode (several new tokens of one sequence attending at once, each to the
positions up to its own) is causal attention over the same rows; both are written here from those
plain definitions:

* page table: position pos of sequence b is row table[b, pos // P] * P + pos % P of a shared pool of
  pages of P rows;
* multi-query decode: with L cached tokens, query i of q sits at position L - q + i and attends to
  positions 0 .. L - q + i (a query at a negative position has no keys and a zero output row).
"""

from __future__ import annotations

import numpy as np

from .attention import attend_ref


def gather_pages(pool, table_row, length, page_size):
    """Rows 0 .. length-1 of one sequence from a page pool [n_pages * P, ...] and its page-table row."""
    out = np.empty((length,) + pool.shape[1:], dtype=pool.dtype)
    for pos in range(length):
        out[pos] = pool[int(table_row[pos // page_size]) * page_size + pos % page_size]
    return out


def multi_query_decode_ref(q, c_kv, k_rope, w_uk, w_uv, pair_idx, d_head, theta):
    """Decode of q query tokens of one sequence with L = len(c_kv) cached tokens (the q newest included):
    q [q, n_heads, d_head] raw queries -> [q, n_heads, d_head]."""
    n_q = q.shape[0]
    length = c_kv.shape[0]
    out = np.zeros(q.shape)
    live = [i for i in range(n_q) if length - n_q + i >= 0]
    if live and length > 0:
        q_pos = [length - n_q + i for i in live]
        out[live] = attend_ref(q[live], q_pos, c_kv, k_rope, np.arange(length), w_uk, w_uv, pair_idx, d_head, theta)
    return out
