"""Hierarchical sparse indexer: token scores, 8-token block maxima, block pool,
top-k tokens, and the Reindex rescoring.

Follows [G] "hierarchical sparse indexer" paragraph (the first Full layer builds
the context is first cut down to a pool of 2,048 eight-token blocks, then to 512 tokens per query;
later indexing searches only the pool), [T] "Mechanism 4: the hierarchical
sparse indexer" (coarse-to-fine: narrow the context to a candidate pool of
about 16,384 positions, then attend over a small selection), and [N] "CSA2:
Sharing Main KV, Indexer K, and Top-K Indices Across Layers" (Full selects a
fresh top-512 and builds the pool; Reindex rescores that pool with its own
indexer Q; Reuse takes over the index list of the last layer that computed one).

The pages do not give the scoring rule; the reading taken is
    score(t) = sum_h w_h * max(0, q_h . k_t)
with one indexer key k_t per token shared by all heads. Ranking is by score
descending, then position ascending. With integer inputs every score is an
integer far below 2^53, so float64 (and BLAS) evaluates it exactly.
"""
from __future__ import annotations

import numpy as np

BLOCK = 8


def token_scores(q: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.ndarray:
    """score[t] = sum_h w[h] * max(0, sum_d q[h, d] * k[t, d]) for each row t of k.

    q [H, D], w [H], k [n, D]  ->  [n] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    dots = k @ q.T                                   # [n, H]
    return (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


def block_maxima(s: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """m[b] = max of s over positions block*b .. block*b+block-1 that exist.

    s holds the scores of the visible positions 0..n-1; the last block may be
    partial and then takes the max over its visible positions only.
    """
    n = s.shape[0]
    nblk = -(-n // block)
    return np.array([s[b * block:min(n, (b + 1) * block)].max() for b in range(nblk)],
                    dtype=np.float64)


def select_top(keys: np.ndarray, ids: np.ndarray, count: int) -> np.ndarray:
    """The `count` ids ranked first by (key descending, id ascending), returned ascending."""
    keys = np.asarray(keys, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -keys))                 # last key is the primary key
    return np.sort(ids[order[:count]])


def pool_positions(pool: np.ndarray, n_visible: int, block: int = BLOCK) -> np.ndarray:
    """Visible positions (< n_visible) of the pool's blocks, ascending."""
    pos = (np.asarray(pool, dtype=np.int64)[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return np.sort(pos[pos < n_visible])


def index_full(q, w, k_rows, q_pos: int, P: int, k_keep: int, block: int = BLOCK):
    """Full-mode indexer for one query at position q_pos.

    k_rows: indexer keys of the sequence, at least positions 0..q_pos; only
    positions t <= q_pos are visible (the query's own token included).
    Returns (pool: block ids ascending, idx: positions ascending, scores of
    positions 0..q_pos). The pool holds min(P, #blocks) blocks; idx holds
    min(k_keep, #visible pool positions) positions.
    """
    n_visible = q_pos + 1
    s = token_scores(q, w, np.asarray(k_rows)[:n_visible])
    m = block_maxima(s, block)
    nblk = m.shape[0]
    pool = select_top(m, np.arange(nblk), min(P, nblk))
    cand = pool_positions(pool, n_visible, block)
    idx = select_top(s[cand], cand, min(k_keep, cand.shape[0]))
    return pool, idx, s


def index_reindex(q, w, k_rows_of, pool, q_pos: int, k_keep: int, block: int = BLOCK):
    """Reindex-mode indexer for one query at position q_pos: rescore only the
    inherited pool's visible positions with this layer's own (q, w).

    k_rows_of(positions) -> indexer keys of those positions (so a caller can
    supply just the pool's rows of a long context).
    Returns idx (positions ascending), min(k_keep, #visible pool positions).
    """
    cand = pool_positions(pool, q_pos + 1, block)
    s = token_scores(q, w, k_rows_of(cand))
    return select_top(s, cand, min(k_keep, cand.shape[0]))
