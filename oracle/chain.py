"""CSA2 mode schedule for one query: which indices each layer attends with.

Follows [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices Across
Layers" and [G] "CSA2 modes" paragraph: every layer has a static mode. Full
computes the pool and a fresh top-k; Reindex reuses the preceding Full layer's
main KV and indexer K and rescores that layer's pool with its own indexer Q;
Reuse runs no indexer and takes the indices of the nearest preceding Full or
Reindex layer.
"""
from __future__ import annotations

from . import indexer

FULL, REINDEX, REUSE = "full", "reindex", "reuse"


def layer_indices(modes, full_fn, reindex_fn):
    """Indices used by each layer of a schedule.

    full_fn(layer) -> (pool, idx) runs a Full layer; reindex_fn(layer, pool) ->
    idx runs a Reindex layer on the pool of the most recent Full layer.
    Returns a list of (pool, idx) per layer (pool is the one in force).
    """
    out = []
    pool = idx = None
    for layer, mode in enumerate(modes):
        if mode == FULL:
            pool, idx = full_fn(layer)
        elif mode == REINDEX:
            if pool is None:
                raise ValueError("Reindex layer before any Full layer")
            idx = reindex_fn(layer, pool)
        elif mode == REUSE:
            if idx is None:
                raise ValueError("Reuse layer before any Full or Reindex layer")
        else:
            raise ValueError(mode)
        out.append((pool, idx))
    return out


__all__ = ["FULL", "REINDEX", "REUSE", "layer_indices", "indexer"]
