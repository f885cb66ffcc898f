"""Sparse attention over the selected FP4 rows, the sliding-window branch, and
their log-sum-exp merge.

Follows [T] "Mechanism 4: the hierarchical sparse indexer" (attention runs over
the selected candidates, so its cost follows the selection, not the context),
[N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices Across Layers" (every
layer has a main query and window keys/values of its own) and [N] "Causal Encoder-Decoder and
Prefill Halving" plus [G] "SWA Bounded Replay" (a sliding window of the most
recent 128 tokens).

Readings taken where the pages are silent: keys and values of the sparse
branch are the same dequantised row (a shared latent); the window branch has
its own bfloat16 keys and values for positions max(0, p-127)..p; both branches
use the same query and softmax scale; the branches are two softmax partitions
merged by their log-sum-exp, with no de-duplication between them.
"""
from __future__ import annotations

import numpy as np


def branch(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of every head over n rows.

    q [Hq, C], keys [n, C], values [n, C] -> (o [Hq, C], lse [Hq]), natural log.
    An empty branch (n = 0) gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    Hq = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((Hq, values.shape[1])), np.full(Hq, -np.inf)
    logits = scale * (q @ keys.T)                          # [Hq, n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    l = e.sum(axis=1)
    o = (e @ values) / l[:, None]
    return o, mx[:, 0] + np.log(l)


def merge(o_s, lse_s, o_w, lse_w):
    """Combine two softmax partitions given their outputs and log-sum-exps.

    out = (e^{lse_s} o_s + e^{lse_w} o_w) / (e^{lse_s} + e^{lse_w}), evaluated
    relative to max(lse_s, lse_w). Returns (out [Hq, C], lse [Hq]). With both
    partitions empty the result is out = 0, lse = -inf (the empty sum).
    """
    M = np.maximum(lse_s, lse_w)
    if np.isneginf(M).any():
        # no row in either branch (a query that sees no token): output 0, lse -inf
        if not np.isneginf(M).all():
            raise ValueError("heads disagree on whether any row is present")
        return np.zeros_like(o_s), M.copy()
    a = np.exp(lse_s - M)
    b = np.exp(lse_w - M)
    out = (a[:, None] * o_s + b[:, None] * o_w) / (a + b)[:, None]
    return out, M + np.log(a + b)


def attend(q, kv_rows, swa_k, swa_v, scale):
    """One query: sparse branch over dequantised rows kv_rows [k, C] (K = V),
    window branch over (swa_k, swa_v) [n_w, C], merged. Returns (out, lse)."""
    o_s, lse_s = branch(q, kv_rows, kv_rows, scale)
    o_w, lse_w = branch(q, swa_k, swa_v, scale)
    return merge(o_s, lse_s, o_w, lse_w)
