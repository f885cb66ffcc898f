"""Expected results of the oracle for single queries of a workload.

Inputs are regenerated on the host from the seeded streams (only the rows a
query needs), quantised and scored by the oracle, never taken from the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention, fp4, indexer, kvformats
from synth import bf16_to_f64
from synth import workloads as wl


def host_idx_k(cfg, s, n_rows):
    return bf16_to_f64(wl.idx_k_rows(cfg, s, torch.arange(n_rows, dtype=torch.int64)))


def full_layer(cfg, i, layer=0, k_rows=None):
    """(pool, idx, scores) of query i for a Full layer."""
    s = wl.sequence_of(cfg, i)
    p = int(cfg.q_pos()[i])
    q, w = wl.indexer_query(cfg, layer, i)
    if k_rows is None:
        k_rows = host_idx_k(cfg, s, p + 1)
    return indexer.index_full(bf16_to_f64(q), w.numpy().astype(np.float64), k_rows, p, cfg.P, cfg.k)


def reindex_layer(cfg, i, layer, pool):
    s = wl.sequence_of(cfg, i)
    p = int(cfg.q_pos()[i])
    q, w = wl.indexer_query(cfg, layer, i)
    rows_of = lambda pos: bf16_to_f64(wl.idx_k_rows(cfg, s, torch.from_numpy(np.asarray(pos, dtype=np.int64))))
    return indexer.index_reindex(bf16_to_f64(q), w.numpy().astype(np.float64), rows_of, pool, p, cfg.k)


def dequantized_rows(cfg, s, positions, fmt=kvformats.FMT_FP4):
    """Main-KV rows at `positions` as the cache in format fmt holds them; fmt None
    gives the unquantised bf16 rows."""
    x = bf16_to_f64(wl.kv_rows(cfg, s, torch.from_numpy(np.asarray(positions, dtype=np.int64))))
    if fmt is None:
        return x
    if fmt == kvformats.FMT_FP4:
        return fp4.dequantize_rows(*fp4.quantize_rows(x))
    return kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, x))


def attend(cfg, i, layer, idx, fmt=kvformats.FMT_FP4):
    """(out [Hq, C], lse [Hq]) of query i in `layer`, attending to positions idx
    of a main-KV cache in format fmt (None: unquantised rows)."""
    s = wl.sequence_of(cfg, i)
    p = int(cfg.q_pos()[i])
    Q = bf16_to_f64(wl.main_query(cfg, layer, i))
    rows = dequantized_rows(cfg, s, idx, fmt) if len(idx) else np.zeros((0, cfg.C))
    wpos = torch.arange(max(0, p - cfg.W + 1), p + 1, dtype=torch.int64)
    wk = bf16_to_f64(wl.window_rows(cfg, layer, s, wpos, "k"))
    wv = bf16_to_f64(wl.window_rows(cfg, layer, s, wpos, "v"))
    return attention.attend(Q, rows, wk, wv, cfg.scale)


def within_tolerance(got, ref):
    """max |got - ref| <= 2e-4 * max |ref| + 1e-6 over the tensor's finite
    reference entries; infinite entries (the lse of a query with no row) must
    match exactly. A NaN anywhere fails."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    inf = np.isinf(ref)
    if inf.any() and not np.array_equal(got[inf], ref[inf]):
        return False, float("inf"), 0.0
    fin = ~inf
    if not fin.any():
        return True, 0.0, 0.0
    err = np.abs(got[fin] - ref[fin]).max()
    tol = 2e-4 * np.abs(ref[fin]).max() + 1e-6
    return bool(err <= tol), err, tol
