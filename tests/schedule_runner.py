"""Runs a CSA2 layer schedule through the C ABI and times each layer.

[N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices Across Layers":
every layer has a static mode. A Full layer calls fp4kv_index_full; a
Reindex layer calls fp4kv_index_reindex on the pool of the most recent Full
layer with its own indexer query; a Reuse layer makes no indexer call and
attends with the indices of the nearest preceding Full or Reindex layer.
Every layer attends with its own main Q and sliding-window K/V.
"""
from __future__ import annotations

import torch


def run_schedule(fk, cfg, dw):
    """Returns one dict per layer: mode, the pool in force, idx, n_idx, out,
    lse, and the milliseconds of its indexer call and of its attention."""
    prefill = cfg.kind == "prefill"
    layers = []
    pool = n_pool = idx = n_idx = None
    for layer, mode in enumerate(cfg.modes):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        if mode == "full":
            pool, n_pool, idx, n_idx = fk.fp4kv_index_full(dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.q_seq_start,
                                                           dw.q_pos, dw.q_per_seq, cfg.ctx, cfg.P, cfg.k)
        elif mode == "reindex":
            idx, n_idx = fk.fp4kv_index_reindex(dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.q_seq_start, dw.q_pos,
                                                dw.q_per_seq, pool, n_pool, cfg.k)
        elif mode != "reuse":
            raise ValueError(mode)
        ev[1].record()
        if prefill:
            out, lse = fk.fp4kv_sparse_attn_prefill(dw.q[layer], dw.codes, dw.scales, 0, idx, n_idx,
                                                    dw.swa_k[layer], dw.swa_v[layer], cfg.pos0, cfg.W, cfg.scale)
        else:
            out, lse = fk.fp4kv_sparse_attn_decode(dw.q[layer], dw.codes, dw.scales, dw.seq_start, idx, n_idx,
                                                   dw.swa_k[layer], dw.swa_v[layer], dw.q_pos, cfg.scale)
        ev[2].record()
        layers.append({"mode": mode, "pool": pool, "n_pool": n_pool, "idx": idx, "n_idx": n_idx, "out": out,
                       "lse": lse, "ev": ev})
    torch.cuda.synchronize()
    for rec in layers:
        ev = rec.pop("ev")
        rec["index_ms"] = ev[0].elapsed_time(ev[1])
        rec["attn_ms"] = ev[1].elapsed_time(ev[2])
    return layers


def timing_table(cfg, layers):
    lines = [f"{cfg.name}: layer mode index_ms attn_ms"]
    for i, rec in enumerate(layers):
        lines.append(f"  {i:2d} {rec['mode']:8s} {rec['index_ms']:8.3f} {rec['attn_ms']:8.3f}")
    tot_i = sum(r["index_ms"] for r in layers)
    tot_a = sum(r["attn_ms"] for r in layers)
    lines.append(f"  total indexer {tot_i:.3f} ms, attention {tot_a:.3f} ms, layers {tot_i + tot_a:.3f} ms")
    return "\n".join(lines)
