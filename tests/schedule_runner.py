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
    lse, and the milliseconds of its indexer call and of its attention. Every
    output and workspace is allocated before the first layer, so the times
    are those of the launches alone."""
    prefill = cfg.kind == "prefill"
    dev = dw.idx_k.device
    n_q = dw.nq
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8

    def buf(nbytes):
        return torch.empty(max(1, nbytes), dtype=u8, device=dev)

    ws_index = buf(fk.fp4kv_index_workspace_bytes(n_q, cfg.ctx))
    ws_reindex = buf(fk.fp4kv_reindex_workspace_bytes(n_q, cfg.P))
    ws_attn = buf(fk.fp4kv_attn_workspace_bytes(n_q, cfg.Hq, cfg.C, cfg.k, cfg.W))
    sel = {}
    for layer, mode in enumerate(cfg.modes):
        if mode in ("full", "reindex"):
            sel[layer] = (torch.empty((n_q, cfg.P), dtype=i32, device=dev), torch.empty((n_q,), dtype=i32, device=dev),
                          torch.empty((n_q, cfg.k), dtype=i32, device=dev), torch.empty((n_q,), dtype=i32, device=dev))
    outs = [(torch.empty((n_q, cfg.Hq, cfg.C), dtype=f32, device=dev), torch.empty((n_q, cfg.Hq), dtype=f32, device=dev))
            for _ in cfg.modes]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in cfg.modes]
    torch.cuda.synchronize()

    layers = []
    pool = n_pool = idx = n_idx = None
    for layer, mode in enumerate(cfg.modes):
        ev = evs[layer]
        ev[0].record()
        if mode == "full":
            pool, n_pool, idx, n_idx = fk.fp4kv_index_full(
                dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.q_seq_start, dw.q_pos, dw.q_per_seq, cfg.ctx, cfg.P,
                cfg.k, pool_out=sel[layer][0], n_pool=sel[layer][1], idx_out=sel[layer][2], n_idx=sel[layer][3],
                workspace=ws_index)
        elif mode == "reindex":
            idx, n_idx = fk.fp4kv_index_reindex(dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.q_seq_start, dw.q_pos,
                                                dw.q_per_seq, pool, n_pool, cfg.k, idx_out=sel[layer][2],
                                                n_idx=sel[layer][3], workspace=ws_reindex)
        elif mode != "reuse":
            raise ValueError(mode)
        ev[1].record()
        out, lse = outs[layer]
        if prefill:
            fk.fp4kv_sparse_attn_prefill(dw.q[layer], dw.codes, dw.scales, 0, idx, n_idx, dw.swa_k[layer],
                                         dw.swa_v[layer], cfg.pos0, cfg.W, cfg.scale, out=out, lse=lse,
                                         workspace=ws_attn)
        else:
            fk.fp4kv_sparse_attn_decode(dw.q[layer], dw.codes, dw.scales, dw.seq_start, idx, n_idx,
                                        dw.swa_k[layer], dw.swa_v[layer], dw.q_pos, cfg.scale, out=out, lse=lse,
                                        workspace=ws_attn)
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
