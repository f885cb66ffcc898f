#!/usr/bin/env python3
"""Benchmark of the Full-layer decode step at 128K context on one MI355X.

Workload (decode128k): 32 queries, each with its own 131,072-token context;
indexer 16 heads x 128 dims (integers in [-8, 8] as bf16, weights in [1, 8]);
pool of the best 2,048 eight-token blocks, top 512 tokens; attention with 64
heads over the 512-channel FP4 main-KV latent plus a 128-token bf16 window.
Inputs are synthetic, seeded, generated on the GPU, resident in HBM before
timing starts.

One step = the whole hot path of the layer for the batch:
  fp4kv_index_scores_append (indexer scan + 8-token block max; the newest
                             token's FP4 KV row of each sequence is quantised
                             and appended by extra workgroups of the same launch)
  fp4kv_index_select        (top-2,048 blocks -> pool -> top-512 tokens)
  fp4kv_sparse_attn_decode  (FP4 gather-dequant attention + window + LSE merge)

--workload tiny|chain1m|prefill|mixed times one of the other workloads instead
(its own step, its indexer scan as the roofline kernel, the oracle on a few
sampled queries as the CPU baseline).

--kv-format mxfp4|fp8 runs the same step over a main-KV cache in one of the
formats the pages compare FP4 with (E2M1 + E8M0 per 32 channels; E4M3 per
channel), appended and attended through the format-generic entry points.

Prints one JSON line: the metric (queries/s), the step time, the roofline of
the layer (its compulsory HBM bytes over the measured step time, against
8 TB/s, with the HBM traffic the byte counters measured) and, inside it, that
of its dominant kernel (the indexer scan), and the float64 oracle's rate on the
host cores as a CPU baseline. The record's detail carries a SHA-256 of the
generated inputs (every tensor the step reads, taken before the first step),
so that runs on different boxes can be checked to have used the same bytes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/s + HBM GB/s (% of peak), Full-layer sparse attn @128K ctx"
HBM_PEAK_GBPS = 8000.0

# HBM bytes of one decode128k step (and of its scan launch) from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes over this command, each scaled by the
# counter's reading for a plain 1 GiB copy (x1.99994 and x1.0). Valid only for
# the kernel sources they were taken on: a change to any of them turns the
# figures into null until the counters are taken again.
KERNEL_SOURCES = ("api.hip", "attn.hip", "attn_common.h", "common.h", "kernels.h", "quant.hip", "quant_dev.h",
                  "scan.hip", "scan_mfma.hip", "select.hip")
# HBM bytes from rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated against a copy of known size:
# one decode128k step (scan carrying the append, selection, attention, combine) and one scan
# launch as the breakdown pass times it. Valid only for the kernel sources they were taken on.
STEP_TRAFFIC = {"sources_sha256_16": "d329774a791f307c", "bytes_per_step": 1191144682,
                "scan_bytes_per_launch": 1095364563}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KV_FORMATS = {"fp4": 0, "mxfp4": 1, "fp8": 2}
KV_ROW_BYTES = {"fp4": 512 // 2 + 512 // 16, "mxfp4": 512 // 2 + 512 // 32, "fp8": 512}   # at C = 512


def algorithmic_bytes(cfg, kv_format="fp4"):
    """Compulsory HBM bytes per call, counting inputs once and outputs once.
    'scan_intermediate' is what the scan writes for the selection to read
    (token scores and block maxima): not part of the layer's compulsory bytes."""
    B, N = cfg.n_seq, cfg.ctx
    nblk = (N + 7) // 8
    scan = (B * N * cfg.D * 2            # indexer keys
            + B * cfg.H * cfg.D * 2      # indexer queries
            + B * cfg.H * 4)             # head weights
    scan_intermediate = B * N * 4 + B * nblk * 4   # token scores + block maxima written
    select = (B * nblk * 4                       # block maxima read
              + B * cfg.P * 8 * 4                # pool token scores read
              + B * (cfg.P + cfg.k + 2) * 4)     # pool, indices, counts written
    row = KV_ROW_BYTES[kv_format]                # 288 B per FP4 row
    attn = B * (cfg.k * row                      # gathered main-KV rows
                + cfg.k * 4                      # indices
                + cfg.Hq * cfg.C * 2             # main Q
                + 2 * cfg.W * cfg.C * 2          # window K and V
                + cfg.Hq * cfg.C * 4 + cfg.Hq * 4)   # output and lse
    append = B * (cfg.C * 2 + row + 8)           # bf16 row in, FP4 row + destination out
    # The layer as the path defines it, per query: indexer keys, indexer query and
    # weights, pool and index lists written, the gathered rows with their
    # indices, main Q, window K and V, and the output (the lse, the counts and
    # the append's bytes are left out).
    layer = B * (N * cfg.D * 2 + cfg.H * cfg.D * 2 + cfg.H * 4 + (cfg.P + cfg.k) * 4
                 + cfg.k * row + cfg.k * 4 + cfg.Hq * cfg.C * 2 + 2 * cfg.W * cfg.C * 2 + cfg.Hq * cfg.C * 4)
    return {"scan": scan, "scan_intermediate": scan_intermediate, "select": select, "attn": attn, "append": append,
            "layer": layer}


def sources_hash():
    """SHA-256 (first 16 hex digits) of the kernel sources, in KERNEL_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_indexer_fp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def inputs_sha256(named):
    """SHA-256 (first 16 hex digits) of generated inputs: each tensor's name,
    dtype and shape, then its bytes, in the given order. Tensors are copied to
    the host in 64 MiB pieces; this runs before the untimed warm-up."""
    import hashlib
    import torch
    h = hashlib.sha256()
    piece = 64 << 20
    for name, t in named:
        if t is None:
            continue
        t = t.contiguous()
        h.update(f"{name}:{t.dtype}:{tuple(t.shape)};".encode())
        flat = t.reshape(-1).view(torch.uint8)
        for i in range(0, flat.numel(), piece):
            h.update(memoryview(flat[i:i + piece].cpu().numpy()))
    return h.hexdigest()[:16]


def step_traffic():
    """Counter-measured HBM bytes (per step, per scan launch) if the kernel
    sources are those they were taken on, else (None, None)."""
    if STEP_TRAFFIC["sources_sha256_16"] != sources_hash():
        return None, None
    return STEP_TRAFFIC["bytes_per_step"], STEP_TRAFFIC["scan_bytes_per_launch"]


def cpu_baseline(cfg, n_sample, min_seconds=10.0, kv_format="fp4"):
    """The oracle, as it stands, on n_sample queries of the same workload:
    Full-layer indexer + attention per query, passes over the sample repeated until
    min_seconds of CPU work. Input generation is not timed."""
    import numpy as np
    import torch
    from synth import bf16_to_f64
    from synth import workloads as wl
    from tests import oracle_runner as orun
    from oracle import attention, indexer, kvformats

    torch.set_num_threads(os.cpu_count() or 1)
    prepared = []
    for i in range(n_sample):
        s = wl.sequence_of(cfg, i)
        p = int(cfg.q_pos()[i])
        krows = orun.host_idx_k(cfg, s, p + 1)
        q, w = wl.indexer_query(cfg, 0, i)
        Q = bf16_to_f64(wl.main_query(cfg, 0, i))
        wpos = torch.arange(max(0, p - cfg.W + 1), p + 1, dtype=torch.int64)
        wk = bf16_to_f64(wl.window_rows(cfg, 0, s, wpos, "k"))
        wv = bf16_to_f64(wl.window_rows(cfg, 0, s, wpos, "v"))
        prepared.append((s, p, krows, bf16_to_f64(q), w.numpy().astype(np.float64), Q, wk, wv))
    # bf16 rows of every position a query may select are regenerated inside the
    # timed region only as the oracle's codec input; their generation is timed
    # separately and subtracted.
    t_gen = 0.0
    done = 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 - t_gen < min_seconds:
        for (s, p, krows, q, w, Q, wk, wv) in prepared:
            pool, idx, _ = indexer.index_full(q, w, krows, p, cfg.P, cfg.k)
            tg = time.perf_counter()
            x = bf16_to_f64(wl.kv_rows(cfg, s, torch.from_numpy(idx)))
            t_gen += time.perf_counter() - tg
            fmt = KV_FORMATS[kv_format]
            rows = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, x))
            attention.attend(Q, rows, wk, wv, cfg.scale)
            done += 1
    dt = time.perf_counter() - t0 - t_gen
    threads = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [threads])
    except Exception:
        pass
    return {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} query evaluations ({done // n_sample} passes over {n_sample} of the 32 queries of "
                      f"decode128k; Full-layer indexer + attention per query, float64 numpy; {dt:.1f} s; "
                      f"input generation excluded)"}


WORKLOAD_TEXT = {
    "tiny": "tiny: one Full-layer decode query over 4,096 tokens, indexer 4x64, pool 64 blocks, top-128, "
            "16 heads x 512-channel FP4 latent, 128-token bf16 window",
    "chain1m": "chain1m: 8 queries x 1,048,576-token contexts through Full, Reuse x3, Reindex, Reuse x3 "
               "(one indexer scan, one rescoring of the pool, 8 attention layers), indexer 16x128, pool 2,048 "
               "blocks, top-512, 64 heads x 512-channel FP4 latent, 128-token bf16 windows",
    "prefill": "prefill: 4,096 causal queries at positions 127,000..131,095 of one 131,096-token context, "
               "matrix-core indexer 16x128, pool 2,048 blocks, top-512, 64 heads x 512-channel FP4 latent, each "
               "query's preceding 128 tokens as the bf16 window",
    "mixed": "mixed: FP4 quantize-append of 65,536 rows, then a Full-layer decode of 64 queries with contexts "
             "log-uniform in 4,096..1,048,576 tokens, indexer 16x128, pool min(2,048, blocks), top-512, 64 heads "
             "x 512-channel FP4 latent, 128-token bf16 window",
}


def cpu_baseline_workload(cfg, sample, min_seconds=10.0):
    """The oracle, as it stands, on the sampled queries of one of the other
    workloads: every layer of the query's schedule (Full indexer, Reindex, the
    codec of the selected rows and attention), passes repeated until
    min_seconds of CPU work. Input generation is not timed."""
    import numpy as np
    import torch
    from synth import bf16_to_f64
    from synth import workloads as wl
    from tests import oracle_runner as orun
    from oracle import attention, fp4, indexer

    torch.set_num_threads(os.cpu_count() or 1)
    modes = cfg.modes or ("full",)
    shared_k = {}
    prepared = []
    for i in sample:
        s = wl.sequence_of(cfg, i)
        p = int(cfg.q_pos()[i])
        if cfg.kind == "prefill":                     # one sequence: generate its keys once
            if s not in shared_k:
                shared_k[s] = orun.host_idx_k(cfg, s, int(cfg.seq_lengths()[s]))
            krows = shared_k[s]
        else:
            krows = orun.host_idx_k(cfg, s, p + 1)
        wpos = torch.arange(max(0, p - cfg.W + 1), p + 1, dtype=torch.int64)
        layers = []
        for layer, mode in enumerate(modes):
            iq = None
            if mode in ("full", "reindex"):
                q, w = wl.indexer_query(cfg, layer, i)
                iq = (bf16_to_f64(q), w.numpy().astype(np.float64))
            layers.append((mode, iq, bf16_to_f64(wl.main_query(cfg, layer, i)),
                           bf16_to_f64(wl.window_rows(cfg, layer, s, wpos, "k")),
                           bf16_to_f64(wl.window_rows(cfg, layer, s, wpos, "v"))))
        prepared.append((s, p, krows, layers))
    t_gen = 0.0
    done = 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 - t_gen < min_seconds:
        for (s, p, krows, layers) in prepared:
            pool = idx = None
            for mode, iq, Q, wk, wv in layers:
                if mode == "full":
                    pool, idx, _ = indexer.index_full(iq[0], iq[1], krows, p, cfg.P, cfg.k)
                elif mode == "reindex":
                    idx = indexer.index_reindex(iq[0], iq[1], lambda pos: krows[pos], pool, p, cfg.k)
                tg = time.perf_counter()
                x = bf16_to_f64(wl.kv_rows(cfg, s, torch.from_numpy(np.asarray(idx, dtype=np.int64))))
                t_gen += time.perf_counter() - tg
                rows = fp4.dequantize_rows(*fp4.quantize_rows(x)) if len(idx) else np.zeros((0, cfg.C))
                attention.attend(Q, rows, wk, wv, cfg.scale)
            done += 1
    dt = time.perf_counter() - t0 - t_gen
    threads = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [threads])
    except Exception:
        pass
    return {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} query evaluations ({done // len(sample)} passes over queries {list(sample)} of "
                      f"{cfg.name}, each through its {len(modes)}-layer schedule; float64 numpy; {dt:.1f} s; "
                      f"input generation excluded)"}


# queries of each of the other workloads that the CPU baseline samples
CPU_SAMPLE = {"tiny": [0], "prefill": [0, 2048, 4095], "chain1m": [0], "mixed": [0, 1, 2, 3]}


def scan_units(cfg):
    """Algorithmic units of one indexer-scan launch over the workload's queries:
    FLOPs for a prefill chunk (4,096 per visible (query, token) pair at 16 heads
    x 128), otherwise compulsory HBM bytes (per visible token its 2*D-byte key;
    per query its H x D bf16 query and H weights). The token scores and block
    maxima the scan writes for the selection are intermediates, reported
    separately (scan_intermediate_bytes)."""
    import numpy as np
    L = cfg.seq_lengths()
    B = cfg.n_queries()
    seq_of = np.zeros(B, dtype=np.int64) if cfg.kind == "prefill" else np.arange(B)
    vis = np.minimum(cfg.q_pos().astype(np.int64) + 1, L[seq_of]).clip(min=0)   # visible tokens per query
    if cfg.kind == "prefill":
        return float(vis.sum()) * cfg.H * cfg.D * 2
    return float((vis * cfg.D * 2).sum() + B * (cfg.H * cfg.D * 2 + cfg.H * 4))


def scan_intermediate_bytes(cfg):
    """Token scores (4 B) and block maxima (4 B per 8-token block) the scan writes."""
    import numpy as np
    L = cfg.seq_lengths()
    B = cfg.n_queries()
    seq_of = np.zeros(B, dtype=np.int64) if cfg.kind == "prefill" else np.arange(B)
    vis = np.minimum(cfg.q_pos().astype(np.int64) + 1, L[seq_of]).clip(min=0)
    return float((vis * 4 + (vis + 7) // 8 * 4).sum())


def run_workload(args, name):
    """One of the other workloads, timed over the launches that make up its step:
    tiny (scores, selection, attention), chain1m (scores, selection, one Reindex,
    8 attention layers), prefill (matrix-core scores, selection, prefill
    attention), mixed (append of 65,536 rows, scores, selection, attention).
    Prints one JSON line like the default run; the roofline is that of the
    indexer scan (HBM bytes, or matrix-core FLOPs for the prefill chunk)."""
    import torch
    import sparse_indexer_fp4_amd as fk
    from synth import workloads as wl
    from tests.gpu_inputs import DeviceWorkload

    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS[name]
    t0 = time.perf_counter()
    log(f"generating {name} inputs on the GPU")
    dw = DeviceWorkload(cfg, dev)
    B = cfg.n_queries()
    L = cfg.seq_lengths()
    max_ctx = int(L.max()) if cfg.kind == "mixed" else cfg.ctx
    nblk = (max_ctx + 7) // 8
    f32, i32 = torch.float32, torch.int32
    scores = torch.empty((B, max_ctx), dtype=f32, device=dev)
    blockmax = torch.empty((B, nblk), dtype=f32, device=dev)
    pool = torch.empty((B, cfg.P), dtype=i32, device=dev)
    n_pool = torch.empty((B,), dtype=i32, device=dev)
    idx = [torch.empty((B, cfg.k), dtype=i32, device=dev) for _ in range(2)]
    n_idx = [torch.empty((B,), dtype=i32, device=dev) for _ in range(2)]
    modes = cfg.modes or ("full",)
    outs = [(torch.empty((B, cfg.Hq, cfg.C), dtype=f32, device=dev), torch.empty((B, cfg.Hq), dtype=f32, device=dev))
            for _ in modes]
    aws = torch.empty(max(1, fk.fp4kv_attn_workspace_bytes(B, cfg.Hq, cfg.C, cfg.k, cfg.W)), dtype=torch.uint8,
                      device=dev)
    rws = torch.empty(max(1, fk.fp4kv_reindex_workspace_bytes(B, cfg.P)), dtype=torch.uint8, device=dev)
    new_x, new_dst = dw.appended_rows() if cfg.kind == "mixed" else (None, None)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    named = [("idx_k", dw.idx_k), ("codes", dw.codes), ("scales", dw.scales), ("seq_start", dw.seq_start),
             ("q_pos", dw.q_pos), ("new_x", new_x), ("new_dst", new_dst)]
    for layer in range(len(modes)):
        named += [(f"q{layer}", dw.q[layer]), (f"swa_k{layer}", dw.swa_k[layer]), (f"swa_v{layer}", dw.swa_v[layer]),
                  (f"idx_q{layer}", dw.idx_q.get(layer)), (f"w{layer}", dw.w.get(layer))]
    in_hash = inputs_sha256(named)
    log(f"inputs hashed: {in_hash}")
    stream = torch.cuda.current_stream()

    def step(scan_ev):
        scan_ev[0].record(stream)
        if new_x is not None:      # the append rides in the scan's launch
            fk.fp4kv_index_scores_append(dw.idx_q[0], dw.w[0], dw.idx_k, dw.q_seq_start, dw.q_pos, dw.q_per_seq,
                                         max_ctx, new_x, dw.codes, dw.scales, dst_rows=new_dst, scores=scores,
                                         blockmax=blockmax, stream=stream)
        else:
            fk.fp4kv_index_scores(dw.idx_q[0], dw.w[0], dw.idx_k, dw.q_seq_start, dw.q_pos, dw.q_per_seq, max_ctx,
                                  scores=scores, blockmax=blockmax, stream=stream)
        scan_ev[1].record(stream)
        fk.fp4kv_index_select(scores, blockmax, dw.total_rows, dw.q_seq_start, dw.q_pos, dw.q_per_seq, cfg.P, cfg.k,
                              pool_out=pool, n_pool=n_pool, idx_out=idx[0], n_idx=n_idx[0], stream=stream)
        cur = 0
        for layer, mode in enumerate(modes):
            if mode == "reindex":
                fk.fp4kv_index_reindex(dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.seq_start, dw.q_pos, 1, pool,
                                       n_pool, cfg.k, idx_out=idx[1], n_idx=n_idx[1], workspace=rws, stream=stream)
                cur = 1
            out, lse = outs[layer]
            if cfg.kind == "prefill":
                fk.fp4kv_sparse_attn_prefill(dw.q[layer], dw.codes, dw.scales, 0, idx[cur], n_idx[cur],
                                             dw.swa_k[layer], dw.swa_v[layer], cfg.pos0, cfg.W, cfg.scale, out=out,
                                             lse=lse, workspace=aws, stream=stream)
            else:
                fk.fp4kv_sparse_attn_decode(dw.q[layer], dw.codes, dw.scales, dw.seq_start, idx[cur], n_idx[cur],
                                            dw.swa_k[layer], dw.swa_v[layer], dw.q_pos, cfg.scale, out=out, lse=lse,
                                            workspace=aws, stream=stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    warm = events()
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    evs = [events() for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    scan_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps

    units = scan_units(cfg)
    if cfg.kind == "prefill":
        flops = units
        achieved = flops / (scan_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "matrix-core indexer scan (fp4kv_index_scores, 32 queries per tile)",
                "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s", "frac": achieved / 2500.0,
                "traffic": None, "flops_per_launch": flops}
    else:
        nbytes = units
        achieved = nbytes / (scan_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "indexer scan (fp4kv_index_scores" +
                ("_append, carrying the 65,536-row append)" if new_x is not None else ")"),
                "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                "traffic": None, "bytes_per_launch": nbytes,
                "intermediate_bytes_written": scan_intermediate_bytes(cfg)}
    rec = {
        "metric": f"queries/s, {name}",
        "value": B / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[name], "queries": B, "max_ctx": max_ctx, "layers": len(modes),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "detail": {"scan_ms_timed_region": scan_ms, "inputs_sha256_16": in_hash,
                   "kernel_sources_sha256_16": sources_hash()},
        "cpu_baseline": None,
    }
    if args.cpu_sample > 0:
        log(f"timing the oracle on queries {CPU_SAMPLE[name]}")
        rec["cpu_baseline"] = cpu_baseline_workload(cfg, CPU_SAMPLE[name])
    log(f"done in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample", type=int, default=32, help="queries timed on the oracle (0: skip)")
    ap.add_argument("--kv-format", choices=sorted(KV_FORMATS), default="fp4",
                    help="main-KV cache format (default fp4: E2M1 + E4M3 per 16 channels)")
    ap.add_argument("--workload", choices=["decode128k"] + sorted(WORKLOAD_TEXT), default="decode128k",
                    help="decode128k (default) is the benchmark line; the others time their own step, with the "
                         "indexer scan as the roofline kernel and the oracle on a few sampled queries "
                         "(--cpu-sample 0 skips it)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes, --steps times (calibrates "
                         "the HBM byte counters against a kernel of known traffic), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the decode batch shards by query "
              f"with no exchange: each GPU runs this same workload on its own queries)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_indexer_fp4_amd as fk
    from synth import workloads as wl
    from tests.gpu_inputs import DeviceWorkload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload != "decode128k":
        run_workload(args, args.workload)
        return
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {src.numel() * 4} bytes {args.steps} times")
        return
    cfg = wl.CONFIGS["decode128k"]
    t0 = time.perf_counter()
    log(f"generating {cfg.name} inputs on the GPU")
    fmt = KV_FORMATS[args.kv_format]
    dw = DeviceWorkload(cfg, dev, build_kv=(fmt == 0))
    codes, scales = dw.codes, dw.scales
    if fmt != 0:
        codes = torch.zeros((dw.total_rows, fk.fp4kv_kv_code_bytes(fmt, cfg.C)), dtype=torch.uint8, device=dev)
        sb = fk.fp4kv_kv_scale_bytes(fmt, cfg.C)
        scales = torch.zeros((dw.total_rows, sb), dtype=torch.uint8, device=dev) if sb > 0 else None
        starts = cfg.seq_starts()
        for sq in range(cfg.n_seq):
            for a, b in wl.chunks(int(dw.lengths[sq]), 1 << 18):
                fk.fp4kv_kv_append(fmt, wl.kv_rows_into(cfg, sq, a, b, dev), codes, scales,
                                   dst_start=int(starts[sq]) + a)
    new_x, new_dst = dw.newest_rows()
    B, N = cfg.n_seq, cfg.ctx
    nblk = (N + 7) // 8
    scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    blockmax = torch.empty((B, nblk), dtype=torch.float32, device=dev)
    pool = torch.empty((B, cfg.P), dtype=torch.int32, device=dev)
    n_pool = torch.empty((B,), dtype=torch.int32, device=dev)
    idx = torch.empty((B, cfg.k), dtype=torch.int32, device=dev)
    n_idx = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, cfg.Hq, cfg.C), dtype=torch.float32, device=dev)
    lse = torch.empty((B, cfg.Hq), dtype=torch.float32, device=dev)
    aws = torch.empty(max(1, fk.fp4kv_attn_workspace_bytes(B, cfg.Hq, cfg.C, cfg.k, cfg.W)), dtype=torch.uint8,
                      device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    in_hash = inputs_sha256([("idx_k", dw.idx_k), ("codes", codes), ("scales", scales), ("seq_start", dw.seq_start),
                             ("q_pos", dw.q_pos), ("idx_q", dw.idx_q[0]), ("w", dw.w[0]), ("q", dw.q[0]),
                             ("swa_k", dw.swa_k[0]), ("swa_v", dw.swa_v[0]), ("new_x", new_x),
                             ("new_dst", new_dst)])
    log(f"inputs hashed: {in_hash}")

    stream = torch.cuda.current_stream()

    def attend():
        if fmt == 0:
            fk.fp4kv_sparse_attn_decode(dw.q[0], codes, scales, dw.seq_start, idx, n_idx, dw.swa_k[0], dw.swa_v[0],
                                        dw.q_pos, cfg.scale, out=out, lse=lse, workspace=aws, stream=stream)
        else:
            fk.fp4kv_sparse_attn_decode_kv(fmt, dw.q[0], codes, scales, dw.seq_start, idx, n_idx, dw.swa_k[0],
                                           dw.swa_v[0], dw.q_pos, cfg.scale, out=out, lse=lse, workspace=aws,
                                           stream=stream)

    def select():
        fk.fp4kv_index_select(scores, blockmax, dw.total_rows, dw.seq_start, dw.q_pos, 1, cfg.P, cfg.k,
                              pool_out=pool, n_pool=n_pool, idx_out=idx, n_idx=n_idx, stream=stream)

    def step():
        """One decode step: the scan carrying the append, the selection, attention."""
        fk.fp4kv_index_scores_append(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1, N, new_x, codes,
                                     scales, dst_rows=new_dst, kv_fmt=fmt, scores=scores, blockmax=blockmax,
                                     stream=stream)
        select()
        attend()

    def breakdown(ev):
        """The same step as separate launches (append on its own), an event
        around each: append, scan, selection, attention (+ combine)."""
        ev[0].record(stream)
        fk.fp4kv_kv_append(fmt, new_x, codes, scales, dst_rows=new_dst, stream=stream)
        ev[1].record(stream)
        fk.fp4kv_index_scores(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1, N, scores=scores,
                              blockmax=blockmax, stream=stream)
        ev[2].record(stream)
        select()
        ev[3].record(stream)
        attend()
        ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: K steps back to back, bracketed by one event pair on the
    # launch stream (and host synchronisation on both sides).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = 1e3 * elapsed / args.steps
    ms_step_events = e0.elapsed_time(e1) / args.steps

    # Untimed breakdown pass: every launch bracketed by events.
    n_bd = min(args.steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_bd)]
    for i in range(n_bd):
        breakdown(evs[i])
    torch.cuda.synchronize()
    per = {"append": 0.0, "scan": 0.0, "select": 0.0, "attn": 0.0}
    for ev in evs:
        per["append"] += ev[0].elapsed_time(ev[1])
        per["scan"] += ev[1].elapsed_time(ev[2])
        per["select"] += ev[2].elapsed_time(ev[3])
        per["attn"] += ev[3].elapsed_time(ev[4])
    per = {k: v / n_bd for k, v in per.items()}          # ms per launch, breakdown pass
    nbytes = algorithmic_bytes(cfg, args.kv_format)
    layer_gbps = nbytes["layer"] / (ms_step_events * 1e-3) / 1e9
    scan_gbps = nbytes["scan"] / (per["scan"] * 1e-3) / 1e9
    step_bytes, scan_bytes = step_traffic()

    rec = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode128k: Full-layer decode step, 32 queries x 131,072-token contexts, "
                               "indexer 16x128, pool 2,048 blocks of 8, top-512, 64 heads x 512-channel "
                               + {"fp4": "FP4 (E2M1 + E4M3 per 16)", "mxfp4": "MXFP4 (E2M1 + E8M0 per 32)",
                                  "fp8": "FP8 (E4M3 per channel)"}[args.kv_format]
                               + " latent, 128-token bf16 window",
                   "batch": B, "ctx": N, "pool_blocks": cfg.P, "top_k": cfg.k, "heads": cfg.Hq,
                   "kv_format": args.kv_format, "kv_bytes_per_row": KV_ROW_BYTES[args.kv_format],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": "whole Full-layer decode step (indexer scan carrying the append, selection, "
                               "attention + combine), per step",
                     "achieved": layer_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": layer_gbps / HBM_PEAK_GBPS, "traffic": step_bytes,
                     "bytes_per_launch": nbytes["layer"], "ms_per_launch": ms_step_events,
                     "dominant_kernel": {
                         "kernel": "indexer scan (fp4kv_index_scores)", "bound": "hbm",
                         "achieved": scan_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": scan_gbps / HBM_PEAK_GBPS, "traffic": scan_bytes,
                         "bytes_per_launch": nbytes["scan"], "ms_per_launch": per["scan"],
                         "intermediate_bytes_written": nbytes["scan_intermediate"],
                         "timing": "HIP events around the scan in an untimed pass of the same step as "
                                   "separate launches"}},
        "detail": {"ms_per_launch": per, "ms_per_step_events": ms_step_events, "algorithmic_bytes": nbytes,
                   "inputs_sha256_16": in_hash, "kernel_sources_sha256_16": sources_hash()},
    }
    if args.cpu_sample > 0:
        log(f"timing the oracle on {args.cpu_sample} queries")
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample, kv_format=args.kv_format)
    else:
        rec["cpu_baseline"] = None
    log(f"done in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
