"""Device-resident inputs of a workload, for the GPU tests and the benchmark.

Generated on the GPU by the seeded streams; the FP4 main-KV cache is produced
from the bf16 rows by fp4kv_quantize_append (the code under test).
"""
from __future__ import annotations

import numpy as np
import torch

import sparse_indexer_fp4_amd as fk
from synth import workloads as wl


class DeviceWorkload:
    def __init__(self, cfg, device="cuda", build_kv=True, layers=None):
        self.cfg = cfg
        self.device = device
        L = cfg.seq_lengths()
        self.lengths = L
        self.total_rows = int(L.sum())
        self.seq_start = torch.from_numpy(cfg.seq_starts()).to(device)
        self.q_pos = torch.from_numpy(cfg.q_pos()).to(device)
        nq = cfg.n_queries()
        self.nq = nq
        if cfg.kind == "prefill":
            self.q_seq_start = torch.zeros(1, dtype=torch.int64, device=device)
            self.q_per_seq = nq
        else:
            self.q_seq_start = self.seq_start
            self.q_per_seq = 1
        self.idx_k = torch.empty((self.total_rows, cfg.D), dtype=torch.bfloat16, device=device)
        wl.fill_idx_k(cfg, self.idx_k)
        self.codes = torch.zeros((self.total_rows, cfg.C // 2), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((self.total_rows, cfg.C // 16), dtype=torch.uint8, device=device)
        if build_kv:
            self.build_kv()
        nl = cfg.layers() if layers is None else layers
        self.idx_q, self.w, self.q, self.swa_k, self.swa_v = {}, {}, {}, {}, {}
        for layer in range(nl):
            self.q[layer] = wl.main_queries_fast(cfg, layer, device)
            if cfg.kind == "prefill":
                self.swa_k[layer], self.swa_v[layer] = wl.prefill_window(cfg, layer, device)
            else:
                self.swa_k[layer], self.swa_v[layer] = wl.decode_windows(cfg, layer, device)
        for layer in range(nl):
            if layer == 0 or (cfg.modes and cfg.modes[layer] in ("full", "reindex")):
                self.idx_q[layer], self.w[layer] = wl.indexer_queries_fast(cfg, layer, device)

    def build_kv(self, chunk_rows=1 << 18):
        """Quantise every context row (appended rows of the mixed step excluded)."""
        cfg = self.cfg
        starts = cfg.seq_starts()
        for s in range(cfg.n_seq):
            n = int(self.lengths[s]) - (cfg.append_per_seq if cfg.kind == "mixed" else 0)
            for a, b in wl.chunks(n, chunk_rows):
                x = wl.kv_rows_into(cfg, s, a, b, self.device)
                fk.fp4kv_quantize_append(x, self.codes, self.scales, dst_start=int(starts[s]) + a)

    def appended_rows(self):
        """(bf16 rows, destination rows) of the mixed step's appended rows."""
        cfg = self.cfg
        starts = cfg.seq_starts()
        xs, dst = [], []
        for s in range(cfg.n_seq):
            L = int(self.lengths[s])
            a = L - cfg.append_per_seq
            xs.append(wl.kv_rows_into(cfg, s, a, L, self.device))
            dst.append(torch.arange(starts[s] + a, starts[s] + L, dtype=torch.int64, device=self.device))
        return torch.cat(xs).contiguous(), torch.cat(dst).contiguous()

    def newest_rows(self):
        """(bf16 rows, destination rows): the row at each decode query's own position."""
        cfg = self.cfg
        starts = cfg.seq_starts()
        xs, dst = [], []
        for s in range(cfg.n_seq):
            p = int(self.lengths[s]) - 1
            xs.append(wl.kv_rows_into(cfg, s, p, p + 1, self.device))
            dst.append(int(starts[s]) + p)
        return torch.cat(xs).contiguous(), torch.tensor(dst, dtype=torch.int64, device=self.device)
