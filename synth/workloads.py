"""Synthetic workloads: shapes, value distributions and seeds of the five
configurations the hot path is measured and checked on, and generators for
every input tensor (on any device, whole or by rows).

Recipe (every value a function of (seed, stream, counter); see synth/__init__):
  * indexer keys k[s, t, :] of sequence s at position t: integers uniform in
    [qk_lo, qk_hi] stored as bf16, one key per token shared by all heads;
  * indexer queries q[layer, i, h, :]: integers in [qk_lo, qk_hi] as bf16;
    head weights w[layer, i, h]: integers in [w_lo, w_hi] as fp32;
  * main-KV latent rows x[s, t, :] (512 channels, K = V): N(0, 1) with
    independent 1% outliers scaled by 20, rounded to bf16 (quantised to FP4 by
    the code under test or by the oracle, never here);
  * main queries Q[layer, i, h, :]: N(0, 1) bf16, softmax scale 1/sqrt(512);
  * sliding-window keys / values of layer `layer` at position t of sequence s:
    N(0, 1) bf16, separate tensors;
  * the mixed-step configuration also zeroes whole 16-channel groups of the
    appended rows with probability 0.001 (exercising the zero scale).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import (bernoulli_rows, int_bf16_rows, int_tensor_f32, normal_bf16, normal_bf16_rows,
               uniform_f64_host, ENTITY_SHIFT)

C_LATENT = 512
ZERO_GROUP_THRESHOLD = 4294967  # round(0.001 * 2**32)


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    kind: str                  # "decode", "chain", "prefill", "mixed"
    n_seq: int
    H: int
    D: int
    qk: tuple
    wr: tuple
    P: int
    k: int
    Hq: int
    W: int = 128
    C: int = C_LATENT
    ctx: int = 0               # context length (equal-length decode / prefill sequence)
    T: int = 0                 # prefill queries
    pos0: int = 0              # prefill first position
    modes: tuple = ()          # chain: layer modes
    append_per_seq: int = 0    # mixed: rows appended per sequence
    lengths: tuple = field(default=(), compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.C)

    def seq_lengths(self) -> np.ndarray:
        if self.kind == "mixed":
            return mixed_lengths(self.seed, self.n_seq)
        return np.full(self.n_seq, self.ctx, dtype=np.int64)

    def seq_starts(self) -> np.ndarray:
        L = self.seq_lengths()
        return np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int64)

    def n_queries(self) -> int:
        return self.T if self.kind == "prefill" else self.n_seq

    def q_pos(self) -> np.ndarray:
        if self.kind == "prefill":
            return (self.pos0 + np.arange(self.T)).astype(np.int32)
        return (self.seq_lengths() - 1).astype(np.int32)

    def layers(self) -> int:
        return len(self.modes) if self.modes else 1


def mixed_lengths(seed: int, n: int) -> np.ndarray:
    """Context lengths log-uniform in [4096, 2^20], rounded to multiples of 8."""
    u = uniform_f64_host(seed, "lengths", n)
    lo, hi = math.log(4096.0), math.log(2.0 ** 20)
    L = 8 * np.round(np.exp(lo + u * (hi - lo)) / 8.0)
    return np.clip(L, 4096, 2 ** 20).astype(np.int64)


CONFIGS = {
    "tiny": Config("tiny", 0, "decode", n_seq=1, H=4, D=64, qk=(-4, 4), wr=(1, 4), P=64, k=128, Hq=16,
                   ctx=4096),
    "decode128k": Config("decode128k", 1, "decode", n_seq=32, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048,
                         k=512, Hq=64, ctx=131072),
    "chain1m": Config("chain1m", 2, "chain", n_seq=8, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048, k=512,
                      Hq=64, ctx=2 ** 20,
                      modes=("full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse")),
    "prefill": Config("prefill", 3, "prefill", n_seq=1, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048, k=512,
                      Hq=64, ctx=131096, T=4096, pos0=127000),
    "mixed": Config("mixed", 4, "mixed", n_seq=64, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048, k=512, Hq=64,
                    append_per_seq=1024),
    # the prefill chunk through a Full group and a Reindex group of the decoder schedule
    "prefill_chain": Config("prefill_chain", 5, "prefill", n_seq=1, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048,
                            k=512, Hq=64, ctx=131096, T=4096, pos0=127000,
                            modes=("full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse")),
    # the 20 decoder layers (1 Full + 3 Reuse, then 4 x (1 Reindex + 3 Reuse)) at 1M context
    "decoder1m": Config("decoder1m", 6, "chain", n_seq=4, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048, k=512,
                        Hq=64, ctx=2 ** 20,
                        modes=("full", "reuse", "reuse", "reuse") + ("reindex", "reuse", "reuse", "reuse") * 4),
    # the 18 encoder layers (3 x (1 Full + 5 Reuse)) over a 1,024-query chunk
    "encoder_chunk": Config("encoder_chunk", 7, "prefill", n_seq=1, H=16, D=128, qk=(-8, 8), wr=(1, 8), P=2048,
                            k=512, Hq=64, ctx=131072, T=1024, pos0=130048,
                            modes=("full", "reuse", "reuse", "reuse", "reuse", "reuse") * 3),
}

# entity ids: sequences use their index; per-(layer, query) tensors use
# (layer + 1) << 16 | query, so streams never collide. Counters are
# entity << 40 | element, so entities stay below 2^23 (127 layers, 65,536 queries).


def lq(layer: int, i: int) -> int:
    if not (0 <= layer < 127 and 0 <= i < (1 << 16)):
        raise ValueError(f"layer {layer} / query {i} outside the stream-id range")
    return ((layer + 1) << 16) | i


# ---- per-row generators (any device) ----------------------------------------

def idx_k_rows(cfg: Config, s: int, rows: torch.Tensor) -> torch.Tensor:
    return int_bf16_rows(cfg.seed, "idx_k", s, rows, cfg.D, *cfg.qk)


def kv_rows(cfg: Config, s: int, rows: torch.Tensor) -> torch.Tensor:
    """bf16 main-KV latent rows of sequence s at positions `rows`."""
    x = normal_bf16_rows(cfg.seed, "kv", s, rows, cfg.C, outliers=True)
    if cfg.kind == "mixed":
        L = int(cfg.seq_lengths()[s])
        appended = (rows >= L - cfg.append_per_seq)
        z = bernoulli_rows(cfg.seed, "kv_zero", s, rows, cfg.C // 16, ZERO_GROUP_THRESHOLD)
        z = z & appended[:, None]
        x = torch.where(z.repeat_interleave(16, dim=1), torch.zeros((), dtype=x.dtype, device=x.device), x)
    return x


def window_rows(cfg: Config, layer: int, s: int, positions: torch.Tensor, which: str) -> torch.Tensor:
    """Sliding-window keys (which='k') or values ('v') of a layer at the given positions."""
    return normal_bf16_rows(cfg.seed, f"swa_{which}/{layer}", s, positions, cfg.C, outliers=False)


def indexer_query(cfg: Config, layer: int, i: int, device="cpu"):
    rows = torch.arange(cfg.H, dtype=torch.int64, device=device)
    q = int_bf16_rows(cfg.seed, "idx_q", lq(layer, i), rows, cfg.D, *cfg.qk)
    w = int_tensor_f32(cfg.seed, "w", lq(layer, i), (cfg.H,), *cfg.wr, device=device)
    return q, w


def main_query(cfg: Config, layer: int, i: int, device="cpu") -> torch.Tensor:
    return normal_bf16(cfg.seed, "q", lq(layer, i), (cfg.Hq, cfg.C), outliers=False, device=device)


def sequence_of(cfg: Config, i: int) -> int:
    return 0 if cfg.kind == "prefill" else i


# ---- whole-tensor generators for the device side -------------------------------

def chunks(n: int, step: int):
    for a in range(0, n, step):
        yield a, min(n, a + step)


def fill_idx_k(cfg: Config, out: torch.Tensor, chunk_rows: int = 1 << 20):
    """All indexer keys, sequences concatenated, into out [total_rows, D] (bf16)."""
    starts, lens = cfg.seq_starts(), cfg.seq_lengths()
    for s in range(cfg.n_seq):
        for a, b in chunks(int(lens[s]), chunk_rows):
            rows = torch.arange(a, b, dtype=torch.int64, device=out.device)
            out[starts[s] + a:starts[s] + b] = idx_k_rows(cfg, s, rows)


def kv_rows_into(cfg: Config, s: int, a: int, b: int, device) -> torch.Tensor:
    return kv_rows(cfg, s, torch.arange(a, b, dtype=torch.int64, device=device))


def indexer_queries(cfg: Config, layer: int, device):
    nq = cfg.n_queries()
    qs, ws = [], []
    for i in range(nq):
        q, w = indexer_query(cfg, layer, i, device)
        qs.append(q); ws.append(w)
    return torch.stack(qs).contiguous(), torch.stack(ws).contiguous()


def indexer_queries_fast(cfg: Config, layer: int, device):
    """Same values as indexer_queries, generated in one pass."""
    nq = cfg.n_queries()
    ent = torch.tensor([lq(layer, i) for i in range(nq)], dtype=torch.int64, device=device)
    hd = torch.arange(cfg.H * cfg.D, dtype=torch.int64, device=device)
    from . import randint
    cq = (ent[:, None] << ENTITY_SHIFT) + hd[None, :]
    q = randint(cfg.seed, "idx_q", cq, *cfg.qk).to(torch.float32).to(torch.bfloat16).reshape(nq, cfg.H, cfg.D)
    cw = (ent[:, None] << ENTITY_SHIFT) + torch.arange(cfg.H, dtype=torch.int64, device=device)[None, :]
    w = randint(cfg.seed, "w", cw, *cfg.wr).to(torch.float32)
    return q.contiguous(), w.contiguous()


def main_queries_fast(cfg: Config, layer: int, device):
    from . import normal_f32, f32_to_bf16_bits, bits_to_bf16
    nq = cfg.n_queries()
    ent = torch.tensor([lq(layer, i) for i in range(nq)], dtype=torch.int64, device=device)
    hc = torch.arange(cfg.Hq * cfg.C, dtype=torch.int64, device=device)
    c = (ent[:, None] << ENTITY_SHIFT) + hc[None, :]
    x = bits_to_bf16(f32_to_bf16_bits(normal_f32(cfg.seed, "q", c, outliers=False)))
    return x.reshape(nq, cfg.Hq, cfg.C).contiguous()


def decode_windows(cfg: Config, layer: int, device):
    """[B, W, C] window keys and values for decode queries (row W-1 = the query's position;
    rows before position 0 are zero and never read)."""
    B, W = cfg.n_seq, cfg.W
    qp = cfg.q_pos()
    ks = torch.zeros((B, W, cfg.C), dtype=torch.bfloat16, device=device)
    vs = torch.zeros_like(ks)
    for s in range(B):
        p = int(qp[s])
        n = min(W, p + 1)
        pos = torch.arange(p - n + 1, p + 1, dtype=torch.int64, device=device)
        ks[s, W - n:] = window_rows(cfg, layer, s, pos, "k")
        vs[s, W - n:] = window_rows(cfg, layer, s, pos, "v")
    return ks, vs


def prefill_window(cfg: Config, layer: int, device):
    """[T+W-1, C] shared window keys and values; row r = position pos0-W+1+r."""
    W = cfg.W
    pos = torch.arange(cfg.pos0 - W + 1, cfg.pos0 + cfg.T, dtype=torch.int64, device=device)
    valid = pos >= 0
    posc = torch.where(valid, pos, torch.zeros_like(pos))
    ks = window_rows(cfg, layer, 0, posc, "k")
    vs = window_rows(cfg, layer, 0, posc, "v")
    z = torch.zeros((), dtype=ks.dtype, device=device)
    return torch.where(valid[:, None], ks, z).contiguous(), torch.where(valid[:, None], vs, z).contiguous()
