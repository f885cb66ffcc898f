"""Paged main-KV and indexer-key storage and the sliding-window ring buffer.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this module; the product path never does.

[N] "FP4 KV Quantization and Cache Lifetime Management" describes serving-side
storage (a global KV cache with a long lifetime, window state kept apart from
it); [G] SWA Bounded Replay paragraph and [N] "Causal Encoder-Decoder and
Prefill Halving": each layer's window is the last 128 tokens. The pages give no
layout; this is the plainest one for a serving cache:

* A sequence's positions are cut into pages of `page_rows` consecutive
  positions; page i holds positions i*page_rows .. (i+1)*page_rows - 1.
  block_table[s, i] is the physical page of sequence s's page i, and physical
  page g is rows g*page_rows .. (g+1)*page_rows - 1 of every per-token store
  (main-KV codes, scales, indexer keys). A block-table entry outside
  [0, n_pages) maps nowhere.
* A layer's window ring holds W rows per sequence; position t lives in slot
  t mod W, so after the appends of positions 0..p it holds positions
  max(0, p-W+1)..p.

Everything the method computes is unchanged: paging only moves rows. The
oracle of a paged call is the oracle of the same logical sequence.
"""
from __future__ import annotations

import numpy as np


def physical_row(block_table: np.ndarray, page_rows: int, n_pages: int, seq: int, pos: int) -> int:
    """Physical row of position pos of sequence seq, or -1 if it maps nowhere."""
    if pos < 0:
        return -1
    page = pos // page_rows
    if page >= block_table.shape[1]:
        return -1
    g = int(block_table[seq, page])
    if g < 0 or g >= n_pages:
        return -1
    return g * page_rows + pos % page_rows


def ring_slot(pos: int, W: int) -> int:
    """Slot of position pos in a window ring of W rows."""
    return pos % W


def paged_store(rows_of_seq: list[np.ndarray], block_table: np.ndarray, page_rows: int, n_pages: int,
                fill=0) -> np.ndarray:
    """A paged store [n_pages*page_rows, width] holding each sequence's rows
    (rows_of_seq[s][t] at the physical row of (s, t)); unmapped rows keep `fill`."""
    width = rows_of_seq[0].shape[1]
    store = np.full((n_pages * page_rows, width), fill, dtype=rows_of_seq[0].dtype)
    for s, rows in enumerate(rows_of_seq):
        for t in range(rows.shape[0]):
            r = physical_row(block_table, page_rows, n_pages, s, t)
            if r >= 0:
                store[r] = rows[t]
    return store


def logical_rows(store: np.ndarray, block_table: np.ndarray, page_rows: int, n_pages: int, seq: int,
                 positions) -> np.ndarray:
    """Rows of `positions` of sequence seq read back through the block table."""
    out = []
    for t in np.asarray(positions, dtype=np.int64):
        r = physical_row(block_table, page_rows, n_pages, seq, int(t))
        assert r >= 0, (seq, t)
        out.append(store[r])
    return np.array(out).reshape(len(out), store.shape[1])


def ring_after_appends(rows: np.ndarray, W: int) -> np.ndarray:
    """A sequence's window ring [W, width] after appending rows[0..n-1] at positions
    0..n-1 in order (slot t mod W holds the last position written there)."""
    ring = np.zeros((W, rows.shape[1]), dtype=rows.dtype)
    for t in range(rows.shape[0]):
        ring[ring_slot(t, W)] = rows[t]
    return ring


def window_from_ring(ring: np.ndarray, p: int, W: int) -> np.ndarray:
    """Window rows of positions max(0, p-W+1)..p, oldest first, read from a ring."""
    return np.array([ring[ring_slot(t, W)] for t in range(max(0, p - W + 1), p + 1)]).reshape(-1, ring.shape[1])
