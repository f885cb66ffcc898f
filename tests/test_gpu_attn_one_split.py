"""Sparse attention in the one-split plan (a batch of 256 or more queries: one
workgroup per query, no partial results to combine), against the oracle for
every query and head.

The cases reach every branch of that path: sparse lists that are empty,
ragged inside a chunk, and long enough (k = 640, 20 chunks) that the positions
of the chunks past the sixteenth are read one by one rather than from the
vector load made at the start; windows clipped at position 0 and a window
length that is not a multiple of 32; a query at a negative position; and the
three main-KV formats.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, kvformats
from synth import bf16_to_f64, normal_bf16
from tests.oracle_runner import within_tolerance

pytestmark = pytest.mark.gpu

FMTS = [kvformats.FMT_FP4, kvformats.FMT_MXFP4, kvformats.FMT_FP8]
IDS = ["fp4", "mxfp4", "fp8"]


@pytest.fixture(scope="module")
def fk():
    import sparse_indexer_fp4_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _say(msg):
    print(msg, flush=True)


def _cache(fk, fmt, x, gpu):
    rows = x.shape[0]
    codes = torch.zeros((rows, fk.fp4kv_kv_code_bytes(fmt, 512)), dtype=torch.uint8, device=gpu)
    sb = fk.fp4kv_kv_scale_bytes(fmt, 512)
    scales = torch.zeros((rows, sb), dtype=torch.uint8, device=gpu) if sb > 0 else None
    fk.fp4kv_kv_append(fmt, x.to(gpu), codes, scales)
    ref = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, bf16_to_f64(x)))
    return codes, scales, ref


@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
@pytest.mark.parametrize("pos0,k,W", [(400, 640, 128), (5, 96, 100)], ids=["long-lists", "clipped-windows"])
def test_one_split_prefill(fk, gpu, fmt, pos0, k, W):
    """288 prefill queries at positions pos0 .. pos0+287; each keeps a random
    number (0 .. min(k, p+1)) of distinct earlier positions."""
    _say(f"one-split prefill fmt={IDS[fmt]} pos0={pos0} k={k} W={W}")
    T, Hq, L = 288, 64, 3000
    seed = 40 + fmt + pos0
    x = normal_bf16(seed, "kv", 0, (L, 512), outliers=True)
    codes, scales, ref = _cache(fk, fmt, x, gpu)
    rng = np.random.default_rng(seed)
    idx = np.full((T, k), -1, dtype=np.int32)
    nidx = np.zeros(T, dtype=np.int32)
    for i in range(T):
        cap = min(k, pos0 + i + 1)
        m = int(rng.integers(0, cap + 1)) if i % 4 else cap      # every fourth list is as long as it can be
        idx[i, :m] = np.sort(rng.choice(pos0 + i + 1, size=m, replace=False))
        nidx[i] = m
    q = normal_bf16(seed, "q", 0, (T, Hq, 512), outliers=False)
    wk = normal_bf16(seed, "wk", 0, (T + W - 1, 512), outliers=False)
    wv = normal_bf16(seed, "wv", 0, (T + W - 1, 512), outliers=False)
    scale = 1.0 / math.sqrt(512)
    out, lse = fk.fp4kv_sparse_attn_prefill_kv(fmt, q.to(gpu), codes, scales, 0, torch.from_numpy(idx).to(gpu),
                                               torch.from_numpy(nidx).to(gpu), wk.to(gpu), wv.to(gpu), pos0, W, scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf, wkf, wvf = bf16_to_f64(q), bf16_to_f64(wk), bf16_to_f64(wv)
    for i in range(T):
        p = pos0 + i
        nw = min(W, p + 1)
        r0 = i + W - nw
        ro, rl = attention.attend(qf[i], ref[idx[i, :nidx[i]]], wkf[r0:i + W], wvf[r0:i + W], scale)
        ok, err, tol = within_tolerance(out[i], ro)
        assert ok, (i, int(nidx[i]), err, tol)
        ok, err, tol = within_tolerance(lse[i], rl)
        assert ok, ("lse", i, err, tol)


@pytest.mark.parametrize("fmt", FMTS, ids=IDS)
def test_one_split_decode(fk, gpu, fmt):
    """260 decode queries over sequences of 0 .. 2,000 rows (a 0-row sequence
    puts its query at position -1: zero output, LSE -inf); k = 640, W = 100."""
    _say(f"one-split decode fmt={IDS[fmt]}")
    B, Hq, k, W = 260, 64, 640, 100
    seed = 60 + fmt
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 2001, size=B)
    lengths[[3, 100]] = 0
    lengths[[5, 7]] = [1, 33]
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(lengths.sum())
    x = normal_bf16(seed, "kv", 0, (total, 512), outliers=True)
    codes, scales, ref = _cache(fk, fmt, x, gpu)
    qpos = (lengths - 1).astype(np.int32)
    idx = np.full((B, k), -1, dtype=np.int32)
    nidx = np.zeros(B, dtype=np.int32)
    for b in range(B):
        cap = int(min(k, lengths[b]))
        m = cap if b % 3 == 0 else int(rng.integers(0, cap + 1))
        idx[b, :m] = np.sort(rng.choice(int(lengths[b]), size=m, replace=False))
        nidx[b] = m
    q = normal_bf16(seed, "q", 0, (B, Hq, 512), outliers=False)
    wk = normal_bf16(seed, "wk", 0, (B, W, 512), outliers=False)
    wv = normal_bf16(seed, "wv", 0, (B, W, 512), outliers=False)
    scale = 1.0 / math.sqrt(512)
    out, lse = fk.fp4kv_sparse_attn_decode_kv(fmt, q.to(gpu), codes, scales, torch.from_numpy(starts).to(gpu),
                                              torch.from_numpy(idx).to(gpu), torch.from_numpy(nidx).to(gpu),
                                              wk.to(gpu), wv.to(gpu), torch.from_numpy(qpos).to(gpu), scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf, wkf, wvf = bf16_to_f64(q), bf16_to_f64(wk), bf16_to_f64(wv)
    for b in range(B):
        if qpos[b] < 0:
            assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b])), b
            continue
        rows = ref[starts[b] + idx[b, :nidx[b]]]
        nw = min(W, int(qpos[b]) + 1)
        ro, rl = attention.attend(qf[b], rows, wkf[b, W - nw:], wvf[b, W - nw:], scale)
        ok, err, tol = within_tolerance(out[b], ro)
        assert ok, (b, int(nidx[b]), err, tol)
        ok, err, tol = within_tolerance(lse[b], rl)
        assert ok, ("lse", b, err, tol)
