"""GPU parity of the paged cache and the window ring through the C ABI.

* Appends: variable-count appends in several calls into a paged store with
  permuted physical pages equal the oracle's paged-store model byte for byte
  (main-KV codes and scales in each format, indexer keys), and the window ring
  equals the oracle's ring after the same appends.
* The method through pages: index_full_paged / index_reindex_paged give the
  same pools and indices as the contiguous calls (and the oracle), and
  sparse_attn_decode_paged with the ring gives the same bits as
  sparse_attn_decode_kv over contiguous rows and windows, and stays within
  max|out - ref| <= 2e-4 * max|ref| + 1e-6 of the oracle.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, indexer, kvformats, paged
from synth import bf16_to_f64, int_tensor_bf16, normal_bf16
from tests.oracle_runner import within_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import sparse_indexer_fp4_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _say(msg):
    print(msg, flush=True)


def _block_tables(lengths, page_rows, spare, seed):
    """Block tables over a random permutation of physical pages (plus spare pages)."""
    rng = np.random.default_rng(seed)
    need = [-(-n // page_rows) for n in lengths]
    n_pages = sum(need) + spare
    perm = rng.permutation(n_pages)
    bt = np.full((len(lengths), max(need) + 1), -1, dtype=np.int32)
    k = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[k:k + n]
        k += n
    return bt, n_pages


def _new_cache(fk, fmt, bt, page_rows, n_pages, C, D, gpu):
    rows = n_pages * page_rows
    codes = torch.zeros((rows, fk.fp4kv_kv_code_bytes(fmt, C)), dtype=torch.uint8, device=gpu)
    sb = fk.fp4kv_kv_scale_bytes(fmt, C)
    scales = torch.zeros((rows, sb), dtype=torch.uint8, device=gpu) if sb else None
    idx_k = torch.zeros((rows, D), dtype=torch.bfloat16, device=gpu)
    return fk.PagedCache(torch.from_numpy(bt).to(gpu), page_rows, n_pages, codes, scales, idx_k, fmt)


def _fill(fk, cache, kv_rows, k_rows, gpu, chunks):
    """Append every sequence's rows in `chunks` calls with interleaved, variable
    per-sequence counts (the varlen form: one (sequence, position) per row)."""
    lengths = [r.shape[0] for r in kv_rows]
    for c in range(chunks):
        seqs, poss, kv, kk = [], [], [], []
        for s, n in enumerate(lengths):
            a, b = n * c // chunks, n * (c + 1) // chunks
            seqs += [s] * (b - a)
            poss += list(range(a, b))
            kv.append(kv_rows[s][a:b]); kk.append(k_rows[s][a:b])
        if not seqs:
            continue
        fk.fp4kv_paged_kv_append(cache, torch.tensor(seqs, dtype=torch.int32, device=gpu),
                                 torch.tensor(poss, dtype=torch.int64, device=gpu),
                                 kv_src=torch.cat(kv).to(gpu), idxk_src=torch.cat(kk).to(gpu))


@pytest.mark.parametrize("fmt", [kvformats.FMT_FP4, kvformats.FMT_MXFP4, kvformats.FMT_FP8],
                         ids=["fp4", "mxfp4", "fp8"])
def test_paged_appends_and_ring(fk, gpu, fmt):
    _say(f"paged appends fmt={fmt}")
    lengths, page_rows, C, D, W = [300, 64, 1, 1000], 64, 512, 128, 100
    bt, n_pages = _block_tables(lengths, page_rows, spare=3, seed=20 + fmt)
    cache = _new_cache(fk, fmt, bt, page_rows, n_pages, C, D, gpu)
    kv_rows = [normal_bf16(20, "kv", s, (n, C), outliers=True) for s, n in enumerate(lengths)]
    k_rows = [int_tensor_bf16(20, "k", s, (n, D), -8, 8) for s, n in enumerate(lengths)]
    _fill(fk, cache, kv_rows, k_rows, gpu, chunks=3)
    # oracle: quantise the logical rows, then place them by the block table
    q = [kvformats.quantize_rows(fmt, bf16_to_f64(x)) for x in kv_rows]
    want_codes = paged.paged_store([c for c, _ in q], bt, page_rows, n_pages)
    assert np.array_equal(cache.codes.cpu().numpy(), want_codes)
    if cache.scales is not None:
        want_scales = paged.paged_store([s for _, s in q], bt, page_rows, n_pages)
        assert np.array_equal(cache.scales.cpu().numpy(), want_scales)
    want_k = paged.paged_store([bf16_to_f64(x) for x in k_rows], bt, page_rows, n_pages)
    assert np.array_equal(bf16_to_f64(cache.idx_k.cpu()), want_k)
    # window ring: the same rows appended as window state, in calls of at most W
    # consecutive positions per sequence (a call's positions of one sequence must
    # be distinct modulo W)
    ring_k = torch.zeros((len(lengths), W, C), dtype=torch.bfloat16, device=gpu)
    ring_v = torch.zeros_like(ring_k)
    wv_rows = [normal_bf16(21, "wv", s, (n, C), outliers=False) for s, n in enumerate(lengths)]
    calls = -(-max(lengths) // W)
    for c in range(calls):
        seqs, poss, kk, vv = [], [], [], []
        for s, n in enumerate(lengths):
            a, b = min(n, c * W), min(n, (c + 1) * W)
            seqs += [s] * (b - a); poss += list(range(a, b))
            kk.append(kv_rows[s][a:b]); vv.append(wv_rows[s][a:b])
        fk.fp4kv_swa_ring_append(torch.cat(kk).to(gpu), torch.cat(vv).to(gpu),
                                 torch.tensor(seqs, dtype=torch.int32, device=gpu),
                                 torch.tensor(poss, dtype=torch.int64, device=gpu), ring_k, ring_v)
    for s, n in enumerate(lengths):
        assert np.array_equal(bf16_to_f64(ring_k[s].cpu()), paged.ring_after_appends(bf16_to_f64(kv_rows[s]), W))
        assert np.array_equal(bf16_to_f64(ring_v[s].cpu()), paged.ring_after_appends(bf16_to_f64(wv_rows[s]), W))


@pytest.mark.parametrize("k,W", [(512, 128), (64, 600)], ids=["k512-W128", "k64-W600"])
@pytest.mark.parametrize("page_rows", [64, 256])
@pytest.mark.parametrize("fmt", [kvformats.FMT_FP4, kvformats.FMT_MXFP4, kvformats.FMT_FP8], ids=["fp4", "mxfp4", "fp8"])
def test_paged_decode_path(fk, gpu, page_rows, fmt, k, W):
    """Full and Reindex indexer and decode attention through pages equal the
    contiguous path bit for bit, and the oracle. With k = 64 and a 600-row
    window the launch takes 16 splits, and those that hold two window chunks
    load the second one a step ahead, from the ring (and its last chunk is
    partial)."""
    _say(f"paged decode path page_rows={page_rows} fmt={fmt} k={k} W={W}")
    lengths = [5000, 1500, 64, 9001]
    H, D, C, Hq, P = 16, 128, 512, 64, 256
    seed = 30 + page_rows + fmt
    n_seq = len(lengths)
    bt, n_pages = _block_tables(lengths, page_rows, spare=2, seed=seed)
    cache = _new_cache(fk, fmt, bt, page_rows, n_pages, C, D, gpu)
    kv_rows = [normal_bf16(seed, "kv", s, (n, C), outliers=True) for s, n in enumerate(lengths)]
    k_rows = [int_tensor_bf16(seed, "k", s, (n, D), -8, 8) for s, n in enumerate(lengths)]
    _fill(fk, cache, kv_rows, k_rows, gpu, chunks=2)
    # the same rows contiguous
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(sum(lengths))
    ccodes = torch.zeros((total, fk.fp4kv_kv_code_bytes(fmt, C)), dtype=torch.uint8, device=gpu)
    sb = fk.fp4kv_kv_scale_bytes(fmt, C)
    cscales = torch.zeros((total, sb), dtype=torch.uint8, device=gpu) if sb else None
    fk.fp4kv_kv_append(fmt, torch.cat(kv_rows).to(gpu), ccodes, cscales)
    ck = torch.cat(k_rows).to(gpu)
    seq_start = torch.from_numpy(starts).to(gpu)
    qpos = torch.tensor(np.asarray(lengths) - 1, dtype=torch.int32, device=gpu)
    q_idx = int_tensor_bf16(seed, "q", 0, (n_seq, H, D), -8, 8).to(gpu)
    w = torch.randint(1, 9, (n_seq, H), generator=torch.Generator().manual_seed(seed)).to(torch.float32).to(gpu)
    max_ctx = max(lengths) + 5
    pool_c, npool_c, idx_c, nidx_c = fk.fp4kv_index_full(q_idx, w, ck, seq_start, qpos, 1, max_ctx, P, k)
    pool_p, npool_p, idx_p, nidx_p = fk.fp4kv_index_full_paged(q_idx, w, cache, qpos, 1, max_ctx, P, k)
    for a, b in ((pool_c, pool_p), (npool_c, npool_p), (idx_c, idx_p), (nidx_c, nidx_p)):
        assert torch.equal(a, b)
    q2 = int_tensor_bf16(seed, "q2", 0, (n_seq, H, D), -8, 8).to(gpu)
    ridx_c, rn_c = fk.fp4kv_index_reindex(q2, w, ck, seq_start, qpos, 1, pool_c, npool_c, k)
    ridx_p, rn_p = fk.fp4kv_index_reindex_paged(q2, w, cache, qpos, 1, pool_p, npool_p, k)
    assert torch.equal(ridx_c, ridx_p) and torch.equal(rn_c, rn_p)
    # windows: contiguous [B, W, C] (row W-1 = newest) and the ring
    win_k = [normal_bf16(seed, "wk", s, (n, C), outliers=False) for s, n in enumerate(lengths)]
    win_v = [normal_bf16(seed, "wv", s, (n, C), outliers=False) for s, n in enumerate(lengths)]
    swa_k = torch.zeros((n_seq, W, C), dtype=torch.bfloat16)
    swa_v = torch.zeros_like(swa_k)
    for s, n in enumerate(lengths):
        m = min(W, n)
        swa_k[s, W - m:] = win_k[s][n - m:]; swa_v[s, W - m:] = win_v[s][n - m:]
    ring_k = torch.zeros((n_seq, W, C), dtype=torch.bfloat16, device=gpu)
    ring_v = torch.zeros_like(ring_k)
    # a prefill leaves only its last W positions in the ring: append those
    tails = [(s, max(0, n - W), n) for s, n in enumerate(lengths)]
    seqs = torch.cat([torch.full((b - a,), s, dtype=torch.int32) for s, a, b in tails]).to(gpu)
    poss = torch.cat([torch.arange(a, b, dtype=torch.int64) for s, a, b in tails]).to(gpu)
    fk.fp4kv_swa_ring_append(torch.cat([win_k[s][a:b] for s, a, b in tails]).to(gpu),
                             torch.cat([win_v[s][a:b] for s, a, b in tails]).to(gpu), seqs, poss, ring_k, ring_v)
    qm = normal_bf16(seed, "qm", 0, (n_seq, Hq, C), outliers=False).to(gpu)
    scale = 1.0 / math.sqrt(C)
    out_c, lse_c = fk.fp4kv_sparse_attn_decode_kv(fmt, qm, ccodes, cscales, seq_start, idx_c, nidx_c,
                                                  swa_k.to(gpu), swa_v.to(gpu), qpos, scale)
    out_p, lse_p = fk.fp4kv_sparse_attn_decode_paged(qm, cache, idx_p, nidx_p, ring_k, ring_v, qpos, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)
    # and the oracle, for the logical sequences
    idx_np, nidx_np = idx_c.cpu().numpy(), nidx_c.cpu().numpy()
    out_np = out_p.cpu().numpy()
    for s in (0, 3):
        kf = bf16_to_f64(k_rows[s])
        p = lengths[s] - 1
        rp, ri, _ = indexer.index_full(bf16_to_f64(q_idx[s].cpu()), w[s].cpu().numpy().astype(np.float64), kf, p, P, k)
        assert np.array_equal(idx_np[s, :nidx_np[s]], ri)
        rows = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, bf16_to_f64(kv_rows[s][ri])))
        m = min(W, p + 1)
        ro, _ = attention.attend(bf16_to_f64(qm[s].cpu()), rows, bf16_to_f64(win_k[s][p + 1 - m:p + 1]),
                                 bf16_to_f64(win_v[s][p + 1 - m:p + 1]), scale)
        ok, err, tol = within_tolerance(out_np[s], ro)
        assert ok, (s, err, tol)


def test_paged_decode128k(fk, gpu):
    """decode128k with its main KV and indexer keys in 256-row pages over a
    permuted page pool, and its windows in rings: pools, indices and attention
    bits equal the contiguous path for all 32 queries. Prints both paths' times."""
    from synth import workloads as wl
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["decode128k"]
    _say("paged decode128k: setup")
    dw = DeviceWorkload(cfg, gpu)
    page_rows = 256
    bt, n_pages = _block_tables([int(n) for n in dw.lengths], page_rows, spare=4, seed=99)
    cache = _new_cache(fk, kvformats.FMT_FP4, bt, page_rows, n_pages, cfg.C, cfg.D, gpu)
    starts = cfg.seq_starts()
    for s in range(cfg.n_seq):
        n = int(dw.lengths[s])
        for a, b in wl.chunks(n, 1 << 16):
            seqs = torch.full((b - a,), s, dtype=torch.int32, device=gpu)
            poss = torch.arange(a, b, dtype=torch.int64, device=gpu)
            fk.fp4kv_paged_kv_append(cache, seqs, poss, kv_src=wl.kv_rows_into(cfg, s, a, b, gpu),
                                     idxk_src=dw.idx_k[int(starts[s]) + a:int(starts[s]) + b])
    # rings holding each context's last W window rows (positions n-W .. n-1)
    W = cfg.W
    ring_k = torch.zeros((cfg.n_seq, W, cfg.C), dtype=torch.bfloat16, device=gpu)
    ring_v = torch.zeros_like(ring_k)
    seqs = torch.arange(cfg.n_seq, dtype=torch.int32, device=gpu).repeat_interleave(W)
    poss = torch.cat([torch.arange(int(n) - W, int(n), dtype=torch.int64) for n in dw.lengths]).to(gpu)
    fk.fp4kv_swa_ring_append(dw.swa_k[0].reshape(-1, cfg.C), dw.swa_v[0].reshape(-1, cfg.C), seqs, poss,
                             ring_k, ring_v)

    def contiguous():
        r = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1, cfg.ctx, cfg.P, cfg.k)
        o = fk.fp4kv_sparse_attn_decode(dw.q[0], dw.codes, dw.scales, dw.seq_start, r[2], r[3], dw.swa_k[0],
                                        dw.swa_v[0], dw.q_pos, cfg.scale)
        return r, o

    def paged_path():
        r = fk.fp4kv_index_full_paged(dw.idx_q[0], dw.w[0], cache, dw.q_pos, 1, cfg.ctx, cfg.P, cfg.k)
        o = fk.fp4kv_sparse_attn_decode_paged(dw.q[0], cache, r[2], r[3], ring_k, ring_v, dw.q_pos, cfg.scale)
        return r, o

    (rc, oc), (rp, op) = contiguous(), paged_path()
    torch.cuda.synchronize()
    _say("paged decode128k: checking")
    for a, b in zip(rc + oc, rp + op):
        assert torch.equal(a, b)
    for name, fn in (("contiguous", contiguous), ("paged (256-row pages, ring)", paged_path)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        _say(f"paged decode128k: {name}: index_full + attention {e0.elapsed_time(e1) / 10 * 1e3:.1f} us per call")
