"""GPU parity at small shapes: every kernel against the oracle, through the C ABI.

Indices, pools and FP4 bytes must be bit-exact; attention must satisfy
max|out - ref| <= 2e-4 * max|ref| + 1e-6 per output tensor.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, fp4, indexer
from synth import bf16_to_f64, bits_to_bf16, f32_to_bf16_bits, int_tensor_bf16, normal_bf16
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


# ------------------------------------------------------------------ codec ----

def test_quantize_all_bf16_values(fk, gpu):
    """Every finite bf16 value, in groups whose amax sweeps the whole range."""
    _say("quantize: all finite bf16 values")
    bits = torch.arange(0, 1 << 16, dtype=torch.int64)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    g = torch.Generator().manual_seed(0)
    bits = bits[torch.randperm(bits.numel(), generator=g)]
    n = bits.numel() // 512 * 512
    x = bits_to_bf16(bits[:n]).reshape(-1, 512)
    codes = torch.empty((x.shape[0], 256), dtype=torch.uint8, device=gpu)
    scales = torch.empty((x.shape[0], 32), dtype=torch.uint8, device=gpu)
    fk.fp4kv_quantize_append(x.to(gpu), codes, scales)
    ref_c, ref_s = fp4.quantize_rows(bf16_to_f64(x))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_scaled_groups(fk, gpu):
    """Groups scaled over 2^-40 .. 2^40, ties planted at scale and value midpoints,
    all-zero groups, negative zeros."""
    _say("quantize: scaled groups and planted ties")
    g = torch.Generator().manual_seed(1)
    R = 4096
    x = torch.randn((R, 512), generator=g)
    e = torch.randint(-40, 41, (R, 32, 1), generator=g).to(torch.float32)
    x = (x.reshape(R, 32, 16) * torch.exp2(e)).reshape(R, 512)
    # planted ties: amax = 6 * midpoint of neighbouring E4M3 values; values at E2M1 midpoints
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(0, R, 7):
        grp = x[r].reshape(32, 16)
        c = int(torch.randint(1, 126, (1,), generator=g))
        s_mid = 0.5 * (fp4.e4m3_value(c) + fp4.e4m3_value(c + 1))
        grp[0, 1:] = s_mid * 1e-3
        grp[0, 0] = 6 * s_mid
        s = fp4.e4m3_value(c)
        grp[1, :7] = mids * s
        grp[1, 7] = 6 * s
        grp[2] = 0.0
        grp[3, :4] = -0.0
    xb = x.to(torch.bfloat16)
    codes = torch.empty((R, 256), dtype=torch.uint8, device=gpu)
    scales = torch.empty((R, 32), dtype=torch.uint8, device=gpu)
    fk.fp4kv_quantize_append(xb.to(gpu), codes, scales)
    ref_c, ref_s = fp4.quantize_rows(bf16_to_f64(xb))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_scatter_and_bounds(fk, gpu):
    """dst_rows scatter; rows outside the cache are skipped; contiguous append at an offset."""
    _say("quantize: scatter, skipped rows, offset append")
    x = normal_bf16(7, "kv", 0, (10, 512), outliers=True).to(gpu)
    codes = torch.full((16, 256), 0xAB, dtype=torch.uint8, device=gpu)
    scales = torch.full((16, 32), 0xCD, dtype=torch.uint8, device=gpu)
    dst = torch.tensor([3, 15, -1, 16, 0, 7, 1000, 2, 9, 4], dtype=torch.int64, device=gpu)
    fk.fp4kv_quantize_append(x, codes, scales, dst_rows=dst)
    ref_c, ref_s = fp4.quantize_rows(bf16_to_f64(x))
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    written = set()
    for i, d in enumerate(dst.tolist()):
        if 0 <= d < 16:
            assert np.array_equal(c[d], ref_c[i]) and np.array_equal(s[d], ref_s[i])
            written.add(d)
    for d in set(range(16)) - written:
        assert (c[d] == 0xAB).all() and (s[d] == 0xCD).all()
    fk.fp4kv_quantize_append(x[:4], codes, scales, dst_start=12)
    assert np.array_equal(codes[12:16].cpu().numpy(), ref_c[:4])


# ---------------------------------------------------------------- indexer ----

def _indexer_case(fk, gpu, lengths, H, D, P, k, seed, lo=-8, hi=8, q_per_seq=1, positions=None):
    """Sequences of the given lengths, one query per sequence at its last
    position (or q_per_seq queries at `positions` of a single sequence)."""
    n_seq = len(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(np.sum(lengths))
    kk = int_tensor_bf16(seed, "k", 0, (total, D), lo, hi)
    if positions is None:
        qpos = (np.asarray(lengths) - 1).astype(np.int32)
    else:
        qpos = np.asarray(positions, dtype=np.int32)
    nq = len(qpos)
    q = int_tensor_bf16(seed, "q", 0, (nq, H, D), lo, hi)
    w = torch.randint(1, 9, (nq, H), generator=torch.Generator().manual_seed(seed)).to(torch.float32)
    max_ctx = int(qpos.max()) + 1 + 3
    pool, npool, idx, nidx = fk.fp4kv_index_full(
        q.to(gpu), w.to(gpu), kk.to(gpu), torch.from_numpy(starts).to(gpu), torch.from_numpy(qpos).to(gpu),
        q_per_seq, max_ctx, P, k)
    torch.cuda.synchronize()
    pool, npool, idx, nidx = pool.cpu().numpy(), npool.cpu().numpy(), idx.cpu().numpy(), nidx.cpu().numpy()
    kf = bf16_to_f64(kk)
    for i in range(nq):
        s = i // q_per_seq
        rows = kf[starts[s]:starts[s] + lengths[s]]
        rp, ri, _ = indexer.index_full(bf16_to_f64(q[i]), w[i].numpy().astype(np.float64), rows, int(qpos[i]), P, k)
        assert npool[i] == len(rp), (i, npool[i], len(rp))
        assert np.array_equal(pool[i, :len(rp)], rp) and (pool[i, len(rp):] == -1).all(), i
        assert nidx[i] == len(ri), (i, nidx[i], len(ri))
        assert np.array_equal(idx[i, :len(ri)], ri) and (idx[i, len(ri):] == -1).all(), i
    return q, w, kk, starts, qpos, pool, npool


@pytest.mark.parametrize("lengths,H,D,P,k", [
    ([4096], 4, 64, 64, 128),                       # the tiny decode shape (pool smaller than k)
    ([1, 7, 8, 9, 63, 64, 65, 1000], 4, 64, 4, 16),  # partial blocks, fewer blocks than P
    ([5000, 3, 12345], 16, 128, 64, 32),
    ([20000, 16384, 777], 8, 128, 2048, 512),      # pool covers all blocks
    ([40000, 40001], 16, 64, 300, 2400),           # k > P positions of small pools
])
def test_index_full_matches_oracle(fk, gpu, lengths, H, D, P, k):
    _say(f"index_full lengths={lengths} H={H} D={D} P={P} k={k}")
    _indexer_case(fk, gpu, lengths, H, D, P, k, seed=len(lengths) * 100 + H)


@pytest.mark.parametrize("P,k", [
    (32, 64),     # pool smaller than k: every visible pool position is a candidate
    (64, 32),     # pool of >= k blocks: positions scoring below the pool threshold are dropped first
])
def test_index_full_ties(fk, gpu, P, k):
    """Tiny value range: scores tie heavily at both selection levels, so the
    k-th best position often scores exactly the pool's threshold."""
    _say(f"index_full heavy ties P={P} k={k}")
    _indexer_case(fk, gpu, [3000, 2999, 16], 4, 64, P, k, seed=5, lo=-1, hi=1)


def test_index_full_all_equal_scores_pool_above_k(fk, gpu):
    """All scores tie and the pool holds more blocks than k: the token search
    keeps every pool position (all at the threshold) and takes the lowest."""
    _say("index_full all-equal scores, P >= k")
    _indexer_case(fk, gpu, [5000, 9, 130], 8, 64, 40, 16, seed=24, lo=1, hi=1)


def test_index_full_empty_contexts(fk, gpu):
    """Zero-length contexts inside a ragged batch (query position -1): empty
    pool and selection, and the neighbours' rows stay invisible to them."""
    _say("index_full empty contexts")
    _indexer_case(fk, gpu, [3000, 0, 17, 0, 1], 16, 128, 64, 100, seed=21)


def test_index_full_all_equal_scores(fk, gpu):
    """Every key and query equal: all scores tie, so both levels take the
    lowest blocks / positions (the radix search ends before its first digit)."""
    _say("index_full all-equal scores")
    _indexer_case(fk, gpu, [5000, 9, 130], 8, 64, 16, 40, seed=23, lo=1, hi=1)


def test_index_full_long_block_lists(fk, gpu):
    """More than 16,384 blocks: the block maxima are re-read in chunks, with a
    ragged last chunk, and the pool is compacted chunk by chunk."""
    _say("index_full long block lists")
    _indexer_case(fk, gpu, [140000, 300001, 5000], 4, 64, 2048, 512, seed=51)


def test_index_full_long_block_lists_ties(fk, gpu):
    """Heavy ties across chunks: ties go to the lowest block ids, so they are
    taken from the first chunks in order."""
    _say("index_full long block lists with ties")
    _indexer_case(fk, gpu, [200000, 150001], 4, 64, 2048, 512, seed=53, lo=-1, hi=1)


def test_index_full_prefill_positions(fk, gpu):
    """One sequence, many queries at consecutive positions (causal)."""
    _say("index_full prefill-style positions")
    L = 3000
    _indexer_case(fk, gpu, [L], 16, 128, 16, 40, seed=9, q_per_seq=37, positions=list(range(L - 37, L)))


@pytest.mark.parametrize("H,D", [(16, 128), (4, 64), (8, 128)])
def test_index_full_many_queries_per_sequence(fk, gpu, H, D):
    """Sequences with >= 16 queries each take the matrix-core scan: ragged
    lengths, a 32-query block cut short by the sequence, positions anywhere in
    the sequence (and -1)."""
    _say(f"index_full many queries per sequence H={H} D={D}")
    lengths, q_per_seq = [2500, 9000, 40], 48
    rng = np.random.default_rng(H * 100 + D)
    positions = []
    for L in lengths:
        positions += rng.integers(-1, L, size=q_per_seq).tolist()
    _indexer_case(fk, gpu, lengths, H, D, 64, 100, seed=31 + H, q_per_seq=q_per_seq, positions=positions)


@pytest.mark.parametrize("H,D", [(16, 128), (4, 64)])
def test_scores_matrix_core_scan_equals_decode_scan(fk, gpu, H, D):
    """Every token score and block maximum of the matrix-core scan (many queries
    per sequence) equals the per-query scan's bit for bit; unwritten entries stay
    untouched in both."""
    _say(f"scores: matrix-core scan vs per-query scan H={H} D={D}")
    L, T = 20000, 100
    kk = int_tensor_bf16(41, "k", 0, (L, D), -8, 8).to(gpu)
    q = int_tensor_bf16(41, "q", 0, (T, H, D), -8, 8).to(gpu)
    w = torch.randint(1, 9, (T, H), generator=torch.Generator().manual_seed(41)).to(torch.float32).to(gpu)
    pos = torch.from_numpy(np.random.default_rng(41).integers(-1, L, size=T).astype(np.int32)).to(gpu)
    max_ctx = L
    nblk = (max_ctx + 7) // 8
    outs = []
    for q_per_seq, starts in ((T, torch.zeros(1, dtype=torch.int64)), (1, torch.zeros(T, dtype=torch.int64))):
        sc = torch.full((T, max_ctx), float("nan"), device=gpu)
        bm = torch.full((T, nblk), float("nan"), device=gpu)
        fk.fp4kv_index_scores(q, w, kk, starts.to(gpu), pos, q_per_seq, max_ctx, scores=sc, blockmax=bm)
        outs.append((sc.view(torch.int32).cpu(), bm.view(torch.int32).cpu()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    written = ~torch.isnan(outs[0][0].view(torch.float32))
    assert int(written.sum()) == int((pos.cpu().clamp(min=-1) + 1).sum())


def test_index_reindex_matches_oracle(fk, gpu):
    _say("index_reindex")
    lengths = [9000, 33, 5000]
    q, w, kk, starts, qpos, pool, npool = _indexer_case(fk, gpu, lengths, 16, 128, 64, 100, seed=11)
    nq = len(lengths)
    q2 = int_tensor_bf16(12, "q2", 0, (nq, 16, 128), -8, 8)
    w2 = torch.randint(1, 9, (nq, 16), generator=torch.Generator().manual_seed(12)).to(torch.float32)
    idx, nidx = fk.fp4kv_index_reindex(q2.to(gpu), w2.to(gpu), kk.to(gpu), torch.from_numpy(starts).to(gpu),
                                       torch.from_numpy(qpos).to(gpu), 1, torch.from_numpy(pool).to(gpu),
                                       torch.from_numpy(npool).to(gpu), 100)
    idx, nidx = idx.cpu().numpy(), nidx.cpu().numpy()
    kf = bf16_to_f64(kk)
    for i in range(nq):
        rows = kf[starts[i]:starts[i] + lengths[i]]
        ref = indexer.index_reindex(bf16_to_f64(q2[i]), w2[i].numpy().astype(np.float64), lambda p: rows[p],
                                    pool[i, :npool[i]], int(qpos[i]), 100)
        assert nidx[i] == len(ref) and np.array_equal(idx[i, :len(ref)], ref), i
    # Reindex with the Full layer's own query reproduces the Full indices
    idx_same, _ = fk.fp4kv_index_reindex(q.to(gpu), w.to(gpu), kk.to(gpu), torch.from_numpy(starts).to(gpu),
                                         torch.from_numpy(qpos).to(gpu), 1, torch.from_numpy(pool).to(gpu),
                                         torch.from_numpy(npool).to(gpu), 100)
    for i in range(nq):
        rows = kf[starts[i]:starts[i] + lengths[i]]
        _, ri, _ = indexer.index_full(bf16_to_f64(q[i]), w[i].numpy().astype(np.float64), rows, int(qpos[i]), 64, 100)
        assert np.array_equal(idx_same[i, :len(ri)].cpu().numpy(), ri)


# -------------------------------------------------------------- attention ----

def _attn_case(fk, gpu, lengths, n_idx, Hq, k, W, seed):
    B = len(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(np.sum(lengths))
    x = normal_bf16(seed, "kv", 0, (total, 512), outliers=True)
    codes = torch.empty((total, 256), dtype=torch.uint8, device=gpu)
    scales = torch.empty((total, 32), dtype=torch.uint8, device=gpu)
    fk.fp4kv_quantize_append(x.to(gpu), codes, scales)
    rng = np.random.default_rng(seed)
    qpos = (np.asarray(lengths) - 1).astype(np.int32)
    idx = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        m = min(n_idx[b], lengths[b])
        idx[b, :m] = np.sort(rng.choice(lengths[b], size=m, replace=False))
    nidx = np.array([min(n_idx[b], lengths[b]) for b in range(B)], dtype=np.int32)
    q = normal_bf16(seed, "q", 0, (B, Hq, 512), outliers=False)
    wk = normal_bf16(seed, "wk", 0, (B, W, 512), outliers=False)
    wv = normal_bf16(seed, "wv", 0, (B, W, 512), outliers=False)
    scale = 1.0 / math.sqrt(512)
    out, lse = fk.fp4kv_sparse_attn_decode(q.to(gpu), codes, scales, torch.from_numpy(starts).to(gpu),
                                           torch.from_numpy(idx).to(gpu), torch.from_numpy(nidx).to(gpu),
                                           wk.to(gpu), wv.to(gpu), torch.from_numpy(qpos).to(gpu), scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ref_rows = fp4.dequantize_rows(*fp4.quantize_rows(bf16_to_f64(x)))
    for b in range(B):
        rows = ref_rows[starts[b] + idx[b, :nidx[b]]]
        nw = min(W, int(qpos[b]) + 1)
        ro, rl = attention.attend(bf16_to_f64(q[b]), rows, bf16_to_f64(wk[b, W - nw:]), bf16_to_f64(wv[b, W - nw:]),
                                  scale)
        ok, err, tol = within_tolerance(out[b], ro)
        assert ok, (b, err, tol)
        ok, err, tol = within_tolerance(lse[b], rl)
        assert ok, ("lse", b, err, tol)


@pytest.mark.parametrize("lengths,n_idx,Hq,k,W", [
    ([4096], [128], 16, 128, 128),                     # tiny decode shape
    ([5000, 300, 70, 1], [512, 300, 17, 1], 64, 512, 128),   # ragged counts, short windows
    ([2000] * 6, [0, 1, 31, 32, 33, 500], 32, 512, 128),      # empty sparse branch, chunk edges
    ([100000, 3000], [512, 512], 64, 512, 100),        # window not a multiple of 32
    ([2000, 0, 40], [100, 0, 40], 64, 512, 128),       # a query with no row at all: out 0, lse -inf
])
def test_attention_matches_oracle(fk, gpu, lengths, n_idx, Hq, k, W):
    _say(f"attention lengths={lengths} n_idx={n_idx} Hq={Hq}")
    _attn_case(fk, gpu, lengths, n_idx, Hq, k, W, seed=sum(lengths) % 1000)


def test_attention_prefill_matches_oracle(fk, gpu):
    """Prefill window addressing: queries at positions pos0..pos0+T-1 share one window buffer."""
    _say("attention prefill")
    L, T, W, Hq, k = 3000, 40, 128, 64, 256
    pos0 = 90          # early queries have windows clipped at position 0
    x = normal_bf16(3, "kv", 0, (L, 512), outliers=True)
    codes = torch.empty((L, 256), dtype=torch.uint8, device=gpu)
    scales = torch.empty((L, 32), dtype=torch.uint8, device=gpu)
    fk.fp4kv_quantize_append(x.to(gpu), codes, scales)
    rng = np.random.default_rng(3)
    idx = np.full((T, k), -1, dtype=np.int32)
    nidx = np.zeros(T, dtype=np.int32)
    for i in range(T):
        m = min(k, pos0 + i + 1)
        idx[i, :m] = np.sort(rng.choice(pos0 + i + 1, size=m, replace=False))
        nidx[i] = m
    q = normal_bf16(3, "q", 0, (T, Hq, 512), outliers=False)
    wbuf_k = normal_bf16(3, "wk", 0, (T + W - 1, 512), outliers=False)
    wbuf_v = normal_bf16(3, "wv", 0, (T + W - 1, 512), outliers=False)
    scale = 1.0 / math.sqrt(512)
    out, lse = fk.fp4kv_sparse_attn_prefill(q.to(gpu), codes, scales, 0, torch.from_numpy(idx).to(gpu),
                                            torch.from_numpy(nidx).to(gpu), wbuf_k.to(gpu), wbuf_v.to(gpu),
                                            pos0, W, scale)
    out = out.cpu().numpy()
    ref_rows = fp4.dequantize_rows(*fp4.quantize_rows(bf16_to_f64(x)))
    for i in range(T):
        p = pos0 + i
        nw = min(W, p + 1)
        r0 = i + W - nw
        ro, _ = attention.attend(bf16_to_f64(q[i]), ref_rows[idx[i, :nidx[i]]], bf16_to_f64(wbuf_k[r0:i + W]),
                                 bf16_to_f64(wbuf_v[r0:i + W]), scale)
        ok, err, tol = within_tolerance(out[i], ro)
        assert ok, (i, err, tol)


# ------------------------------------------------------------ error paths ----

def test_abi_rejects_bad_arguments(fk, gpu):
    _say("ABI validation")
    x = torch.zeros((4, 512), dtype=torch.bfloat16, device=gpu)
    codes = torch.zeros((4, 256), dtype=torch.uint8, device=gpu)
    scales = torch.zeros((4, 32), dtype=torch.uint8, device=gpu)
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_quantize_append(x, codes, scales, dst_start=2)
    assert e.value.status == -2
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device=gpu)
    w = torch.ones((1, 4), dtype=torch.float32, device=gpu)
    kk = torch.zeros((64, 64), dtype=torch.bfloat16, device=gpu)
    ss = torch.zeros(1, dtype=torch.int64, device=gpu)
    qp = torch.tensor([63], dtype=torch.int32, device=gpu)
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_index_full(q, w, kk, ss, qp, 1, 64, 8, 65)         # k > P*8
    assert e.value.status == -2
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_index_full(q, w, kk, ss, qp, 1, 64, 8, 8, workspace=torch.zeros(4, dtype=torch.uint8, device=gpu))
    assert e.value.status == -3
    q3 = torch.zeros((1, 3, 64), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_index_full(q3, w[:, :3].contiguous(), kk, ss, qp, 1, 64, 8, 8)
    assert e.value.status == -4
    # attention reads the scales as aligned 32-bit words: a scales pointer off
    # a 4-byte boundary is refused before anything is launched
    qa = torch.zeros((1, 16, 512), dtype=torch.bfloat16, device=gpu)
    sbuf = torch.zeros(4 * 32 + 4, dtype=torch.uint8, device=gpu)
    idx = torch.zeros((1, 8), dtype=torch.int32, device=gpu)
    nidx = torch.ones(1, dtype=torch.int32, device=gpu)
    win = torch.zeros((1, 8, 512), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_sparse_attn_decode(qa, codes, sbuf[1:1 + 4 * 32].view(4, 32), ss, idx, nidx, win, win, qp, 1.0)
    assert e.value.status == -2
    out, _ = fk.fp4kv_sparse_attn_decode(qa, codes, sbuf[4:4 + 4 * 32].view(4, 32), ss, idx, nidx, win, win, qp, 1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_repeatable_bits(fk, gpu):
    """Two runs give identical bits (no dependence on atomic ordering)."""
    _say("determinism")
    a = _indexer_case(fk, gpu, [30000, 7777], 16, 128, 256, 512, seed=21, lo=-1, hi=1)
    b = _indexer_case(fk, gpu, [30000, 7777], 16, 128, 256, 512, seed=21, lo=-1, hi=1)
    assert np.array_equal(a[5], b[5])


@pytest.mark.parametrize("P,k", [(64, 96), (64, 40)])
def test_index_full_many_queries_narrow_selection(fk, gpu, P, k):
    """300 queries (one selection workgroup per query, which writes the pool
    and narrows it to the k best blocks, in the instance held to 64 VGPRs so
    that two share a CU), short ragged contexts with heavy ties, the pool
    smaller and larger than k: every query's pool and indices against the oracle."""
    _say(f"index_full 300 queries, narrow selection instance, P={P} k={k}")
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 3000, 300)]
    _indexer_case(fk, gpu, lengths, 4, 64, P, k, seed=31, lo=-1, hi=1)


@pytest.mark.parametrize("P,k,lo,hi", [
    (1024, 2048, -8, 8),    # pool of 1,024 blocks, smaller than k: all of its positions searched
    (2048, 1024, -8, 8),    # k = 1,024 best blocks of the pool
    (2048, 1024, -1, 1),    # the same with heavy ties
])
def test_index_full_wide_token_search(fk, gpu, P, k, lo, hi):
    """More than 512 blocks reach the token search, so each thread holds 16
    candidates (two blocks): few queries (two workgroups per query) and 260
    queries of one sequence (one workgroup per query, the pool narrowed to k)."""
    _say(f"index_full wide token search P={P} k={k} values {lo}..{hi}")
    _indexer_case(fk, gpu, [30000, 20001, 12345], 4, 64, P, k, seed=71, lo=lo, hi=hi)
    rng = np.random.default_rng(73)
    positions = sorted(int(x) for x in rng.integers(9000, 30000, 260))
    _indexer_case(fk, gpu, [30000], 4, 64, P, k, seed=73, lo=lo, hi=hi, q_per_seq=260, positions=positions)


@pytest.mark.parametrize("P,k", [(64, 96), (64, 40)])
def test_index_full_two_roles_narrow_instance(fk, gpu, P, k):
    """200 queries: two selection workgroups per query (pool, positions) in
    the instance held to 64 VGPRs, short ragged contexts with heavy ties, the
    pool smaller and larger than k: every query against the oracle."""
    _say(f"index_full 200 queries, two roles, narrow instance, P={P} k={k}")
    rng = np.random.default_rng(37)
    lengths = [int(x) for x in rng.integers(1, 3000, 200)]
    _indexer_case(fk, gpu, lengths, 4, 64, P, k, seed=37, lo=-1, hi=1)


@pytest.mark.parametrize("lo,hi", [(-8, 8), (-1, 1)])
def test_index_full_one_workgroup_per_query_long(fk, gpu, lo, hi):
    """260 queries of one 140,000-token sequence (one selection workgroup per
    query, which writes the pool and then narrows it to its k best blocks),
    positions on both sides of 16,384 blocks (block maxima in registers or
    re-read in chunks), P >= k, and heavy ties in the second case: every
    query's pool and indices against the oracle."""
    _say(f"index_full 260 queries, one workgroup each, long contexts, values {lo}..{hi}")
    rng = np.random.default_rng(67)
    L = 140000
    positions = sorted(int(x) for x in rng.integers(100000, L, 260))
    _indexer_case(fk, gpu, [L], 4, 64, 2048, 512, seed=67, lo=lo, hi=hi, q_per_seq=260, positions=positions)


def test_repeatable_bits_attention_and_append(fk, gpu):
    """Attention (split partials + combine) and the quantize-append give
    identical bits when run twice on the same inputs."""
    _say("determinism: attention and append")
    lengths = [50000, 3000, 777, 20000]
    B, k, W, Hq = len(lengths), 512, 128, 64
    starts = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)).to(gpu)
    total = int(np.sum(lengths))
    x = normal_bf16(41, "kv", 0, (total, 512), outliers=True, device=gpu)
    caches = []
    for _ in range(2):
        codes = torch.empty((total, 256), dtype=torch.uint8, device=gpu)
        scales = torch.empty((total, 32), dtype=torch.uint8, device=gpu)
        fk.fp4kv_quantize_append(x, codes, scales)
        caches.append((codes, scales))
    torch.cuda.synchronize()
    assert torch.equal(caches[0][0], caches[1][0]) and torch.equal(caches[0][1], caches[1][1])
    rng = np.random.default_rng(41)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(n, size=k, replace=False)) for n in lengths])
                           .astype(np.int32)).to(gpu)
    nidx = torch.full((B,), k, dtype=torch.int32, device=gpu)
    qpos = torch.tensor([n - 1 for n in lengths], dtype=torch.int32, device=gpu)
    q = normal_bf16(41, "q", 0, (B, Hq, 512), outliers=False, device=gpu)
    wk = normal_bf16(41, "wk", 0, (B, W, 512), outliers=False, device=gpu)
    wv = normal_bf16(41, "wv", 0, (B, W, 512), outliers=False, device=gpu)
    assert fk.fp4kv_attn_workspace_bytes(B, Hq, 512, k, W) > 0        # several splits and a combine
    runs = [fk.fp4kv_sparse_attn_decode(q, caches[0][0], caches[0][1], starts, idx, nidx, wk, wv, qpos,
                                        1.0 / math.sqrt(512)) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
