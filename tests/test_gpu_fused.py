"""The indexer with the layer's main-KV append in the same launch
(fp4kv_index_full_append, fp4kv_index_scores_append) against the separate calls
through the C ABI: identical pools, indices, scores and cache bytes, for the
three cache formats, scattered and contiguous destinations, an empty append, and
the matrix-core scan (which launches the append on its own)."""
import numpy as np
import pytest
import torch

from oracle import fp4
from synth import bf16_to_f64, int_tensor_bf16, normal_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import sparse_indexer_fp4_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _say(msg):
    print(msg, flush=True)


def _indexer(gpu, lengths, H, D, seed, positions=None):
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    kk = int_tensor_bf16(seed, "k", 0, (int(np.sum(lengths)), D), -8, 8, device=gpu)
    qpos = (np.asarray(lengths) - 1) if positions is None else np.asarray(positions)
    q = int_tensor_bf16(seed, "q", 0, (len(qpos), H, D), -8, 8, device=gpu)
    w = torch.randint(1, 9, (len(qpos), H), generator=torch.Generator().manual_seed(seed)).to(torch.float32).to(gpu)
    return q, w, kk, torch.from_numpy(starts).to(gpu), torch.from_numpy(qpos.astype(np.int32)).to(gpu), int(qpos.max()) + 1


def _cache(fk, gpu, fmt, rows, C=512):
    codes = torch.full((rows, fk.fp4kv_kv_code_bytes(fmt, C)), 0x5A, dtype=torch.uint8, device=gpu)
    sb = fk.fp4kv_kv_scale_bytes(fmt, C)
    scales = torch.full((rows, sb), 0x3C, dtype=torch.uint8, device=gpu) if sb > 0 else None
    return codes, scales


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("scatter", [False, True])
def test_index_full_append_matches_separate_calls(fk, gpu, fmt, scatter):
    _say(f"index_full_append fmt={fmt} scatter={scatter}")
    q, w, kk, starts, qpos, max_ctx = _indexer(gpu, [40000, 9, 70001, 513], 16, 128, seed=81 + fmt)
    n_new, cap = 37, 4096
    x = normal_bf16(82, "kv", fmt, (n_new, 512), outliers=True).to(gpu)
    dst = None
    if scatter:   # includes rows outside the cache, which are skipped
        perm = torch.randperm(cap, generator=torch.Generator().manual_seed(fmt))[:n_new].to(torch.int64)
        perm[3], perm[11] = -1, cap + 5
        dst = perm.to(gpu)
    ref_c, ref_s = _cache(fk, gpu, fmt, cap)
    fk.fp4kv_kv_append(fmt, x, ref_c, ref_s, dst_rows=dst, dst_start=100)
    ref = fk.fp4kv_index_full(q, w, kk, starts, qpos, 1, max_ctx, 2048, 512)
    got_c, got_s = _cache(fk, gpu, fmt, cap)
    got = fk.fp4kv_index_full_append(q, w, kk, starts, qpos, 1, max_ctx, 2048, 512, x, got_c, got_s, dst_rows=dst,
                                     dst_start=100, kv_fmt=fmt)
    torch.cuda.synchronize()
    for name, a, b in zip(("pool", "n_pool", "idx", "n_idx"), ref, got):
        assert torch.equal(a, b), name
    assert torch.equal(ref_c, got_c)
    if ref_s is not None:
        assert torch.equal(ref_s, got_s)
    if fmt == 0:                 # and the FP4 bytes are the oracle's codec
        oc, os_ = fp4.quantize_rows(bf16_to_f64(x.cpu()))
        rows = np.arange(100, 100 + n_new) if dst is None else dst.cpu().numpy()
        for i, r in enumerate(rows):
            if 0 <= r < cap:
                assert np.array_equal(got_c[r].cpu().numpy(), oc[i]) and np.array_equal(got_s[r].cpu().numpy(), os_[i])


def test_index_scores_append_and_empty_append(fk, gpu):
    _say("index_scores_append: scores bit-equal; zero appended rows")
    q, w, kk, starts, qpos, max_ctx = _indexer(gpu, [5000, 20000, 1], 8, 64, seed=85)
    x = normal_bf16(86, "kv", 0, (1000, 512), outliers=True).to(gpu)
    ref_c, ref_s = _cache(fk, gpu, 0, 1000)
    fk.fp4kv_quantize_append(x, ref_c, ref_s)
    rs, rb = fk.fp4kv_index_scores(q, w, kk, starts, qpos, 1, max_ctx)
    got_c, got_s = _cache(fk, gpu, 0, 1000)
    gs, gb = fk.fp4kv_index_scores_append(q, w, kk, starts, qpos, 1, max_ctx, x, got_c, got_s)
    torch.cuda.synchronize()
    L = [5000, 20000, 1]
    for i, n in enumerate(L):
        assert torch.equal(rs[i, :n], gs[i, :n])
        assert torch.equal(rb[i, :(n + 7) // 8], gb[i, :(n + 7) // 8])
    assert torch.equal(ref_c, got_c) and torch.equal(ref_s, got_s)
    # an empty append leaves the cache as it was
    before = got_c.clone()
    fk.fp4kv_index_scores_append(q, w, kk, starts, qpos, 1, max_ctx, x[:0], got_c, got_s)
    torch.cuda.synchronize()
    assert torch.equal(before, got_c)


def test_index_full_append_matrix_core_scan(fk, gpu):
    _say("index_full_append with many queries per sequence")
    L = 6000
    q, w, kk, starts, qpos, max_ctx = _indexer(gpu, [L], 16, 128, seed=87, positions=list(range(L - 64, L)))
    x = normal_bf16(88, "kv", 0, (64, 512), outliers=True).to(gpu)
    ref_c, ref_s = _cache(fk, gpu, 0, 8192)
    fk.fp4kv_quantize_append(x, ref_c, ref_s, dst_start=L - 64)
    ref = fk.fp4kv_index_full(q, w, kk, starts, qpos, 64, max_ctx, 256, 128)
    got_c, got_s = _cache(fk, gpu, 0, 8192)
    got = fk.fp4kv_index_full_append(q, w, kk, starts, qpos, 64, max_ctx, 256, 128, x, got_c, got_s,
                                     dst_start=L - 64)
    torch.cuda.synchronize()
    for name, a, b in zip(("pool", "n_pool", "idx", "n_idx"), ref, got):
        assert torch.equal(a, b), name
    assert torch.equal(ref_c, got_c) and torch.equal(ref_s, got_s)


@pytest.mark.parametrize("fmt", [0, 2])
def test_index_scores_append_single_query_grid(fk, gpu, fmt):
    """One query: the scan takes its 2-D grid (no work list) with the append rows as
    a second grid row."""
    _say(f"index_scores_append: one query, 2-D grid, fmt={fmt}")
    q, w, kk, starts, qpos, max_ctx = _indexer(gpu, [50001], 16, 128, seed=89 + fmt)
    x = normal_bf16(90, "kv", fmt, (300, 512), outliers=True).to(gpu)
    ref_c, ref_s = _cache(fk, gpu, fmt, 2000)
    fk.fp4kv_kv_append(fmt, x, ref_c, ref_s, dst_start=1700)
    rs, rb = fk.fp4kv_index_scores(q, w, kk, starts, qpos, 1, max_ctx)
    got_c, got_s = _cache(fk, gpu, fmt, 2000)
    gs, gb = fk.fp4kv_index_scores_append(q, w, kk, starts, qpos, 1, max_ctx, x, got_c, got_s, dst_start=1700,
                                          kv_fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(rs[0, :50001], gs[0, :50001])
    assert torch.equal(rb[0, :(50001 + 7) // 8], gb[0, :(50001 + 7) // 8])
    assert torch.equal(ref_c, got_c)
    if ref_s is not None:
        assert torch.equal(ref_s, got_s)
