"""GPU parity on the five workloads at full size, in the launch configuration
the benchmark uses. The whole batch runs on the GPU; sampled queries are
recomputed one by one by the oracle from host-regenerated inputs. Pools,
indices and FP4 bytes are bit-exact; attention within
max|out - ref| <= 2e-4 * max|ref| + 1e-6 per (query, layer) output.
"""
import numpy as np
import pytest
import torch

from oracle import fp4
from synth import bf16_to_f64
from synth import workloads as wl
from tests import oracle_runner as orun

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_indexer_fp4_amd as m
    return m


def _say(msg):
    print(msg, flush=True)


def _check_index(i, pool, n_pool, idx, n_idx, rp, ri):
    assert int(n_pool[i]) == len(rp), (i, int(n_pool[i]), len(rp))
    assert np.array_equal(pool[i, :len(rp)], rp), i
    assert (pool[i, len(rp):] == -1).all(), i
    assert int(n_idx[i]) == len(ri), (i, int(n_idx[i]), len(ri))
    assert np.array_equal(idx[i, :len(ri)], ri), i
    assert (idx[i, len(ri):] == -1).all(), i


def _check_attn(cfg, i, layer, out, lse, ri):
    ro, rl = orun.attend(cfg, i, layer, ri)
    ok, err, tol = orun.within_tolerance(out[i], ro)
    assert ok, ("out", i, layer, err, tol)
    ok, err, tol = orun.within_tolerance(lse[i], rl)
    assert ok, ("lse", i, layer, err, tol)


def _check_cache_rows(cfg, dw, n_sample=2048, seed=0):
    """Sampled FP4 cache rows equal the oracle's quantisation of the same bf16 rows."""
    rng = np.random.default_rng(seed)
    starts, lens = cfg.seq_starts(), cfg.seq_lengths()
    s = rng.integers(0, cfg.n_seq, n_sample)
    t = (rng.random(n_sample) * lens[s]).astype(np.int64)
    for si in np.unique(s):
        sel = t[s == si]
        x = bf16_to_f64(wl.kv_rows(cfg, int(si), torch.from_numpy(sel)))
        rc, rs = fp4.quantize_rows(x)
        rows = torch.from_numpy(starts[si] + sel).to(dw.codes.device)
        gc = dw.codes[rows].cpu().numpy()
        gs = dw.scales[rows].cpu().numpy()
        assert np.array_equal(gc, rc) and np.array_equal(gs, rs), int(si)


def test_tiny(fk, gpu):
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["tiny"]
    _say("tiny: setup")
    dw = DeviceWorkload(cfg, gpu)
    pool, n_pool, idx, n_idx = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1,
                                                   cfg.ctx, cfg.P, cfg.k)
    out, lse = fk.fp4kv_sparse_attn_decode(dw.q[0], dw.codes, dw.scales, dw.seq_start, idx, n_idx, dw.swa_k[0],
                                           dw.swa_v[0], dw.q_pos, cfg.scale)
    torch.cuda.synchronize()
    _check_cache_rows(cfg, dw, 4096)
    rp, ri, _ = orun.full_layer(cfg, 0)
    _check_index(0, pool.cpu().numpy(), n_pool.cpu().numpy(), idx.cpu().numpy(), n_idx.cpu().numpy(), rp, ri)
    _check_attn(cfg, 0, 0, out.cpu().numpy(), lse.cpu().numpy(), ri)


def test_decode128k(fk, gpu):
    """The benchmark's workload and launch sequence (scores with the append in
    their launch, select, attention); every query against the oracle."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["decode128k"]
    _say("decode128k: setup")
    dw = DeviceWorkload(cfg, gpu)
    new_x, new_dst = dw.newest_rows()
    scores, blockmax = fk.fp4kv_index_scores_append(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1,
                                                    cfg.ctx, new_x, dw.codes, dw.scales, dst_rows=new_dst)
    pool, n_pool, idx, n_idx = fk.fp4kv_index_select(scores, blockmax, dw.total_rows, dw.seq_start, dw.q_pos, 1,
                                                     cfg.P, cfg.k)
    out, lse = fk.fp4kv_sparse_attn_decode(dw.q[0], dw.codes, dw.scales, dw.seq_start, idx, n_idx, dw.swa_k[0],
                                           dw.swa_v[0], dw.q_pos, cfg.scale)
    torch.cuda.synchronize()
    _say("decode128k: checking all 32 queries")
    _check_cache_rows(cfg, dw)
    pool, n_pool, idx, n_idx = (t.cpu().numpy() for t in (pool, n_pool, idx, n_idx))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(cfg.n_seq):
        rp, ri, s = orun.full_layer(cfg, i)
        _check_index(i, pool, n_pool, idx, n_idx, rp, ri)
        assert np.array_equal(scores[i].cpu().numpy().astype(np.float64), s), i
        _check_attn(cfg, i, 0, out, lse, ri)
    # the same through the single-call entry points
    pool2, _, idx2, _ = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1, cfg.ctx,
                                           cfg.P, cfg.k)
    assert np.array_equal(pool2.cpu().numpy(), pool) and np.array_equal(idx2.cpu().numpy(), idx)
    pool3, _, idx3, _ = fk.fp4kv_index_full_append(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1,
                                                   cfg.ctx, cfg.P, cfg.k, new_x, dw.codes, dw.scales,
                                                   dst_rows=new_dst)
    assert np.array_equal(pool3.cpu().numpy(), pool) and np.array_equal(idx3.cpu().numpy(), idx)


def test_chain1m(fk, gpu):
    """Full -> Reuse x3, then Reindex -> Reuse x3, at 1M context."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["chain1m"]
    _say("chain1m: setup")
    dw = DeviceWorkload(cfg, gpu)
    outs = {}
    pool, n_pool, idx, n_idx = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1,
                                                   cfg.ctx, cfg.P, cfg.k)
    cur = (idx, n_idx)
    layer_idx = {}
    for layer, mode in enumerate(cfg.modes):
        if mode == "reindex":
            cur = fk.fp4kv_index_reindex(dw.idx_q[layer], dw.w[layer], dw.idx_k, dw.seq_start, dw.q_pos, 1, pool,
                                         n_pool, cfg.k)
        layer_idx[layer] = cur
        outs[layer] = fk.fp4kv_sparse_attn_decode(dw.q[layer], dw.codes, dw.scales, dw.seq_start, cur[0], cur[1],
                                                  dw.swa_k[layer], dw.swa_v[layer], dw.q_pos, cfg.scale)
    torch.cuda.synchronize()
    _say("chain1m: checking")
    _check_cache_rows(cfg, dw, 1024)
    pool_h, n_pool_h = pool.cpu().numpy(), n_pool.cpu().numpy()
    for i in range(cfg.n_seq):
        rp, ri, _ = orun.full_layer(cfg, i)
        _check_index(i, pool_h, n_pool_h, idx.cpu().numpy(), n_idx.cpu().numpy(), rp, ri)
        rri = orun.reindex_layer(cfg, i, 4, rp)
        for layer, mode in enumerate(cfg.modes):
            want = ri if layer < 4 else rri
            got_idx, got_n = (t.cpu().numpy() for t in layer_idx[layer])
            assert int(got_n[i]) == len(want) and np.array_equal(got_idx[i, :len(want)], want), (i, layer)
            o, l = (t.cpu().numpy() for t in outs[layer])
            _check_attn(cfg, i, layer, o, l, want)


def test_prefill(fk, gpu):
    """4,096 causal queries at positions 127,000..131,095 of one 131,096-token context."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["prefill"]
    _say("prefill: setup")
    dw = DeviceWorkload(cfg, gpu)
    pool, n_pool, idx, n_idx = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.q_seq_start, dw.q_pos,
                                                   cfg.T, cfg.ctx, cfg.P, cfg.k)
    out, lse = fk.fp4kv_sparse_attn_prefill(dw.q[0], dw.codes, dw.scales, 0, idx, n_idx, dw.swa_k[0], dw.swa_v[0],
                                            cfg.pos0, cfg.W, cfg.scale)
    torch.cuda.synchronize()
    _say("prefill: checking")
    pool, n_pool, idx, n_idx = (t.cpu().numpy() for t in (pool, n_pool, idx, n_idx))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    k_rows = orun.host_idx_k(cfg, 0, cfg.ctx)
    # every in-block offset of the first and the last 32-query block of the
    # matrix-core scan, and one query in the middle
    for i in list(range(32)) + [2048] + list(range(cfg.T - 32, cfg.T)):
        rp, ri, _ = orun.full_layer(cfg, i, k_rows=k_rows)
        _check_index(i, pool, n_pool, idx, n_idx, rp, ri)
        _check_attn(cfg, i, 0, out, lse, ri)


def test_mixed(fk, gpu):
    """Quantize-append of 65,536 rows (1,024 per sequence, 0.1% zero groups),
    then a Full-layer decode of 64 queries with log-uniform 4K..1M contexts."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["mixed"]
    _say("mixed: setup")
    dw = DeviceWorkload(cfg, gpu)
    x, dst = dw.appended_rows()
    max_ctx = int(cfg.seq_lengths().max())
    # the 65,536-row append rides in the indexer scan's launch, as in the benchmark
    pool, n_pool, idx, n_idx = fk.fp4kv_index_full_append(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos,
                                                          1, max_ctx, cfg.P, cfg.k, x, dw.codes, dw.scales,
                                                          dst_rows=dst)
    out, lse = fk.fp4kv_sparse_attn_decode(dw.q[0], dw.codes, dw.scales, dw.seq_start, idx, n_idx, dw.swa_k[0],
                                           dw.swa_v[0], dw.q_pos, cfg.scale)
    torch.cuda.synchronize()
    _say("mixed: checking appended rows")
    xc = bf16_to_f64(x.cpu())
    rc, rs = fp4.quantize_rows(xc)
    dst_h = dst.cpu()
    assert np.array_equal(dw.codes[dst_h.to(gpu)].cpu().numpy(), rc)
    assert np.array_equal(dw.scales[dst_h.to(gpu)].cpu().numpy(), rs)
    assert (rs == 0).sum() > 0                      # the zero-scale path was exercised
    _check_cache_rows(cfg, dw, 1024)
    _say("mixed: checking queries")
    L = cfg.seq_lengths()
    pool, n_pool, idx, n_idx = (t.cpu().numpy() for t in (pool, n_pool, idx, n_idx))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in sorted({int(np.argmin(L)), int(np.argmax(L))} | set(range(0, 64, 5))):
        rp, ri, _ = orun.full_layer(cfg, i)
        _check_index(i, pool, n_pool, idx, n_idx, rp, ri)
        _check_attn(cfg, i, 0, out, lse, ri)


def test_prefill_matrix_core_scan_equals_per_query_scan(fk, gpu):
    """At full prefill size, the matrix-core scan (32 queries per key tile) and
    the per-query scan give the same scores and block maxima, bit for bit, for
    all 4,096 queries."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["prefill"]
    _say("prefill: matrix-core scan vs per-query scan, all queries")
    dw = DeviceWorkload(cfg, gpu, build_kv=False)
    s_mfma, b_mfma = fk.fp4kv_index_scores(dw.idx_q[0], dw.w[0], dw.idx_k, dw.q_seq_start, dw.q_pos, cfg.T, cfg.ctx)
    starts = dw.q_seq_start.repeat(cfg.T)           # one "sequence" per query: the per-query scan
    s_one, b_one = fk.fp4kv_index_scores(dw.idx_q[0], dw.w[0], dw.idx_k, starts, dw.q_pos, 1, cfg.ctx)
    torch.cuda.synchronize()
    vis = (dw.q_pos.to(torch.int64) + 1)
    cols = torch.arange(cfg.ctx, device=gpu)
    mask = cols[None, :] < vis[:, None]
    assert torch.equal(torch.where(mask, s_mfma, 0.0), torch.where(mask, s_one, 0.0))
    bmask = torch.arange(b_mfma.shape[1], device=gpu)[None, :] < ((vis + 7) // 8)[:, None]
    assert torch.equal(torch.where(bmask, b_mfma, 0.0), torch.where(bmask, b_one, 0.0))
