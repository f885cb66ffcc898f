"""GPU parity of the main-KV format variants through the C ABI: MXFP4 (E2M1 +
E8M0 per 32 channels) and FP8 (E4M3FN per channel), with the FP4 cache run
through the same format-generic entry points.

Appended code and scale bytes must equal the oracle's bit for bit; attention
must satisfy max|out - ref| <= 2e-4 * max|ref| + 1e-6 against the oracle on the
rows the cache in that format holds.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, kvformats
from synth import bf16_to_f64, normal_bf16
from synth import workloads as wl
from tests import oracle_runner as orun
from tests.oracle_runner import within_tolerance

pytestmark = pytest.mark.gpu

FORMATS = [kvformats.FMT_FP4, kvformats.FMT_MXFP4, kvformats.FMT_FP8]
NAMES = {kvformats.FMT_FP4: "fp4", kvformats.FMT_MXFP4: "mxfp4", kvformats.FMT_FP8: "fp8"}


@pytest.fixture(scope="module")
def fk():
    import sparse_indexer_fp4_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _say(msg):
    print(msg, flush=True)


def _cache(fk, fmt, rows, C, gpu):
    codes = torch.zeros((rows, fk.fp4kv_kv_code_bytes(fmt, C)), dtype=torch.uint8, device=gpu)
    sb = fk.fp4kv_kv_scale_bytes(fmt, C)
    scales = torch.zeros((rows, sb), dtype=torch.uint8, device=gpu) if sb > 0 else None
    return codes, scales


def _oracle_bytes(fmt, x):
    codes, scales = kvformats.quantize_rows(fmt, bf16_to_f64(x))
    return codes, scales


def _check_append(fk, fmt, x, gpu):
    R, C = x.shape
    codes, scales = _cache(fk, fmt, R, C, gpu)
    fk.fp4kv_kv_append(fmt, x.to(gpu), codes, scales)
    rc, rs = _oracle_bytes(fmt, x)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, (NAMES[fmt], bad[:4], got[tuple(bad[0])], rc[tuple(bad[0])])
    if scales is not None:
        assert np.array_equal(scales.cpu().numpy(), rs), NAMES[fmt]
    # scattered destinations: the same rows written in reverse order
    codes2, scales2 = _cache(fk, fmt, R + 3, C, gpu)
    dst = torch.arange(R + 2, 2, -1, dtype=torch.int64, device=gpu)
    fk.fp4kv_kv_append(fmt, x.to(gpu), codes2, scales2, dst_rows=dst)
    assert np.array_equal(codes2.cpu().numpy()[np.arange(R + 2, 2, -1)], rc)
    if scales2 is not None:
        assert np.array_equal(scales2.cpu().numpy()[np.arange(R + 2, 2, -1)], rs)


def test_fp8_append_all_bf16_values(fk, gpu):
    """Every finite bf16 value of either sign, plus normal rows with outliers."""
    _say("kv append fp8: all bf16 values")
    pos = np.arange(0x7F80, dtype=np.uint32)
    bits = np.concatenate([pos, pos | 0x8000, np.zeros(65536 - 2 * 0x7F80, dtype=np.uint32)])
    x = torch.from_numpy((bits << 16).view(np.float32)).to(torch.bfloat16).reshape(128, 512)
    x = torch.cat([x, normal_bf16(41, "kv", 0, (64, 512), outliers=True)])
    _check_append(fk, kvformats.FMT_FP8, x, gpu)


def test_mxfp4_append_every_block_scale(fk, gpu):
    """One 32-value block per positive finite bf16 amax (its first value; the rest
    random below it), plus tie-heavy, saturating, subnormal, zero and huge blocks."""
    _say("kv append mxfp4: every amax")
    rng = np.random.default_rng(5)
    amax = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    amax = np.concatenate([amax, np.zeros(16 - amax.size % 16)])           # whole rows of 16 blocks
    blocks = amax[:, None] * rng.uniform(-1.0, 1.0, (amax.size, 32))
    blocks[:, 0] = amax * rng.choice([-1.0, 1.0], amax.size)
    x = torch.from_numpy(blocks.reshape(-1, 512)).to(torch.bfloat16)       # |x| <= amax survives rounding
    special = []
    for e in (-130, -20, 0, 7, 120):
        g = rng.choice([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 7.5], (16, 32)) * 2.0 ** e
        special.append(g * rng.choice([-1.0, 1.0], g.shape))
    special.append(np.zeros((16, 32)))
    x = torch.cat([x, torch.from_numpy(np.concatenate(special).reshape(-1, 512)).to(torch.bfloat16),
                   normal_bf16(43, "kv", 0, (64, 512), outliers=True)])
    _check_append(fk, kvformats.FMT_MXFP4, x, gpu)


def _decode_case(fk, gpu, fmt, lengths, n_idx, Hq, k, W, seed):
    B = len(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(np.sum(lengths))
    x = normal_bf16(seed, "kv", 0, (max(total, 1), 512), outliers=True)
    codes, scales = _cache(fk, fmt, max(total, 1), 512, gpu)
    fk.fp4kv_kv_append(fmt, x.to(gpu), codes, scales)
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
    out, lse = fk.fp4kv_sparse_attn_decode_kv(fmt, q.to(gpu), codes, scales, torch.from_numpy(starts).to(gpu),
                                              torch.from_numpy(idx).to(gpu), torch.from_numpy(nidx).to(gpu),
                                              wk.to(gpu), wv.to(gpu), torch.from_numpy(qpos).to(gpu), scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ref_rows = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, bf16_to_f64(x)))
    for b in range(B):
        rows = ref_rows[starts[b] + idx[b, :nidx[b]]]
        nw = min(W, int(qpos[b]) + 1)
        ro, rl = attention.attend(bf16_to_f64(q[b]), rows, bf16_to_f64(wk[b, W - nw:]), bf16_to_f64(wv[b, W - nw:]),
                                  scale)
        ok, err, tol = within_tolerance(out[b], ro)
        assert ok, (NAMES[fmt], b, err, tol)
        ok, err, tol = within_tolerance(lse[b], rl)
        assert ok, (NAMES[fmt], "lse", b, err, tol)


@pytest.mark.parametrize("fmt", FORMATS, ids=[NAMES[f] for f in FORMATS])
@pytest.mark.parametrize("lengths,n_idx,Hq,k,W", [
    ([4096], [128], 16, 128, 128),
    ([5000, 300, 70, 1], [512, 300, 17, 1], 64, 512, 128),
    ([2000, 0, 40], [100, 0, 40], 32, 512, 100),
])
def test_decode_attention_formats(fk, gpu, fmt, lengths, n_idx, Hq, k, W):
    _say(f"kv decode attention {NAMES[fmt]} lengths={lengths} Hq={Hq}")
    _decode_case(fk, gpu, fmt, lengths, n_idx, Hq, k, W, seed=sum(lengths) % 997 + fmt)


@pytest.mark.parametrize("fmt", FORMATS, ids=[NAMES[f] for f in FORMATS])
def test_prefill_attention_formats(fk, gpu, fmt):
    _say(f"kv prefill attention {NAMES[fmt]}")
    L, T, W, Hq, k = 3000, 40, 128, 64, 256
    pos0 = 90
    x = normal_bf16(13, "kv", 0, (L, 512), outliers=True)
    codes, scales = _cache(fk, fmt, L, 512, gpu)
    fk.fp4kv_kv_append(fmt, x.to(gpu), codes, scales)
    rng = np.random.default_rng(13)
    idx = np.full((T, k), -1, dtype=np.int32)
    nidx = np.zeros(T, dtype=np.int32)
    for i in range(T):
        m = min(k, pos0 + i + 1)
        idx[i, :m] = np.sort(rng.choice(pos0 + i + 1, size=m, replace=False))
        nidx[i] = m
    q = normal_bf16(13, "q", 0, (T, Hq, 512), outliers=False)
    wbuf_k = normal_bf16(13, "wk", 0, (T + W - 1, 512), outliers=False)
    wbuf_v = normal_bf16(13, "wv", 0, (T + W - 1, 512), outliers=False)
    scale = 1.0 / math.sqrt(512)
    out, _ = fk.fp4kv_sparse_attn_prefill_kv(fmt, q.to(gpu), codes, scales, 0, torch.from_numpy(idx).to(gpu),
                                             torch.from_numpy(nidx).to(gpu), wbuf_k.to(gpu), wbuf_v.to(gpu),
                                             pos0, W, scale)
    out = out.cpu().numpy()
    ref_rows = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, bf16_to_f64(x)))
    for i in range(T):
        nw = min(W, pos0 + i + 1)
        r0 = i + W - nw
        ro, _ = attention.attend(bf16_to_f64(q[i]), ref_rows[idx[i, :nidx[i]]], bf16_to_f64(wbuf_k[r0:i + W]),
                                 bf16_to_f64(wbuf_v[r0:i + W]), scale)
        ok, err, tol = within_tolerance(out[i], ro)
        assert ok, (NAMES[fmt], i, err, tol)


@pytest.mark.parametrize("fmt", [kvformats.FMT_MXFP4, kvformats.FMT_FP8], ids=["mxfp4", "fp8"])
def test_decode128k_formats(fk, gpu, fmt):
    """decode128k with its main-KV cache in format fmt, in the benchmark's launch
    configuration: sampled queries against the oracle on that format's rows. Also
    prints each format's distance from attention over the unquantised rows."""
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS["decode128k"]
    _say(f"decode128k {NAMES[fmt]}: setup")
    dw = DeviceWorkload(cfg, gpu, build_kv=False)
    codes, scales = _cache(fk, fmt, dw.total_rows, cfg.C, gpu)
    starts = cfg.seq_starts()
    for s in range(cfg.n_seq):
        for a, b in wl.chunks(int(dw.lengths[s]), 1 << 18):
            fk.fp4kv_kv_append(fmt, wl.kv_rows_into(cfg, s, a, b, gpu), codes, scales, dst_start=int(starts[s]) + a)
    pool, n_pool, idx, n_idx = fk.fp4kv_index_full(dw.idx_q[0], dw.w[0], dw.idx_k, dw.seq_start, dw.q_pos, 1,
                                                   cfg.ctx, cfg.P, cfg.k)
    out, lse = fk.fp4kv_sparse_attn_decode_kv(fmt, dw.q[0], codes, scales, dw.seq_start, idx, n_idx, dw.swa_k[0],
                                              dw.swa_v[0], dw.q_pos, cfg.scale)
    torch.cuda.synchronize()
    _say(f"decode128k {NAMES[fmt]}: checking")
    idx, n_idx, out, lse = idx.cpu().numpy(), n_idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    for i in (0, 31):
        ri = idx[i, :n_idx[i]]
        ro, rl = orun.attend(cfg, i, 0, ri, fmt)
        ok, err, tol = within_tolerance(out[i], ro)
        assert ok, (NAMES[fmt], i, err, tol)
        ok, err, tol = within_tolerance(lse[i], rl)
        assert ok, (NAMES[fmt], "lse", i, err, tol)
        exact, _ = orun.attend(cfg, i, 0, ri, None)
        rel = np.abs(out[i] - exact).max() / np.abs(exact).max()
        _say(f"decode128k {NAMES[fmt]} query {i}: max|out - attention on bf16 rows| / max|.| = {rel:.3e}")
