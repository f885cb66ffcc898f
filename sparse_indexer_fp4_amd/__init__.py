"""Python binding of libfp4kv (include/fp4kv.h): argument marshalling only.

Every function takes torch tensors on the GPU, passes their device pointers and
the current HIP stream to the C ABI, and raises Fp4kvError on a negative
status. Nothing here computes any part of the method; all of it runs in the
HIP kernels of libfp4kv.so. The library must have been built
(python sparse_indexer_fp4_amd/build.py); importing this package without it
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4kv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_indexer_fp4_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

_SIGS = {
    "fp4kv_abi_version": (_i32, []),
    "fp4kv_last_error": (ctypes.c_char_p, []),
    "fp4kv_quantize_append": (_i32, [_p, _i64, _i32, _p, _i64, _p, _p, _i64, _p]),
    "fp4kv_index_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "fp4kv_index_full": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                _p, _p, _p, _p, _p, _sz, _p]),
    "fp4kv_index_scores": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _p, _p, _p]),
    "fp4kv_index_select": (_i32, [_p, _p, _i64, _p, _p, _i32, _i32, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "fp4kv_reindex_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fp4kv_index_reindex": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _i32, _i32, _i32,
                                   _p, _p, _p, _sz, _p]),
    "fp4kv_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "fp4kv_sparse_attn_decode": (_i32, [_p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                        _f32, _p, _p, _p, _sz, _p]),
    "fp4kv_sparse_attn_prefill": (_i32, [_p, _p, _p, _i64, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _f32, _p, _p, _p, _sz, _p]),
    "fp4kv_kv_code_bytes": (_i64, [_i32, _i32]),
    "fp4kv_kv_scale_bytes": (_i64, [_i32, _i32]),
    "fp4kv_kv_append": (_i32, [_i32, _p, _i64, _i32, _p, _i64, _p, _p, _i64, _p]),
    "fp4kv_sparse_attn_decode_kv": (_i32, [_i32, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                           _i32, _f32, _p, _p, _p, _sz, _p]),
    "fp4kv_sparse_attn_prefill_kv": (_i32, [_i32, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _p, _p, _p, _sz, _p]),
    "fp4kv_paged_kv_append": (_i32, [_i32, _p, _p, _i64, _i32, _i32, _p, _p, _p, _i32, _i32, _i32, _i64, _p, _p, _p,
                                     _p]),
    "fp4kv_swa_ring_append": (_i32, [_p, _p, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p]),
    "fp4kv_index_full_paged": (_i32, [_p, _p, _p, _p, _i32, _i32, _i32, _i64, _p, _i32, _i32, _i32, _i32, _i64, _i32,
                                      _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "fp4kv_index_reindex_paged": (_i32, [_p, _p, _p, _p, _i32, _i32, _i32, _i64, _p, _i32, _i32, _i32, _i32, _p, _p,
                                         _i32, _i32, _i32, _p, _p, _p, _sz, _p]),
    "fp4kv_sparse_attn_decode_paged": (_i32, [_i32, _p, _p, _p, _p, _i32, _i32, _i64, _p, _p, _p, _p, _p, _i32, _i32,
                                              _i32, _i32, _i32, _f32, _p, _p, _p, _sz, _p]),
}

# Main-KV formats (FP4KV_KV_* in the header).
KV_FP4, KV_MXFP4, KV_FP8 = 0, 1, 2
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


class Fp4kvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fp4kv status {status}: {message}")
        self.status = status


def _check(status: int):
    if status != 0:
        raise Fp4kvError(status, lib.fp4kv_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp4kv arguments must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("fp4kv arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _expect(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def abi_version() -> int:
    return lib.fp4kv_abi_version()


def fp4kv_quantize_append(src, codes, scales, dst_rows=None, dst_start=0, stream=None):
    """FP4 quantize-append of bf16 rows src [n, C] into (codes [cap, C/2], scales [cap, C/16])."""
    _expect(src, torch.bfloat16, "src"); _expect(codes, torch.uint8, "codes"); _expect(scales, torch.uint8, "scales")
    if dst_rows is not None:
        _expect(dst_rows, torch.int64, "dst_rows")
    n, C = src.shape
    _check(lib.fp4kv_quantize_append(_ptr(src), n, C, _ptr(dst_rows), dst_start, _ptr(codes), _ptr(scales),
                                     codes.shape[0], _stream(stream)))


def fp4kv_index_workspace_bytes(n_q, max_ctx, block=8):
    return lib.fp4kv_index_workspace_bytes(n_q, max_ctx, block)


def fp4kv_reindex_workspace_bytes(n_q, P, block=8):
    return lib.fp4kv_reindex_workspace_bytes(n_q, P, block)


def fp4kv_attn_workspace_bytes(n_q, Hq, C, k, W):
    return lib.fp4kv_attn_workspace_bytes(n_q, Hq, C, k, W)


def _workspace(nbytes, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _expect(workspace, torch.uint8, "workspace")
    return workspace


def fp4kv_index_full(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, P, k, block=8,
                     pool_out=None, n_pool=None, idx_out=None, n_idx=None, workspace=None, stream=None):
    """Full-mode indexer. idx_q bf16 [n_q, H, D], w f32 [n_q, H], idx_k bf16 [rows, D],
    seq_start i64 [n_seq], q_pos i32 [n_q]. Returns (pool [n_q, P], n_pool, idx [n_q, k], n_idx)."""
    _expect(idx_q, torch.bfloat16, "idx_q"); _expect(w, torch.float32, "w"); _expect(idx_k, torch.bfloat16, "idx_k")
    _expect(seq_start, torch.int64, "seq_start"); _expect(q_pos, torch.int32, "q_pos")
    n_q, H, D = idx_q.shape
    dev = idx_q.device
    pool_out = torch.empty((n_q, P), dtype=torch.int32, device=dev) if pool_out is None else pool_out
    n_pool = torch.empty((n_q,), dtype=torch.int32, device=dev) if n_pool is None else n_pool
    idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    n_idx = torch.empty((n_q,), dtype=torch.int32, device=dev) if n_idx is None else n_idx
    ws = _workspace(fp4kv_index_workspace_bytes(n_q, max_ctx, block), dev, workspace)
    _check(lib.fp4kv_index_full(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                n_q, q_per_seq, H, D, max_ctx, block, P, k, _ptr(pool_out), _ptr(n_pool),
                                _ptr(idx_out), _ptr(n_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def fp4kv_index_scores(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, block=8, scores=None, blockmax=None,
                       stream=None):
    """Scan half of the Full indexer. Returns (scores f32 [n_q, max_ctx], blockmax f32 [n_q, nblk])."""
    _expect(idx_q, torch.bfloat16, "idx_q"); _expect(w, torch.float32, "w"); _expect(idx_k, torch.bfloat16, "idx_k")
    n_q, H, D = idx_q.shape
    dev = idx_q.device
    nblk = (max_ctx + block - 1) // block
    scores = torch.empty((n_q, max_ctx), dtype=torch.float32, device=dev) if scores is None else scores
    blockmax = torch.empty((n_q, nblk), dtype=torch.float32, device=dev) if blockmax is None else blockmax
    _check(lib.fp4kv_index_scores(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                  n_q, q_per_seq, H, D, max_ctx, block, _ptr(scores), _ptr(blockmax),
                                  _stream(stream)))
    return scores, blockmax


def fp4kv_index_select(scores, blockmax, total_rows, seq_start, q_pos, q_per_seq, P, k, block=8, pool_out=None,
                       n_pool=None, idx_out=None, n_idx=None, stream=None):
    """Selection half of the Full indexer. Returns (pool, n_pool, idx, n_idx)."""
    _expect(scores, torch.float32, "scores"); _expect(blockmax, torch.float32, "blockmax")
    n_q, max_ctx = scores.shape
    dev = scores.device
    pool_out = torch.empty((n_q, P), dtype=torch.int32, device=dev) if pool_out is None else pool_out
    n_pool = torch.empty((n_q,), dtype=torch.int32, device=dev) if n_pool is None else n_pool
    idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    n_idx = torch.empty((n_q,), dtype=torch.int32, device=dev) if n_idx is None else n_idx
    _check(lib.fp4kv_index_select(_ptr(scores), _ptr(blockmax), int(total_rows), _ptr(seq_start), _ptr(q_pos), n_q,
                                  q_per_seq, max_ctx, block, P, k, _ptr(pool_out), _ptr(n_pool), _ptr(idx_out),
                                  _ptr(n_idx), _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def fp4kv_index_reindex(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, pool, n_pool, k, block=8,
                        idx_out=None, n_idx=None, workspace=None, stream=None):
    """Reindex-mode indexer over an inherited pool [n_q, P]. Returns (idx [n_q, k], n_idx)."""
    _expect(idx_q, torch.bfloat16, "idx_q"); _expect(w, torch.float32, "w"); _expect(idx_k, torch.bfloat16, "idx_k")
    _expect(pool, torch.int32, "pool"); _expect(n_pool, torch.int32, "n_pool")
    n_q, H, D = idx_q.shape
    P = pool.shape[1]
    dev = idx_q.device
    idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    n_idx = torch.empty((n_q,), dtype=torch.int32, device=dev) if n_idx is None else n_idx
    ws = _workspace(fp4kv_reindex_workspace_bytes(n_q, P, block), dev, workspace)
    _check(lib.fp4kv_index_reindex(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                   n_q, q_per_seq, H, D, _ptr(pool), _ptr(n_pool), block, P, k, _ptr(idx_out),
                                   _ptr(n_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return idx_out, n_idx


def fp4kv_sparse_attn_decode(q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, q_pos, scale,
                             out=None, lse=None, workspace=None, stream=None):
    """Decode attention. q bf16 [B, Hq, C]; codes/scales the FP4 cache; idx i32 [B, k];
    swa_k/swa_v bf16 [B, W, C]. Returns (out f32 [B, Hq, C], lse f32 [B, Hq])."""
    _expect(q, torch.bfloat16, "q"); _expect(swa_k, torch.bfloat16, "swa_k"); _expect(swa_v, torch.bfloat16, "swa_v")
    _expect(idx, torch.int32, "idx"); _expect(n_idx, torch.int32, "n_idx")
    B, Hq, C = q.shape
    k = idx.shape[1]
    W = swa_k.shape[1]
    dev = q.device
    out = torch.empty((B, Hq, C), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace(fp4kv_attn_workspace_bytes(B, Hq, C, k, W), dev, workspace)
    _check(lib.fp4kv_sparse_attn_decode(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], _ptr(seq_start),
                                        _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), _ptr(q_pos), B, Hq, C, k, W,
                                        float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def fp4kv_sparse_attn_prefill(q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, pos0, W, scale,
                              out=None, lse=None, workspace=None, stream=None):
    """Prefill-chunk attention. q bf16 [T, Hq, C] at positions pos0..pos0+T-1; swa_k/swa_v
    bf16 [T+W-1, C] (row r = position pos0-W+1+r). Returns (out, lse)."""
    _expect(q, torch.bfloat16, "q"); _expect(swa_k, torch.bfloat16, "swa_k"); _expect(swa_v, torch.bfloat16, "swa_v")
    T, Hq, C = q.shape
    k = idx.shape[1]
    if swa_k.shape[0] != T + W - 1 or swa_v.shape[0] != T + W - 1:
        raise ValueError("swa_k/swa_v must hold T+W-1 rows")
    dev = q.device
    out = torch.empty((T, Hq, C), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace(fp4kv_attn_workspace_bytes(T, Hq, C, k, W), dev, workspace)
    _check(lib.fp4kv_sparse_attn_prefill(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], int(seq_start),
                                         _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), int(pos0), T, Hq, C, k, W,
                                         float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def fp4kv_kv_code_bytes(fmt, C):
    return lib.fp4kv_kv_code_bytes(fmt, C)


def fp4kv_kv_scale_bytes(fmt, C):
    return lib.fp4kv_kv_scale_bytes(fmt, C)


def fp4kv_kv_append(fmt, src, codes, scales, dst_rows=None, dst_start=0, stream=None):
    """Quantize-append of bf16 rows src [n, C] in format fmt into codes [cap, code bytes]
    and scales [cap, scale bytes] (scales may be None for KV_FP8)."""
    _expect(src, torch.bfloat16, "src"); _expect(codes, torch.uint8, "codes")
    if scales is not None:
        _expect(scales, torch.uint8, "scales")
    if dst_rows is not None:
        _expect(dst_rows, torch.int64, "dst_rows")
    n, C = src.shape
    _check(lib.fp4kv_kv_append(fmt, _ptr(src), n, C, _ptr(dst_rows), dst_start, _ptr(codes), _ptr(scales),
                               codes.shape[0], _stream(stream)))


def fp4kv_sparse_attn_decode_kv(fmt, q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, q_pos, scale,
                                out=None, lse=None, workspace=None, stream=None):
    """Decode attention over a cache in format fmt (scales may be None for KV_FP8)."""
    _expect(q, torch.bfloat16, "q"); _expect(swa_k, torch.bfloat16, "swa_k"); _expect(swa_v, torch.bfloat16, "swa_v")
    _expect(idx, torch.int32, "idx"); _expect(n_idx, torch.int32, "n_idx")
    B, Hq, C = q.shape
    k = idx.shape[1]
    W = swa_k.shape[1]
    dev = q.device
    out = torch.empty((B, Hq, C), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace(fp4kv_attn_workspace_bytes(B, Hq, C, k, W), dev, workspace)
    _check(lib.fp4kv_sparse_attn_decode_kv(fmt, _ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], _ptr(seq_start),
                                           _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), _ptr(q_pos), B, Hq, C, k,
                                           W, float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                           _stream(stream)))
    return out, lse


def fp4kv_sparse_attn_prefill_kv(fmt, q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, pos0, W, scale,
                                 out=None, lse=None, workspace=None, stream=None):
    """Prefill-chunk attention over a cache in format fmt (scales may be None for KV_FP8)."""
    _expect(q, torch.bfloat16, "q"); _expect(swa_k, torch.bfloat16, "swa_k"); _expect(swa_v, torch.bfloat16, "swa_v")
    T, Hq, C = q.shape
    k = idx.shape[1]
    if swa_k.shape[0] != T + W - 1 or swa_v.shape[0] != T + W - 1:
        raise ValueError("swa_k/swa_v must hold T+W-1 rows")
    dev = q.device
    out = torch.empty((T, Hq, C), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace(fp4kv_attn_workspace_bytes(T, Hq, C, k, W), dev, workspace)
    _check(lib.fp4kv_sparse_attn_prefill_kv(fmt, _ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], int(seq_start),
                                            _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), int(pos0), T, Hq, C, k,
                                            W, float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                            _stream(stream)))
    return out, lse


class PagedCache:
    """Device tensors of a paged cache: block_table int32 [n_seq, max_pages],
    codes/scales of n_pages*page_rows rows in format fmt, indexer keys idx_k
    [n_pages*page_rows, D] bf16. A plain holder; nothing is computed here."""

    def __init__(self, block_table, page_rows, n_pages, codes, scales, idx_k, fmt=KV_FP4):
        self.block_table, self.page_rows, self.n_pages = block_table, int(page_rows), int(n_pages)
        self.codes, self.scales, self.idx_k, self.fmt = codes, scales, idx_k, fmt

    @property
    def n_seq(self):
        return self.block_table.shape[0]

    @property
    def max_pages(self):
        return self.block_table.shape[1]


def fp4kv_paged_kv_append(cache, row_seq, row_pos, kv_src=None, idxk_src=None, stream=None):
    """Append rows (main KV and/or indexer keys) at (row_seq[i], row_pos[i]) of a PagedCache."""
    _expect(row_seq, torch.int32, "row_seq"); _expect(row_pos, torch.int64, "row_pos")
    n = (kv_src if kv_src is not None else idxk_src).shape[0]
    C = kv_src.shape[1] if kv_src is not None else 0
    D = idxk_src.shape[1] if idxk_src is not None else 0
    _check(lib.fp4kv_paged_kv_append(cache.fmt, _ptr(kv_src), _ptr(idxk_src), n, C, D, _ptr(row_seq), _ptr(row_pos),
                                     _ptr(cache.block_table), cache.n_seq, cache.max_pages, cache.page_rows,
                                     cache.n_pages, _ptr(cache.codes), _ptr(cache.scales), _ptr(cache.idx_k),
                                     _stream(stream)))


def fp4kv_swa_ring_append(k_src, v_src, row_seq, row_pos, ring_k, ring_v, stream=None):
    """Write window rows to slot row_pos mod W of each row's sequence in a ring [n_seq, W, C]."""
    _expect(k_src, torch.bfloat16, "k_src"); _expect(v_src, torch.bfloat16, "v_src")
    n, C = k_src.shape
    n_seq, W, _ = ring_k.shape
    _check(lib.fp4kv_swa_ring_append(_ptr(k_src), _ptr(v_src), n, C, _ptr(row_seq), _ptr(row_pos), n_seq, W,
                                     _ptr(ring_k), _ptr(ring_v), _stream(stream)))


def fp4kv_index_full_paged(idx_q, w, cache, q_pos, q_per_seq, max_ctx, P, k, block=8, workspace=None, stream=None):
    """Full-layer indexer over the paged keys of a PagedCache. Returns (pool, n_pool, idx, n_idx)."""
    n_q, H, D = idx_q.shape
    dev = idx_q.device
    pool = torch.empty((n_q, P), dtype=torch.int32, device=dev)
    n_pool = torch.empty((n_q,), dtype=torch.int32, device=dev)
    idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    n_idx = torch.empty((n_q,), dtype=torch.int32, device=dev)
    ws = _workspace(fp4kv_index_workspace_bytes(n_q, max_ctx, block), dev, workspace)
    _check(lib.fp4kv_index_full_paged(_ptr(idx_q), _ptr(w), _ptr(cache.idx_k), _ptr(cache.block_table), cache.n_seq,
                                      cache.max_pages, cache.page_rows, cache.n_pages, _ptr(q_pos), n_q, q_per_seq, H,
                                      D, max_ctx, block, P, k, _ptr(pool), _ptr(n_pool), _ptr(idx), _ptr(n_idx),
                                      _ptr(ws), ws.numel(), _stream(stream)))
    return pool, n_pool, idx, n_idx


def fp4kv_index_reindex_paged(idx_q, w, cache, q_pos, q_per_seq, pool, n_pool, k, block=8, workspace=None,
                              stream=None):
    """Reindex over the paged keys of a PagedCache with an inherited pool. Returns (idx, n_idx)."""
    n_q, H, D = idx_q.shape
    P = pool.shape[1]
    dev = idx_q.device
    idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    n_idx = torch.empty((n_q,), dtype=torch.int32, device=dev)
    ws = _workspace(fp4kv_reindex_workspace_bytes(n_q, P, block), dev, workspace)
    _check(lib.fp4kv_index_reindex_paged(_ptr(idx_q), _ptr(w), _ptr(cache.idx_k), _ptr(cache.block_table),
                                         cache.n_seq, cache.max_pages, cache.page_rows, cache.n_pages, _ptr(q_pos),
                                         n_q, q_per_seq, H, D, _ptr(pool), _ptr(n_pool), block, P, k, _ptr(idx),
                                         _ptr(n_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, n_idx


def fp4kv_sparse_attn_decode_paged(q, cache, idx, n_idx, ring_k, ring_v, q_pos, scale, out=None, lse=None,
                                   workspace=None, stream=None):
    """Decode attention over the paged main KV of a PagedCache and a window ring [B, W, C]."""
    _expect(q, torch.bfloat16, "q"); _expect(idx, torch.int32, "idx"); _expect(n_idx, torch.int32, "n_idx")
    B, Hq, C = q.shape
    k = idx.shape[1]
    W = ring_k.shape[1]
    dev = q.device
    out = torch.empty((B, Hq, C), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace(fp4kv_attn_workspace_bytes(B, Hq, C, k, W), dev, workspace)
    _check(lib.fp4kv_sparse_attn_decode_paged(cache.fmt, _ptr(q), _ptr(cache.codes), _ptr(cache.scales),
                                              _ptr(cache.block_table), cache.max_pages, cache.page_rows,
                                              cache.n_pages, _ptr(idx), _ptr(n_idx), _ptr(ring_k), _ptr(ring_v),
                                              _ptr(q_pos), B, Hq, C, k, W, float(scale), _ptr(out), _ptr(lse),
                                              _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse
