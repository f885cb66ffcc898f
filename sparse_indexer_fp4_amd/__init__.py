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
    "fp4kv_index_full_append": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                       _p, _p, _p, _p, _i32, _p, _i64, _i32, _p, _i64, _p, _p, _i64, _p, _sz, _p]),
    "fp4kv_index_scores_append": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _p, _p,
                                         _i32, _p, _i64, _i32, _p, _i64, _p, _p, _i64, _p]),
    "fp4kv_index_full_noalloc": (_i32, [_p, _p, _p, _i64, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                        _p, _p, _p, _p, _p]),
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


def _expect(t, dtype, name, shape=None):
    """dtype (and, if given, shape: a tuple whose None entries match any size) of a
    tensor argument, checked before its pointer is handed to the library, which
    trusts the sizes the call implies."""
    if t is None:
        raise ValueError(f"{name}: a tensor is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(d) != int(s) for d, s in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if s is None else str(int(s)) for s in shape) + "]"
            raise ValueError(f"{name}: expected shape {want}, got {list(t.shape)}")


def _out(t, shape, dtype, device, name):
    """A caller-supplied output checked like an input, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _expect(t, dtype, name, shape)
    return t


def _cache_planes(codes, scales, fmt, C, rows=None):
    """Code and scale planes of a main-KV cache in format fmt at C channels."""
    cb, sb = lib.fp4kv_kv_code_bytes(fmt, C), lib.fp4kv_kv_scale_bytes(fmt, C)
    if cb < 0:
        raise ValueError(f"format {fmt} with C={C} is not supported")
    _expect(codes, torch.uint8, "codes", (rows, cb))
    if sb > 0:
        _expect(scales, torch.uint8, "scales", (codes.shape[0], sb))
    elif scales is not None:
        _expect(scales, torch.uint8, "scales")


def abi_version() -> int:
    return lib.fp4kv_abi_version()


def fp4kv_quantize_append(src, codes, scales, dst_rows=None, dst_start=0, stream=None):
    """FP4 quantize-append of bf16 rows src [n, C] into (codes [cap, C/2], scales [cap, C/16])."""
    _expect(src, torch.bfloat16, "src", (None, None))
    n, C = src.shape
    _cache_planes(codes, scales, KV_FP4, C)
    if dst_rows is not None:
        _expect(dst_rows, torch.int64, "dst_rows", (n,))
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


def _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start=None, n_seq=None):
    """Checks of the indexer's query-side inputs; returns (n_q, H, D)."""
    _expect(idx_q, torch.bfloat16, "idx_q", (None, None, None))
    n_q, H, D = idx_q.shape
    _expect(w, torch.float32, "w", (n_q, H))
    _expect(idx_k, torch.bfloat16, "idx_k", (None, D))
    _expect(q_pos, torch.int32, "q_pos", (n_q,))
    if seq_start is not None or n_seq is not None:
        _expect(seq_start, torch.int64, "seq_start", (n_seq,))
    return n_q, H, D


def _n_seq(n_q, q_per_seq):
    if q_per_seq < 1:
        raise ValueError("q_per_seq must be >= 1")
    return (n_q + q_per_seq - 1) // q_per_seq


def fp4kv_index_full(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, P, k, block=8,
                     pool_out=None, n_pool=None, idx_out=None, n_idx=None, workspace=None, stream=None):
    """Full-mode indexer. idx_q bf16 [n_q, H, D], w f32 [n_q, H], idx_k bf16 [rows, D],
    seq_start i64 [n_seq], q_pos i32 [n_q]. Returns (pool [n_q, P], n_pool, idx [n_q, k], n_idx)."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    dev = idx_q.device
    pool_out = _out(pool_out, (n_q, P), torch.int32, dev, "pool_out")
    n_pool = _out(n_pool, (n_q,), torch.int32, dev, "n_pool")
    idx_out = _out(idx_out, (n_q, k), torch.int32, dev, "idx_out")
    n_idx = _out(n_idx, (n_q,), torch.int32, dev, "n_idx")
    ws = _workspace(fp4kv_index_workspace_bytes(n_q, max_ctx, block), dev, workspace)
    _check(lib.fp4kv_index_full(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                n_q, q_per_seq, H, D, max_ctx, block, P, k, _ptr(pool_out), _ptr(n_pool),
                                _ptr(idx_out), _ptr(n_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def _append_args(fmt, kv_src, codes, scales, dst_rows, dst_start):
    """Checks of a main-KV append carried by an indexer call; returns the C arguments."""
    _expect(kv_src, torch.bfloat16, "kv_src", (None, None))
    n, C = kv_src.shape
    _cache_planes(codes, scales, fmt, C)
    if dst_rows is not None:
        _expect(dst_rows, torch.int64, "dst_rows", (n,))
    return [fmt, _ptr(kv_src), n, C, _ptr(dst_rows), dst_start, _ptr(codes), _ptr(scales), codes.shape[0]]


def fp4kv_index_full_append(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, P, k, kv_src, codes, scales,
                            dst_rows=None, dst_start=0, kv_fmt=KV_FP4, block=8, pool_out=None, n_pool=None,
                            idx_out=None, n_idx=None, workspace=None, stream=None):
    """fp4kv_index_full plus the main-KV append of kv_src (bf16 [n, C]) into (codes,
    scales), the append riding in the indexer scan's launch. Returns (pool, n_pool, idx, n_idx)."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    app = _append_args(kv_fmt, kv_src, codes, scales, dst_rows, dst_start)
    dev = idx_q.device
    pool_out = _out(pool_out, (n_q, P), torch.int32, dev, "pool_out")
    n_pool = _out(n_pool, (n_q,), torch.int32, dev, "n_pool")
    idx_out = _out(idx_out, (n_q, k), torch.int32, dev, "idx_out")
    n_idx = _out(n_idx, (n_q,), torch.int32, dev, "n_idx")
    ws = _workspace(fp4kv_index_workspace_bytes(n_q, max_ctx, block), dev, workspace)
    _check(lib.fp4kv_index_full_append(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start),
                                       _ptr(q_pos), n_q, q_per_seq, H, D, max_ctx, block, P, k, _ptr(pool_out),
                                       _ptr(n_pool), _ptr(idx_out), _ptr(n_idx), *app, _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def fp4kv_index_scores_append(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, kv_src, codes, scales,
                              dst_rows=None, dst_start=0, kv_fmt=KV_FP4, block=8, scores=None, blockmax=None,
                              stream=None):
    """fp4kv_index_scores plus the main-KV append of kv_src in the same launch.
    Returns (scores, blockmax)."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    app = _append_args(kv_fmt, kv_src, codes, scales, dst_rows, dst_start)
    dev = idx_q.device
    nblk = (max_ctx + block - 1) // block
    scores = _out(scores, (n_q, max_ctx), torch.float32, dev, "scores")
    blockmax = _out(blockmax, (n_q, nblk), torch.float32, dev, "blockmax")
    _check(lib.fp4kv_index_scores_append(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start),
                                         _ptr(q_pos), n_q, q_per_seq, H, D, max_ctx, block, _ptr(scores),
                                         _ptr(blockmax), *app, _stream(stream)))
    return scores, blockmax


def fp4kv_index_full_noalloc(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, P, k, pool_out, n_pool,
                             idx_out, n_idx, block=8, stream=None):
    """fp4kv_index_full with the library's fixed device workspace: the caller passes
    every output, and neither this wrapper nor the library allocates anything."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    _expect(pool_out, torch.int32, "pool_out", (n_q, P))
    _expect(n_pool, torch.int32, "n_pool", (n_q,))
    _expect(idx_out, torch.int32, "idx_out", (n_q, k))
    _expect(n_idx, torch.int32, "n_idx", (n_q,))
    _check(lib.fp4kv_index_full_noalloc(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start),
                                        _ptr(q_pos), n_q, q_per_seq, H, D, max_ctx, block, P, k, _ptr(pool_out),
                                        _ptr(n_pool), _ptr(idx_out), _ptr(n_idx), _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def fp4kv_index_scores(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, max_ctx, block=8, scores=None, blockmax=None,
                       stream=None):
    """Scan half of the Full indexer. Returns (scores f32 [n_q, max_ctx], blockmax f32 [n_q, nblk])."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    dev = idx_q.device
    nblk = (max_ctx + block - 1) // block
    scores = _out(scores, (n_q, max_ctx), torch.float32, dev, "scores")
    blockmax = _out(blockmax, (n_q, nblk), torch.float32, dev, "blockmax")
    _check(lib.fp4kv_index_scores(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                  n_q, q_per_seq, H, D, max_ctx, block, _ptr(scores), _ptr(blockmax),
                                  _stream(stream)))
    return scores, blockmax


def fp4kv_index_select(scores, blockmax, total_rows, seq_start, q_pos, q_per_seq, P, k, block=8, pool_out=None,
                       n_pool=None, idx_out=None, n_idx=None, stream=None):
    """Selection half of the Full indexer. Returns (pool, n_pool, idx, n_idx)."""
    _expect(scores, torch.float32, "scores", (None, None))
    n_q, max_ctx = scores.shape
    _expect(blockmax, torch.float32, "blockmax", (n_q, (max_ctx + block - 1) // block))
    _expect(seq_start, torch.int64, "seq_start", (_n_seq(n_q, q_per_seq),))
    _expect(q_pos, torch.int32, "q_pos", (n_q,))
    dev = scores.device
    pool_out = _out(pool_out, (n_q, P), torch.int32, dev, "pool_out")
    n_pool = _out(n_pool, (n_q,), torch.int32, dev, "n_pool")
    idx_out = _out(idx_out, (n_q, k), torch.int32, dev, "idx_out")
    n_idx = _out(n_idx, (n_q,), torch.int32, dev, "n_idx")
    _check(lib.fp4kv_index_select(_ptr(scores), _ptr(blockmax), int(total_rows), _ptr(seq_start), _ptr(q_pos), n_q,
                                  q_per_seq, max_ctx, block, P, k, _ptr(pool_out), _ptr(n_pool), _ptr(idx_out),
                                  _ptr(n_idx), _stream(stream)))
    return pool_out, n_pool, idx_out, n_idx


def fp4kv_index_reindex(idx_q, w, idx_k, seq_start, q_pos, q_per_seq, pool, n_pool, k, block=8,
                        idx_out=None, n_idx=None, workspace=None, stream=None):
    """Reindex-mode indexer over an inherited pool [n_q, P]. Returns (idx [n_q, k], n_idx)."""
    n_q = idx_q.shape[0]
    n_q, H, D = _indexer_inputs(idx_q, w, idx_k, q_pos, seq_start, _n_seq(n_q, q_per_seq))
    _expect(pool, torch.int32, "pool", (n_q, None))
    _expect(n_pool, torch.int32, "n_pool", (n_q,))
    P = pool.shape[1]
    dev = idx_q.device
    idx_out = _out(idx_out, (n_q, k), torch.int32, dev, "idx_out")
    n_idx = _out(n_idx, (n_q,), torch.int32, dev, "n_idx")
    ws = _workspace(fp4kv_reindex_workspace_bytes(n_q, P, block), dev, workspace)
    _check(lib.fp4kv_index_reindex(_ptr(idx_q), _ptr(w), _ptr(idx_k), idx_k.shape[0], _ptr(seq_start), _ptr(q_pos),
                                   n_q, q_per_seq, H, D, _ptr(pool), _ptr(n_pool), block, P, k, _ptr(idx_out),
                                   _ptr(n_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return idx_out, n_idx


def _attn_common(fmt, q, codes, scales, idx, n_idx, B, out, lse, workspace, W):
    """Checks shared by the attention wrappers; returns (Hq, C, k, out, lse, ws)."""
    _expect(q, torch.bfloat16, "q", (B, None, None))
    _, Hq, C = q.shape
    _cache_planes(codes, scales, fmt, C)
    _expect(idx, torch.int32, "idx", (B, None))
    _expect(n_idx, torch.int32, "n_idx", (B,))
    k = idx.shape[1]
    dev = q.device
    out = _out(out, (B, Hq, C), torch.float32, dev, "out")
    if lse is not None:
        _expect(lse, torch.float32, "lse", (B, Hq))
    else:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(fp4kv_attn_workspace_bytes(B, Hq, C, k, W), dev, workspace)
    return Hq, C, k, out, lse, ws


def fp4kv_sparse_attn_decode(q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, q_pos, scale,
                             out=None, lse=None, workspace=None, stream=None):
    """Decode attention. q bf16 [B, Hq, C]; codes/scales the FP4 cache; idx i32 [B, k];
    swa_k/swa_v bf16 [B, W, C]. Returns (out f32 [B, Hq, C], lse f32 [B, Hq])."""
    B, W, _ = _decode_inputs(q, seq_start, swa_k, swa_v, q_pos)
    Hq, C, k, out, lse, ws = _attn_common(KV_FP4, q, codes, scales, idx, n_idx, B, out, lse, workspace, W)
    _check(lib.fp4kv_sparse_attn_decode(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], _ptr(seq_start),
                                        _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), _ptr(q_pos), B, Hq, C, k, W,
                                        float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def _decode_inputs(q, seq_start, swa_k, swa_v, q_pos):
    B = q.shape[0]
    _expect(swa_k, torch.bfloat16, "swa_k", (B, None, q.shape[2] if q.dim() == 3 else None))
    _expect(swa_v, torch.bfloat16, "swa_v", tuple(swa_k.shape))
    _expect(seq_start, torch.int64, "seq_start", (B,))
    _expect(q_pos, torch.int32, "q_pos", (B,))
    return B, swa_k.shape[1], None


def fp4kv_sparse_attn_prefill(q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, pos0, W, scale,
                              out=None, lse=None, workspace=None, stream=None):
    """Prefill-chunk attention. q bf16 [T, Hq, C] at positions pos0..pos0+T-1; swa_k/swa_v
    bf16 [T+W-1, C] (row r = position pos0-W+1+r). Returns (out, lse)."""
    T = q.shape[0]
    C = q.shape[2] if q.dim() == 3 else None
    _expect(swa_k, torch.bfloat16, "swa_k", (T + W - 1, C))
    _expect(swa_v, torch.bfloat16, "swa_v", (T + W - 1, C))
    Hq, C, k, out, lse, ws = _attn_common(KV_FP4, q, codes, scales, idx, n_idx, T, out, lse, workspace, W)
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
    _expect(src, torch.bfloat16, "src", (None, None))
    n, C = src.shape
    _cache_planes(codes, scales, fmt, C)
    if dst_rows is not None:
        _expect(dst_rows, torch.int64, "dst_rows", (n,))
    _check(lib.fp4kv_kv_append(fmt, _ptr(src), n, C, _ptr(dst_rows), dst_start, _ptr(codes), _ptr(scales),
                               codes.shape[0], _stream(stream)))


def fp4kv_sparse_attn_decode_kv(fmt, q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, q_pos, scale,
                                out=None, lse=None, workspace=None, stream=None):
    """Decode attention over a cache in format fmt (scales may be None for KV_FP8)."""
    B, W, _ = _decode_inputs(q, seq_start, swa_k, swa_v, q_pos)
    Hq, C, k, out, lse, ws = _attn_common(fmt, q, codes, scales, idx, n_idx, B, out, lse, workspace, W)
    _check(lib.fp4kv_sparse_attn_decode_kv(fmt, _ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], _ptr(seq_start),
                                           _ptr(idx), _ptr(n_idx), _ptr(swa_k), _ptr(swa_v), _ptr(q_pos), B, Hq, C, k,
                                           W, float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                           _stream(stream)))
    return out, lse


def fp4kv_sparse_attn_prefill_kv(fmt, q, codes, scales, seq_start, idx, n_idx, swa_k, swa_v, pos0, W, scale,
                                 out=None, lse=None, workspace=None, stream=None):
    """Prefill-chunk attention over a cache in format fmt (scales may be None for KV_FP8)."""
    T = q.shape[0]
    C = q.shape[2] if q.dim() == 3 else None
    _expect(swa_k, torch.bfloat16, "swa_k", (T + W - 1, C))
    _expect(swa_v, torch.bfloat16, "swa_v", (T + W - 1, C))
    Hq, C, k, out, lse, ws = _attn_common(fmt, q, codes, scales, idx, n_idx, T, out, lse, workspace, W)
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

    @property
    def rows(self):
        return self.n_pages * self.page_rows

    def check(self, C=None, D=None):
        """Dtypes and shapes of every store against the page geometry: each
        store holds n_pages * page_rows rows."""
        _expect(self.block_table, torch.int32, "block_table", (None, None))
        if C is not None and self.codes is not None:
            _cache_planes(self.codes, self.scales, self.fmt, C, rows=self.rows)
        if D is not None and self.idx_k is not None:
            _expect(self.idx_k, torch.bfloat16, "idx_k", (self.rows, D))


def fp4kv_paged_kv_append(cache, row_seq, row_pos, kv_src=None, idxk_src=None, stream=None):
    """Append rows (main KV and/or indexer keys) at (row_seq[i], row_pos[i]) of a PagedCache."""
    src = kv_src if kv_src is not None else idxk_src
    if src is None:
        raise ValueError("one of kv_src and idxk_src is required")
    n = src.shape[0]
    C = D = 0
    if kv_src is not None:
        _expect(kv_src, torch.bfloat16, "kv_src", (n, None))
        C = kv_src.shape[1]
    if idxk_src is not None:
        _expect(idxk_src, torch.bfloat16, "idxk_src", (n, None))
        D = idxk_src.shape[1]
    cache.check(C=C or None, D=D or None)
    _expect(row_seq, torch.int32, "row_seq", (n,))
    _expect(row_pos, torch.int64, "row_pos", (n,))
    _check(lib.fp4kv_paged_kv_append(cache.fmt, _ptr(kv_src), _ptr(idxk_src), n, C, D, _ptr(row_seq), _ptr(row_pos),
                                     _ptr(cache.block_table), cache.n_seq, cache.max_pages, cache.page_rows,
                                     cache.n_pages, _ptr(cache.codes if kv_src is not None else None),
                                     _ptr(cache.scales if kv_src is not None else None),
                                     _ptr(cache.idx_k if idxk_src is not None else None), _stream(stream)))


def fp4kv_swa_ring_append(k_src, v_src, row_seq, row_pos, ring_k, ring_v, stream=None):
    """Write window rows to slot row_pos mod W of each row's sequence in a ring [n_seq, W, C]."""
    _expect(k_src, torch.bfloat16, "k_src", (None, None))
    n, C = k_src.shape
    _expect(v_src, torch.bfloat16, "v_src", (n, C))
    _expect(ring_k, torch.bfloat16, "ring_k", (None, None, C))
    _expect(ring_v, torch.bfloat16, "ring_v", tuple(ring_k.shape))
    _expect(row_seq, torch.int32, "row_seq", (n,))
    _expect(row_pos, torch.int64, "row_pos", (n,))
    n_seq, W, _ = ring_k.shape
    _check(lib.fp4kv_swa_ring_append(_ptr(k_src), _ptr(v_src), n, C, _ptr(row_seq), _ptr(row_pos), n_seq, W,
                                     _ptr(ring_k), _ptr(ring_v), _stream(stream)))


def fp4kv_index_full_paged(idx_q, w, cache, q_pos, q_per_seq, max_ctx, P, k, block=8, workspace=None, stream=None):
    """Full-layer indexer over the paged keys of a PagedCache. Returns (pool, n_pool, idx, n_idx)."""
    n_q, H, D = _indexer_inputs(idx_q, w, cache.idx_k, q_pos)
    cache.check(D=D)
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
    n_q, H, D = _indexer_inputs(idx_q, w, cache.idx_k, q_pos)
    cache.check(D=D)
    _expect(pool, torch.int32, "pool", (n_q, None))
    _expect(n_pool, torch.int32, "n_pool", (n_q,))
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
    B = q.shape[0]
    C = q.shape[2] if q.dim() == 3 else None
    _expect(ring_k, torch.bfloat16, "ring_k", (B, None, C))
    _expect(ring_v, torch.bfloat16, "ring_v", tuple(ring_k.shape))
    _expect(q_pos, torch.int32, "q_pos", (B,))
    _expect(cache.block_table, torch.int32, "block_table", (B, None))
    W = ring_k.shape[1]
    Hq, C, k, out, lse, ws = _attn_common(cache.fmt, q, cache.codes, cache.scales, idx, n_idx, B, out, lse,
                                          workspace, W)
    cache.check(C=C)
    _check(lib.fp4kv_sparse_attn_decode_paged(cache.fmt, _ptr(q), _ptr(cache.codes), _ptr(cache.scales),
                                              _ptr(cache.block_table), cache.max_pages, cache.page_rows,
                                              cache.n_pages, _ptr(idx), _ptr(n_idx), _ptr(ring_k), _ptr(ring_v),
                                              _ptr(q_pos), B, Hq, C, k, W, float(scale), _ptr(out), _ptr(lse),
                                              _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse
