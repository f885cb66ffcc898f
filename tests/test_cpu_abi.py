"""The C-ABI library loads and exports every entry point include/fp4kv.h
declares; host-side argument checks and workspace sizing work without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4kv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import sparse_indexer_fp4_amd as fk
    return fk


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(lib.lib, n), n
    assert sorted(lib.EXPORTS) == names


def test_abi_version(lib):
    assert lib.abi_version() == 1


def test_null_and_shape_errors_without_gpu(lib):
    L = lib.lib
    assert L.fp4kv_quantize_append(None, 4, 512, None, 0, None, None, 4, None) == -1
    assert b"non-NULL" in L.fp4kv_last_error()
    fake = ctypes.c_void_p(4096)   # never dereferenced: the call fails validation first
    assert L.fp4kv_quantize_append(fake, 4, 500, None, 0, fake, fake, 4, None) == -2
    assert L.fp4kv_quantize_append(fake, 4, 512, None, 1, fake, fake, 4, None) == -2
    assert L.fp4kv_quantize_append(fake, 0, 512, None, 0, fake, fake, 4, None) == 0
    assert L.fp4kv_quantize_append(None, 0, 512, None, 0, None, None, 4, None) == 0   # nothing to append
    assert L.fp4kv_last_error() == b""
    # index_full: block must be 8, P*block <= 16384, k <= P*block, workspace large enough
    args = [fake, fake, fake, 100, fake, fake, 1, 1, 16, 128, 100]
    out = [fake, fake, fake, fake]
    assert L.fp4kv_index_full(*args, 16, 4, 2, *out, fake, 1 << 30, None) == -4
    assert L.fp4kv_index_full(*args, 8, 4096, 2, *out, fake, 1 << 30, None) == -4
    assert L.fp4kv_index_full(*args, 8, 4, 33, *out, fake, 1 << 30, None) == -2
    assert L.fp4kv_index_full(*args, 8, 4, 2, *out, fake, 10, None) == -3
    assert L.fp4kv_index_full(*[fake, fake, fake, 100, fake, fake, 1, 1, 3, 128, 100], 8, 4, 2, *out, fake,
                              1 << 30, None) == -4
    # attention: only C = 512 and Hq in {16, 32, 64}
    a = [fake, fake, fake, 100, fake, fake, fake, fake, fake, fake, 1]
    assert L.fp4kv_sparse_attn_decode(*a, 64, 256, 8, 128, ctypes.c_float(0.1), fake, None, fake, 1 << 30, None) == -4
    assert L.fp4kv_sparse_attn_decode(*a, 48, 512, 8, 128, ctypes.c_float(0.1), fake, None, fake, 1 << 30, None) == -4
    assert L.fp4kv_sparse_attn_decode(*a, 64, 512, 0, 128, ctypes.c_float(0.1), fake, None, fake, 1 << 30, None) == -2


def test_noalloc_limit_without_gpu(lib):
    """The allocation-free Full indexer refuses calls whose scores would not fit its
    fixed 64 MiB device array, before touching the device."""
    L = lib.lib
    fake = ctypes.c_void_p(4096)
    out = [fake, fake, fake, fake]
    # 64 queries x 2^20 positions of fp32 scores (256 MiB) > 64 MiB
    assert L.fp4kv_index_full_noalloc(fake, fake, fake, 1 << 26, fake, fake, 64, 1, 16, 128, 1 << 20, 8, 2048,
                                      512, *out, None) == -3
    assert b"64" in L.fp4kv_last_error() or b"67108864" in L.fp4kv_last_error()
    assert L.fp4kv_index_full_noalloc(fake, fake, fake, 1 << 26, fake, fake, 0, 1, 16, 128, 1 << 20, 8, 2048,
                                      512, *out, None) == 0
    assert L.fp4kv_index_full_noalloc(fake, fake, fake, 1 << 26, fake, fake, 1, 1, 16, 128, 1 << 20, 16, 2048,
                                      512, *out, None) == -4


def test_workspace_sizes(lib):
    assert lib.fp4kv_index_workspace_bytes(32, 131072) >= 32 * 131072 * 4 + 32 * 16384 * 4
    assert lib.fp4kv_reindex_workspace_bytes(8, 2048) >= 8 * 2048 * 8 * 4
    assert lib.fp4kv_attn_workspace_bytes(4096, 64, 512, 512, 128) == 0   # one split when queries fill the GPU
    assert lib.fp4kv_attn_workspace_bytes(1, 64, 512, 512, 128) > 0


def test_kv_format_sizes_and_checks_without_gpu(lib):
    """Row bytes per main-KV format; unknown formats are refused; an FP8 cache
    needs no scale plane. Nothing is launched (zero rows or queries)."""
    L = lib.lib
    assert [L.fp4kv_kv_code_bytes(f, 512) for f in (0, 1, 2)] == [256, 256, 512]
    assert [L.fp4kv_kv_scale_bytes(f, 512) for f in (0, 1, 2)] == [32, 16, 0]
    assert L.fp4kv_kv_code_bytes(3, 512) == -1 and L.fp4kv_kv_scale_bytes(1, 48) == -1
    fake = ctypes.c_void_p(4096)
    assert L.fp4kv_kv_append(3, fake, 4, 512, None, 0, fake, fake, 4, None) == -4
    assert L.fp4kv_kv_append(1, fake, 4, 512, None, 0, fake, None, 4, None) == -1     # MXFP4 needs scales
    assert L.fp4kv_kv_append(2, fake, 0, 512, None, 0, fake, None, 4, None) == 0      # FP8: no scale plane
    assert L.fp4kv_kv_append(1, fake, 4, 64, None, 2, fake, fake, 4, None) == -2      # rows past the cache
    # q, codes, scales = NULL, total_rows, seq_start, idx, n_idx, swa_k, swa_v, q_pos, B = 0, Hq, C, k, W, ...
    a = [fake, fake, None, 100, fake, fake, fake, fake, fake, fake, 0, 64, 512, 8, 128, ctypes.c_float(0.1), fake,
         None, fake, 1 << 30, None]
    assert L.fp4kv_sparse_attn_decode_kv(2, *a) == 0                        # FP8, no queries, no scale plane
    assert L.fp4kv_sparse_attn_decode_kv(1, *a) == -1                       # MXFP4 needs scales
    assert L.fp4kv_sparse_attn_decode_kv(5, *a) == -4


def test_paged_checks_without_gpu(lib):
    """Page arguments are validated before anything runs: page_rows a power of two
    in [64, 2^20], a block table, max_ctx within the table's reach."""
    L = lib.lib
    fake = ctypes.c_void_p(4096)
    # fmt, kv_src, idxk_src, n_rows, C, D, row_seq, row_pos, block_table, n_seq, max_pages, page_rows, n_pages, ...
    base = [0, fake, None, 4, 512, 0, fake, fake, fake, 2, 8]
    tail = [fake, fake, None, None]
    assert L.fp4kv_paged_kv_append(*base, 96, 16, *tail) == -2          # not a power of two
    assert L.fp4kv_paged_kv_append(*base, 32, 16, *tail) == -2          # below 64
    assert L.fp4kv_paged_kv_append(*[0, fake, None, 4, 512, 0, fake, fake, None, 2, 8], 64, 16, *tail) == -1
    assert L.fp4kv_paged_kv_append(*[0, fake, None, 0, 512, 0, fake, fake, fake, 2, 8], 64, 16, *tail) == 0
    assert L.fp4kv_swa_ring_append(fake, fake, 0, 512, fake, fake, 2, 128, fake, fake, None) == 0
    assert L.fp4kv_swa_ring_append(fake, fake, 4, 512, fake, fake, 2, 0, fake, fake, None) == -2
    # index_full_paged: max_ctx beyond max_pages * page_rows
    out = [fake, fake, fake, fake, fake, 1 << 40, None]
    assert L.fp4kv_index_full_paged(fake, fake, fake, fake, 2, 8, 64, 16, fake, 2, 1, 16, 128, 513, 8, 64, 32,
                                    *out) == -2
    assert L.fp4kv_index_full_paged(fake, fake, fake, fake, 2, 8, 64, 16, fake, 0, 1, 16, 128, 512, 8, 64, 32,
                                    *out) == 0
