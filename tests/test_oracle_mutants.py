"""Plant plausible mistakes in the oracle (CPU only) and require the pins to
catch each of them: a dropped term, a wrong sign, an off-by-one, a wrong
tie-break or order, a transposed or swapped operand."""
import math

import numpy as np
import pytest

from oracle import attention, chain, fp4, indexer, kvformats, paged
from tests import oracle_pins


def _no_relu(q, w, k):
    q = np.asarray(q, float); k = np.asarray(k, float)
    return ((k @ q.T) * np.asarray(w, float)[None, :]).sum(axis=1)


def _drop_last_head(q, w, k):
    q = np.asarray(q, float)
    if q.shape[0] > 1:
        q = q[:-1]; w = np.asarray(w)[:-1]
    return np.maximum(np.asarray(k, float) @ q.T, 0) @ np.asarray(w, float)


def _relu_after_weight_sum(q, w, k):
    return np.maximum((np.asarray(k, float) @ np.asarray(q, float).T) @ np.asarray(w, float), 0)


def _block_of_9(s, block=8):
    return indexer.__dict__["_orig_block_maxima"](s, block + 1)


def _block_first_only(s, block=8):
    n = s.shape[0]
    return np.array([s[b * block] for b in range(-(-n // block))], dtype=float)


def _ties_to_higher(keys, ids, count):
    keys = np.asarray(keys, float); ids = np.asarray(ids)
    order = np.lexsort((-ids, -keys))
    return np.sort(ids[order[:count]])


def _rank_order(keys, ids, count):
    keys = np.asarray(keys, float); ids = np.asarray(ids)
    return ids[np.lexsort((ids, -keys))[:count]]


def _scale_floor(amax):
    a = np.minimum(np.asarray(amax, float), 6 * 448.0)
    vals = fp4.E4M3_TABLE[:127]
    return np.array([np.nonzero(vals <= x / 6)[0][-1] for x in np.atleast_1d(a)], dtype=np.uint8).reshape(np.shape(a))


def _scale_ties_up(amax):
    a = np.minimum(np.asarray(amax, float), 6 * 448.0)
    d = np.abs(a[..., None] - 6 * fp4.E4M3_TABLE[:127])
    return (d.shape[-1] - 1 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)


def _values_ties_up(x, scale):
    x = np.asarray(x, float); s = np.broadcast_to(np.asarray(scale, float), x.shape)
    ax = np.minimum(np.abs(x), 6 * s)
    d = np.abs(ax[..., None] - s[..., None] * fp4.E2M1_TABLE[:8])
    mag = 7 - np.argmin(d[..., ::-1], axis=-1)
    mag = np.where(s == 0, 0, mag)
    return ((np.signbit(x).astype(int) << 3) | mag).astype(np.uint8)


def _values_no_sign(x, scale):
    return fp4.__dict__["_orig_encode_values"](np.abs(x), scale)


def _swap_nibbles(x):
    codes, scales = fp4.__dict__["_orig_quantize_rows"](x)
    return ((codes >> 4) | ((codes & 0xF) << 4)).astype(np.uint8), scales


def _e4m3_bias8(code):
    v = fp4.__dict__["_orig_e4m3_value"](code)
    return v / 2.0


def _branch_no_scale(q, keys, values, scale):
    return attention.__dict__["_orig_branch"](q, keys, values, 1.0)


def _merge_swapped(o_s, lse_s, o_w, lse_w):
    return attention.__dict__["_orig_merge"](o_s, lse_w, o_w, lse_s)


def _reindex_everything(q, w, k_rows_of, pool, q_pos, k_keep, block=8):
    cand = np.arange(q_pos + 1)
    s = indexer.token_scores(q, w, k_rows_of(cand))
    return indexer.select_top(s, cand, min(k_keep, cand.shape[0]))


def _full_sees_next(q, w, k_rows, q_pos, P, k_keep, block=8):
    return indexer.__dict__["_orig_index_full"](q, w, k_rows, q_pos + 1, P, k_keep, block)


def _layers_reuse_full(modes, full_fn, reindex_fn):
    out = []; pool = idx = full_idx = None
    for layer, mode in enumerate(modes):
        if mode == chain.FULL:
            pool, idx = full_fn(layer); full_idx = idx
        elif mode == chain.REINDEX:
            idx = reindex_fn(layer, pool)
        out.append((pool, full_idx if mode == chain.REUSE else idx))
    return out


def _mx_exponent_minus_one(amax):
    a = np.asarray(amax, float)
    _, e = np.frexp(a)
    return np.where(a == 0, -127, np.clip(e.astype(np.int64) - 1 - 1, -127, 127))


def _mx_exponent_ceil(amax):
    a = np.asarray(amax, float)
    _, e = np.frexp(a)
    exact = np.ldexp(0.5, e) == a
    fl = e.astype(np.int64) - 1
    return np.where(a == 0, -127, np.clip(np.where(exact, fl, fl + 1) - 2, -127, 127))


def _mx_scale_bias_128(x):
    codes, scales = kvformats.__dict__["_orig_mxfp4_quantize_rows"](x)
    return codes, (scales.astype(np.int64) + 1).astype(np.uint8)


def _fp8_ties_up(x):
    x = np.asarray(x, float)
    pos = fp4.E4M3_TABLE[:127]
    ax = np.minimum(np.abs(x), 448.0)
    d = np.abs(ax[..., None] - pos)
    mag = 126 - np.argmin(d[..., ::-1], axis=-1)
    return ((np.signbit(x).astype(int) << 7) | mag).astype(np.uint8)


def _fp8_sign_dropped(x):
    return kvformats.__dict__["_orig_fp8_encode"](np.abs(np.asarray(x, float)))


def _fp8_overflow_nan(x):
    c = kvformats.__dict__["_orig_fp8_encode"](x)
    return np.where(np.abs(np.asarray(x, float)) > 448.0, c | 0x7F, c).astype(np.uint8)


def _page_offset_swapped(block_table, page_rows, n_pages, seq, pos):
    if pos < 0 or pos // page_rows >= block_table.shape[1]:
        return -1
    g = int(block_table[seq, pos // page_rows])
    return -1 if g < 0 or g >= n_pages else g + (pos % page_rows) * n_pages


def _page_no_bounds(block_table, page_rows, n_pages, seq, pos):
    if pos < 0 or pos // page_rows >= block_table.shape[1]:
        return -1
    return int(block_table[seq, pos // page_rows]) * page_rows + pos % page_rows


def _ring_slot_off_by_one(pos, W):
    return (pos + 1) % W


MUTANTS = [
    ("scores: no ReLU", indexer, "token_scores", _no_relu),
    ("scores: dropped head", indexer, "token_scores", _drop_last_head),
    ("scores: ReLU after the head sum", indexer, "token_scores", _relu_after_weight_sum),
    ("blocks of 9", indexer, "block_maxima", _block_of_9),
    ("block score = first token", indexer, "block_maxima", _block_first_only),
    ("ties to the higher index", indexer, "select_top", _ties_to_higher),
    ("output in rank order", indexer, "select_top", _rank_order),
    ("scale truncates", fp4, "encode_scale", _scale_floor),
    ("scale ties upward", fp4, "encode_scale", _scale_ties_up),
    ("value ties upward", fp4, "encode_values", _values_ties_up),
    ("value sign dropped", fp4, "encode_values", _values_no_sign),
    ("nibbles swapped", fp4, "quantize_rows", _swap_nibbles),
    ("E4M3 bias 8", fp4, "e4m3_value", _e4m3_bias8),
    ("softmax scale dropped", attention, "branch", _branch_no_scale),
    ("merge weights swapped", attention, "merge", _merge_swapped),
    ("reindex ignores the pool", indexer, "index_reindex", _reindex_everything),
    ("full sees position q_pos+1", indexer, "index_full", _full_sees_next),
    ("reuse copies the Full layer", chain, "layer_indices", _layers_reuse_full),
    ("MX exponent floor(log2) - 1", kvformats, "mx_shared_exponent", _mx_exponent_minus_one),
    ("MX exponent from ceil(log2)", kvformats, "mx_shared_exponent", _mx_exponent_ceil),
    ("MX scale byte biased by 128", kvformats, "mxfp4_quantize_rows", _mx_scale_bias_128),
    ("FP8 ties upward", kvformats, "fp8_encode", _fp8_ties_up),
    ("FP8 sign dropped", kvformats, "fp8_encode", _fp8_sign_dropped),
    ("FP8 overflow to NaN", kvformats, "fp8_encode", _fp8_overflow_nan),
    ("page row and page swapped", paged, "physical_row", _page_offset_swapped),
    ("page ids not bounded", paged, "physical_row", _page_no_bounds),
    ("ring slot off by one", paged, "ring_slot", _ring_slot_off_by_one),
]


@pytest.mark.parametrize("name,mod,attr,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, mod, attr, fn, monkeypatch):
    monkeypatch.setitem(mod.__dict__, "_orig_" + attr, getattr(mod, attr))
    monkeypatch.setattr(mod, attr, fn)
    if mod is fp4 and attr == "e4m3_value":
        monkeypatch.setattr(fp4, "E4M3_TABLE", np.array([fn(c) for c in range(256)]))
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(check.__name__)
    assert failed, f"mutant '{name}' passed every pin"
