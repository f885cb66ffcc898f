"""Checks that pin the oracle to something other than itself.

Each check raises AssertionError when the oracle disagrees with a library
routine, a closed form, a brute force over tiny inputs, a value the pages
state, or an invariant of the method. test_oracle_pins.py runs every check on
the oracle; test_oracle_mutants.py plants plausible mistakes in the oracle and
requires some check to fail for each of them.

Page references: [G] "DeepSeek V4.1 Flash KV Cache: 890 Bytes per Token
Explained"; [T] "890 bytes per token: how DeepSeek V4.1-Flash's KV cache
works"; [N] "DeepSeek-V4.1-Flash: 890 Bytes Per Token, 437x Smaller KV Cache".
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import scipy.special
import torch

from oracle import attention, chain, fp4, indexer, kvformats, paged

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def pages_constants():
    return {k: float(v) for k, v in golden_lines("pages_constants.txt")}


def all_bf16_nonneg_finite():
    """Every finite non-negative bfloat16 value, as float64 (0x0000..0x7F7F)."""
    bits = np.arange(0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- codec ----

def check_e2m1_table():
    """E2M1 decode equals the format's value set (golden, cited)."""
    for code, val in golden_lines("e2m1_values.txt"):
        got = fp4.e2m1_value(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got, val)


def check_e4m3_table():
    """E4M3 decode equals torch's float8_e4m3fn for all 256 codes, and the cited landmarks."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([fp4.e4m3_value(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)[0][:8]
    for code, val in golden_lines("e4m3_points.txt"):
        g = fp4.e4m3_value(int(code, 16))
        v = float(val)
        assert (math.isnan(g) and math.isnan(v)) or g == v, (code, g, v)


def check_scale_encode_exhaustive():
    """Scale code for every finite non-negative bf16 amax equals torch's
    round-to-nearest-even float8_e4m3fn conversion of fp32(amax)/6 after
    saturation at 448. (Rounding the fp32 quotient again to 4 significant bits
    is innocuous: 24 >= 2*4 + 2.)"""
    a = all_bf16_nonneg_finite()
    got = fp4.encode_scale(a)
    q = (torch.from_numpy(a.astype(np.float32)) / 6.0).clamp(max=448.0)
    ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (bad.size, a[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # saturation and underflow landmarks
    assert fp4.E4M3_TABLE[fp4.encode_scale(np.array([1e30]))[0]] == 448.0
    assert fp4.encode_scale(np.array([6 * 2.0 ** -10]))[0] == 0       # tie 0 | 2^-9 -> even code 0
    assert fp4.encode_scale(np.array([6 * 1.5 * 2.0 ** -9]))[0] == 2  # tie codes 1|2 -> 2


def _e2m1_rne_reference(r):
    """E2M1 magnitude code of ratio r >= 0 by library round-half-even (np.round)
    on the grid spacing of each binade, saturating at 6."""
    r = np.asarray(r, dtype=np.float64)
    v = np.where(r < 2.0, np.round(r * 2.0) / 2.0,
                 np.where(r < 4.0, np.round(r), 2.0 * np.round(r / 2.0)))
    v = np.minimum(v, 6.0)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    return np.searchsorted(mags, v)


def check_value_encode_exhaustive():
    """Value codes for every finite bf16 |x| times every nonzero finite E4M3
    scale equal the np.round (half-to-even) reference on |x|/s."""
    x = all_bf16_nonneg_finite()
    scales = np.array([fp4.e4m3_value(c) for c in range(1, 127)])
    for s in scales:
        sel = x
        got = fp4.encode_values(sel, s).astype(np.int64)
        ref = _e2m1_rne_reference(sel / s)
        assert np.array_equal(got, ref), (s, sel[got != ref][:4])
        gotn = fp4.encode_values(-sel, s).astype(np.int64)
        assert np.array_equal(gotn, ref | 8), s
    # saturation and zero scale
    assert fp4.encode_values(np.array([1e6]), 1.0)[0] == 7
    assert fp4.encode_values(np.array([3.0, -3.0]), 0.0).tolist() == [0, 8]


def check_tie_table():
    """Ties of the E2M1 grid round to the even code: 0.25->0, 0.75->1, 1.25->1,
    1.75->2, 2.5->2, 3.5->4, 5->4 (nearest-even on the value set)."""
    r = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    got = fp4.E2M1_TABLE[fp4.encode_values(r, 1.0)]
    assert got.tolist() == want, got


def check_quantize_worked_row():
    """A hand-worked 32-channel row: group 0 starts [6, -3, 0.5, -0.1, 2.5, 7,
    -1.25, 0] and is zero after that; group 1 is all zeros (scale byte 0x00)."""
    row = np.zeros(32)
    row[:8] = [6.0, -3.0, 0.5, -0.1, 2.5, 7.0, -1.25, 0.0]
    codes, scales = fp4.quantize_rows(row[None, :])
    # scale: amax = 7, 7/6 = 1.1667; E4M3 neighbours 1.125 (0x39) and 1.25 (0x3A);
    # midpoint 1.1875 > 1.1667, so 1.125.
    assert scales.tolist() == [[0x39, 0x00]]
    # values / 1.125: 5.333->6 (7), 2.667->3 (5, neg: 0xD), 0.444->0.5 (1),
    # 0.0889->0 (neg: 8), 2.222->2 (4), 6.222->6 (7), 1.111->1 (2, neg: 0xA), 0->0 (0)
    want = [0x7 | (0xD << 4), 0x1 | (0x8 << 4), 0x4 | (0x7 << 4), 0xA | (0x0 << 4)] + [0] * 12
    assert codes[0].tolist() == want, [hex(c) for c in codes[0]]
    deq = fp4.dequantize_rows(codes, scales)[0]
    assert deq[:8].tolist() == [6.75, -3.375, 0.5625, -0.0, 2.25, 6.75, -1.125, 0.0]


def check_byte_accounting():
    """288 B per 512-channel row; about half of FP8 ([G], [N]) and about 4x
    smaller than 16-bit ([T]); pool and selection sizes as the pages state."""
    c = pages_constants()
    C = 512
    b = fp4.bytes_per_row(C)
    assert b == C * c["e2m1_bits"] / 8 + C / c["scale_group_channels"] * c["scale_bits"] / 8 == 288
    assert abs(b / C - c["fp4_over_fp8_approx"]) < 0.1            # 0.5625
    assert abs(2 * C / b - c["bf16_over_fp4_approx"]) < 0.5       # 3.56
    assert c["pool_blocks"] * c["block_tokens"] == c["pool_positions"] == c["pool_positions_approx"]
    assert indexer.BLOCK == c["block_tokens"]


# --------------------------------------------------- KV format variants ----

def all_bf16_finite():
    """Every finite bfloat16 value of either sign, as float64."""
    pos = np.arange(0x7F80, dtype=np.uint32)
    bits = np.concatenate([pos, pos | 0x8000]) << 16
    return bits.view(np.float32).astype(np.float64)


def check_fp8_encode_exhaustive():
    """E4M3FN codes of every finite bf16 value equal torch's round-to-nearest-even
    float8_e4m3fn cast wherever that cast is finite (|x| <= 464); beyond it the
    oracle saturates at 448 (torch returns NaN there)."""
    x = all_bf16_finite()
    got = kvformats.fp8_encode(x)
    inr = np.abs(x) <= 464.0
    ref = torch.from_numpy(x[inr].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got[inr] != ref)[0]
    assert bad.size == 0, (bad.size, x[inr][bad[:5]], got[inr][bad[:5]], ref[bad[:5]])
    out = ~inr
    assert (got[out] & 0x7F == 0x7E).all() and np.array_equal(got[out] >> 7, np.signbit(x[out]).astype(np.uint8))
    # decode of the encoding is the value itself wherever x is an E4M3 value
    vals = fp4.E4M3_TABLE[:127]
    assert np.array_equal(kvformats.fp8_dequantize_rows(kvformats.fp8_encode(vals)), vals)
    assert np.array_equal(kvformats.fp8_dequantize_rows(kvformats.fp8_encode(-vals)), -vals)


def check_fp8_worked_values():
    """Hand-worked E4M3FN codes: 1 -> 0x38; 448 and 500 -> 0x7E (saturation);
    -0 -> 0x80; 2^-9 -> 0x01 (smallest subnormal); 2^-10 -> 0x00 and
    3 * 2^-10 -> 0x02 (ties to the even code); 17 -> 0x58 (16, the even neighbour
    of the tie 16 | 18)."""
    x = np.array([1.0, 448.0, 500.0, -0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 17.0])
    assert kvformats.fp8_encode(x).tolist() == [0x38, 0x7E, 0x7E, 0x80, 0x01, 0x00, 0x02, 0x58]


def _bf16_floor_log2(bits):
    """floor(log2 v) of a positive finite bf16 value from its bit fields."""
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e > 0:
        return int(e) - 127
    return -133 + int(m).bit_length() - 1          # subnormal: v = m * 2^-133


def check_mx_shared_exponent_exhaustive():
    """The MX shared exponent of every positive finite bf16 amax equals
    floor(log2 amax) - 2 read off the bf16 exponent field (subnormals from the
    leading mantissa bit), clamped to [-127, 127]; 0 gives -127."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    a = (bits << 16).view(np.float32).astype(np.float64)
    got = kvformats.mx_shared_exponent(a)
    ref = np.array([min(max(_bf16_floor_log2(int(b)) - 2, -127), 127) for b in bits])
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:5]
    assert kvformats.mx_shared_exponent(np.array([0.0]))[0] == -127
    assert kvformats.E8M0_TABLE[0] == 2.0 ** -127 and kvformats.E8M0_TABLE[254] == 2.0 ** 127
    assert math.isnan(kvformats.E8M0_TABLE[255])


def _mxfp4_bruteforce(block):
    """MXFP4 of one 32-value block with exact rationals: X = 2^(floor(log2 amax) - 2),
    then per value the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} to |x| / X (ties to
    the even code), sign bit from x."""
    from fractions import Fraction
    fr = [Fraction(float(v)) for v in block]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        e = -127
    else:
        e = amax.numerator.bit_length() - amax.denominator.bit_length()
        if Fraction(2) ** e > amax:
            e -= 1                                     # floor(log2 amax)
        e = min(max(e - 2, -127), 127)
    X = Fraction(2) ** e
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    codes = []
    for v, f in zip(block, fr):
        r = abs(f) / X
        d = [abs(r - g) for g in grid]
        best = min(d)
        cand = [i for i, di in enumerate(d) if di == best]
        mag = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        codes.append((8 if math.copysign(1.0, float(v)) < 0 else 0) | mag)
    return codes, e + 127


def check_mxfp4_bruteforce():
    """MXFP4 rows (normal data with outliers, exact grid points and midpoints,
    values saturating in [6, 8) * 2^e, subnormal and all-zero blocks) equal the
    exact-rational brute force block by block."""
    rng = np.random.default_rng(7)
    rows = []
    for kind in range(6):
        for _ in range(4):
            if kind == 0:
                r = rng.standard_normal(64) * np.where(rng.random(64) < 0.05, 20.0, 1.0)
            elif kind == 1:                      # grid points and midpoints times one power of two
                e = int(rng.integers(-20, 20))
                r = rng.choice([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], 64) * 2.0 ** e
                r[0] = 6 * 2.0 ** e
                r *= rng.choice([-1.0, 1.0], 64)
            elif kind == 2:                      # saturation: amax in [6, 8) * 2^e
                r = rng.uniform(-8, 8, 64) * 2.0 ** int(rng.integers(-5, 5))
            elif kind == 3:                      # bf16 subnormals and tiny values
                r = rng.standard_normal(64) * 2.0 ** -130
            elif kind == 4:
                r = np.zeros(64)
                r[rng.integers(0, 64)] = -0.0
            else:                                # huge values near the bf16 maximum
                r = rng.standard_normal(64) * 2.0 ** 120
            rows.append(r)
    x = torch.tensor(np.array(rows), dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = kvformats.mxfp4_quantize_rows(x)
    for i in range(x.shape[0]):
        for g in range(2):
            bc, bs = _mxfp4_bruteforce(x[i, 32 * g:32 * g + 32])
            got = []
            for j in range(16):
                byte = int(codes[i, 16 * g + j])
                got += [byte & 0xF, byte >> 4]
            assert got == bc and int(scales[i, g]) == bs, (i, g)


def check_mxfp4_roundtrip():
    """Blocks of exact MXFP4 values (E2M1 values times 2^e, with one of magnitude
    4 * 2^e or 6 * 2^e fixing the shared exponent at e) decode to themselves."""
    rng = np.random.default_rng(11)
    for e in (-127, -60, -3, 0, 5, 60, 125):
        v = rng.choice(fp4.E2M1_TABLE[:16], (3, 32)) * 2.0 ** e
        v[:, 0] = rng.choice([4.0, 6.0, -4.0, -6.0], 3) * 2.0 ** e
        codes, scales = kvformats.mxfp4_quantize_rows(v)
        assert (scales == e + 127).all(), e
        assert np.array_equal(kvformats.mxfp4_dequantize_rows(codes, scales), v), e


def check_kv_format_bytes():
    """Bytes per 512-channel row: FP4 with E4M3 per 16 = 288, MXFP4 = 256 + 16 =
    272, FP8 = 512. FP4 is 0.5625 of FP8, which the pages round to a half."""
    c = pages_constants()
    C = 512
    b = [kvformats.bytes_per_row(f, C) for f in (kvformats.FMT_FP4, kvformats.FMT_MXFP4, kvformats.FMT_FP8)]
    assert b == [288, 272, 512] and b[0] == fp4.bytes_per_row(C)
    assert abs(b[0] / b[2] - c["fp4_over_fp8_approx"]) < 0.1


# ------------------------------------------------- paged cache and ring ----

def check_paged_worked_example():
    """Hand-worked mapping with pages of 4 rows: sequence 1's block table
    [5, 2, -1]; position 6 is page 1 (physical page 2), offset 2 -> row 10;
    position 3 -> page 5 -> row 23; position 9 is page 2, which maps nowhere;
    a page id past n_pages (7 >= 6) maps nowhere too."""
    bt = np.array([[0, 1, 3], [5, 2, -1], [7, 4, 4]])
    assert paged.physical_row(bt, 4, 6, 1, 6) == 10
    assert paged.physical_row(bt, 4, 6, 1, 3) == 23
    assert paged.physical_row(bt, 4, 6, 1, 9) == -1
    assert paged.physical_row(bt, 4, 6, 2, 1) == -1
    assert paged.physical_row(bt, 4, 6, 0, 12) == -1          # past the table
    assert paged.physical_row(bt, 4, 6, 0, -1) == -1


def check_paged_round_trip():
    """With a random permutation of physical pages as the block tables, every
    position of every sequence has its own physical row, and reading a sequence
    back through the table gives its rows in order (the storage is transparent)."""
    rng = np.random.default_rng(3)
    page, lengths = 64, [130, 64, 1, 300]
    need = [-(-n // page) for n in lengths]
    perm = rng.permutation(sum(need) + 3)
    bt = np.full((len(lengths), max(need)), -1)
    k = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[k:k + n]; k += n
    n_pages = sum(need) + 3
    rows = [rng.integers(-100, 100, (n, 5)) for n in lengths]
    store = paged.paged_store(rows, bt, page, n_pages, fill=12345)
    seen = set()
    for s, n in enumerate(lengths):
        phys = [paged.physical_row(bt, page, n_pages, s, t) for t in range(n)]
        assert min(phys) >= 0 and not (seen & set(phys)); seen |= set(phys)
        assert np.array_equal(paged.logical_rows(store, bt, page, n_pages, s, np.arange(n)), rows[s])
    assert (store == 12345).all(axis=1).sum() == n_pages * page - sum(lengths)


def check_ring_window():
    """After appending positions 0..p in order, the ring read for position p gives
    exactly the last min(W, p+1) rows, oldest first, for p below, at and far past W."""
    # the layout itself (the library's ring buffers follow it): position t in slot t mod W
    assert [paged.ring_slot(t, 128) for t in (0, 127, 128, 130, 1000)] == [0, 127, 0, 2, 104]
    rng = np.random.default_rng(4)
    W = 8
    for n in (1, 5, 8, 9, 30):
        rows = rng.integers(0, 1000, (n, 3))
        ring = paged.ring_after_appends(rows, W)
        got = paged.window_from_ring(ring, n - 1, W)
        assert np.array_equal(got, rows[max(0, n - W):n]), n


# -------------------------------------------------------------- indexer ----

def check_scores_worked_example():
    """Two heads, three dims, three tokens, by hand.

    q0 = [1, 2, -1], q1 = [-2, 0, 3], w = [2, 5]
    k0 = [1, 1, 1]:  q0.k0 = 2,  q1.k0 = 1   -> 2*2 + 5*1 = 9
    k1 = [3, -1, 2]: q0.k1 = -1, q1.k1 = 0   -> 0 + 0     = 0
    k2 = [0, -2, 4]: q0.k2 = -8, q1.k2 = 12  -> 0 + 5*12  = 60
    """
    q = np.array([[1, 2, -1], [-2, 0, 3]], dtype=float)
    w = np.array([2.0, 5.0])
    k = np.array([[1, 1, 1], [3, -1, 2], [0, -2, 4]], dtype=float)
    assert indexer.token_scores(q, w, k).tolist() == [9.0, 0.0, 60.0]


def check_scores_closed_forms():
    """Unit queries pick out one coordinate; ReLU clips the negative half; the
    weights scale linearly; heads add."""
    rng = np.random.default_rng(5)
    k = rng.integers(-8, 9, size=(40, 6)).astype(float)
    for d in range(6):
        e = np.zeros((1, 6)); e[0, d] = 1.0
        assert np.array_equal(indexer.token_scores(e, np.array([1.0]), k), np.maximum(k[:, d], 0))
        assert np.array_equal(indexer.token_scores(-e, np.array([3.0]), k), 3 * np.maximum(-k[:, d], 0))
    q = rng.integers(-8, 9, size=(4, 6)).astype(float)
    w = rng.integers(1, 9, size=4).astype(float)
    whole = indexer.token_scores(q, w, k)
    parts = sum(indexer.token_scores(q[h:h + 1], w[h:h + 1], k) for h in range(4))
    assert np.array_equal(whole, parts)
    assert np.array_equal(indexer.token_scores(q, 2 * w, k), 2 * whole)


def check_scores_bruteforce():
    """Pure-Python integer loops on tiny random inputs."""
    rng = np.random.default_rng(6)
    for _ in range(20):
        H, D, n = rng.integers(1, 5), rng.integers(1, 9), rng.integers(1, 12)
        q = rng.integers(-8, 9, size=(H, D)); w = rng.integers(1, 9, size=H)
        k = rng.integers(-8, 9, size=(n, D))
        ref = []
        for t in range(n):
            tot = 0
            for h in range(H):
                dot = 0
                for d in range(D):
                    dot += int(q[h, d]) * int(k[t, d])
                tot += int(w[h]) * (dot if dot > 0 else 0)
            ref.append(float(tot))
        assert indexer.token_scores(q, w, k).tolist() == ref


def check_block_maxima():
    """Ramps: increasing scores put the max at each block's last visible
    position, decreasing at its first; a partial last block uses what exists."""
    for n in (1, 7, 8, 9, 23, 64):
        up = np.arange(n, dtype=float)
        assert indexer.block_maxima(up).tolist() == [float(min(8 * b + 7, n - 1)) for b in range(-(-n // 8))]
        down = -up
        assert indexer.block_maxima(down).tolist() == [-8.0 * b for b in range(-(-n // 8))]


def _dominance_ok(keys, ids, chosen, count):
    chosen = list(chosen)
    assert chosen == sorted(chosen) and len(set(chosen)) == len(chosen)
    assert len(chosen) == min(count, len(ids))
    rank = {i: (-k, i) for k, i in zip(keys, ids)}
    inside = set(chosen)
    for a in inside:
        for b in ids:
            if b not in inside:
                assert rank[a] < rank[b], (a, b)


def check_select_top_bruteforce():
    """Selection: every chosen id outranks every other id under (key desc, id
    asc); the count is min(count, n); the output is ascending."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 14))
        keys = rng.integers(0, 4, size=n).astype(float)    # many ties
        ids = rng.permutation(50)[:n]
        count = int(rng.integers(1, n + 3))
        _dominance_ok(keys.tolist(), ids.tolist(), indexer.select_top(keys, ids, count).tolist(), count)
    # exhaustive on a 6-element tie-heavy case: the chosen set is the best of all subsets
    keys = np.array([2.0, 5.0, 5.0, 1.0, 5.0, 2.0]); ids = np.arange(6)
    for count in range(1, 7):
        best = min(itertools.combinations(ids.tolist(), count),
                   key=lambda s: sorted((-keys[i], i) for i in s))
        assert indexer.select_top(keys, ids, count).tolist() == sorted(best)


def _global_top(s, k):
    order = sorted(range(len(s)), key=lambda t: (-s[t], t))
    return sorted(order[:k])


def check_hierarchy_invariant():
    """With P >= k, the top-k through the block pool equals the top-k of all
    visible tokens (each block ranked ahead of a chosen token's block holds a
    distinct token ranked ahead of it)."""
    rng = np.random.default_rng(8)
    for _ in range(200):
        n = int(rng.integers(1, 120)); H, D = 2, 3
        q = rng.integers(-2, 3, size=(H, D)).astype(float); w = rng.integers(1, 3, size=H).astype(float)
        k = rng.integers(-2, 3, size=(n, D)).astype(float)
        kk = int(rng.integers(1, 12)); P = int(rng.integers(kk, 16))
        pool, idx, s = indexer.index_full(q, w, k, n - 1, P, kk)
        assert idx.tolist() == _global_top(s.tolist(), min(kk, n))
        assert pool.tolist() == sorted(pool.tolist()) and len(pool) == min(P, -(-n // 8))


def check_pool_worked_example():
    """Blocks of 8, P = 2, k = 3, by hand. Scores for 20 tokens (3 blocks, the
    last partial with 4 visible tokens):
      block 0: [1,9,1,1,1,1,1,1]  max 9
      block 1: [9,0,0,0,0,0,0,8]  max 9   (ties block 0; lower id wins order)
      block 2: [3,4,20,5]         max 20
    Pool = top-2 blocks by (max desc, id asc) = {2, 0}; candidates are
    positions 0..7 and 16..19; top-3 = 18 (20), 1 (9), 19 (5) -> [1, 18, 19].
    Position 8 (score 9, block 1) is outside the pool and is not chosen."""
    s = np.array([1, 9, 1, 1, 1, 1, 1, 1, 9, 0, 0, 0, 0, 0, 0, 8, 3, 4, 20, 5], dtype=float)
    m = indexer.block_maxima(s)
    assert m.tolist() == [9.0, 9.0, 20.0]
    pool = indexer.select_top(m, np.arange(3), 2)
    assert pool.tolist() == [0, 2]
    cand = indexer.pool_positions(pool, 20)
    assert cand.tolist() == list(range(8)) + [16, 17, 18, 19]
    assert indexer.select_top(s[cand], cand, 3).tolist() == [1, 18, 19]


def check_causal_visibility():
    """Only positions 0..q_pos are visible: a planted top-scoring key at q_pos+1
    is never chosen, nor is its block pooled; the partial last block holds
    exactly the visible positions; a key planted at q_pos itself is chosen."""
    rng = np.random.default_rng(9)
    q = rng.integers(-8, 9, size=(4, 16)).astype(float); w = np.ones(4)
    k = rng.integers(-8, 9, size=(100, 16)).astype(float)
    top = np.where(q[0] >= 0, 8.0, -8.0)
    for q_pos in (84, 87, 95):
        kp = k.copy(); kp[q_pos + 1] = top
        pool, idx, s = indexer.index_full(q, w, kp, q_pos, 4, 6)
        assert s.shape[0] == q_pos + 1 and idx.max() <= q_pos
        assert not ((q_pos + 1) // 8 in pool.tolist() and (q_pos + 1) % 8 == 0)
        kp[q_pos] = top
        pool, idx, s = indexer.index_full(q, w, kp, q_pos, 4, 6)
        assert q_pos in idx.tolist()
    assert indexer.pool_positions(np.array([10]), 85).tolist() == [80, 81, 82, 83, 84]


def check_empty_query():
    """A query that sees no token (position -1, e.g. an empty context slot):
    no scores, an empty pool and selection, and attention over no row at all
    is the empty sum: output 0, log-sum-exp -inf (no NaN)."""
    rng = np.random.default_rng(19)
    q = rng.integers(-8, 9, size=(4, 16)).astype(float); w = np.ones(4)
    k = rng.integers(-8, 9, size=(40, 16)).astype(float)
    pool, idx, s = indexer.index_full(q, w, k, -1, 4, 6)
    assert s.shape[0] == 0 and pool.size == 0 and idx.size == 0
    assert indexer.index_reindex(q, w, lambda pos: k[pos], np.array([0, 1]), -1, 6).size == 0
    Q = rng.standard_normal((3, 16)); none = np.zeros((0, 16))
    out, lse = attention.attend(Q, none, none, none, 0.25)
    assert out.shape == (3, 16) and (out == 0).all() and np.isneginf(lse).all()


def check_cover_all():
    """When the pool covers every block and k covers every token, every
    visible position is selected."""
    rng = np.random.default_rng(10)
    k = rng.integers(-8, 9, size=(37, 8)).astype(float)
    q = rng.integers(-8, 9, size=(2, 8)).astype(float)
    pool, idx, _ = indexer.index_full(q, np.ones(2), k, 36, 5, 64)
    assert pool.tolist() == [0, 1, 2, 3, 4] and idx.tolist() == list(range(37))


def check_reindex():
    """Reindex with the Full layer's own (q, w) returns the Full indices; its
    indices lie in the pool; a planted top key outside the pool is never chosen."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        n = int(rng.integers(20, 200))
        q = rng.integers(-4, 5, size=(3, 8)).astype(float); w = rng.integers(1, 5, size=3).astype(float)
        k = rng.integers(-4, 5, size=(n, 8)).astype(float)
        pool, idx, _ = indexer.index_full(q, w, k, n - 1, 4, 5)
        same = indexer.index_reindex(q, w, lambda p: k[p], pool, n - 1, 5)
        assert same.tolist() == idx.tolist()
        q2 = rng.integers(-4, 5, size=(3, 8)).astype(float)
        outside = [t for t in range(n) if t // 8 not in set(pool.tolist())]
        k2 = k.copy()
        if outside:
            k2[outside[0]] = 4 * np.where(q2[0] >= 0, 1, -1)
        r = indexer.index_reindex(q2, w, lambda p: k2[p], pool, n - 1, 5)
        allowed = set(indexer.pool_positions(pool, n).tolist())
        assert set(r.tolist()) <= allowed
        if outside:
            assert outside[0] not in set(r.tolist())


# ------------------------------------------------------------ attention ----

def check_branch_vs_scipy():
    """Softmax and log-sum-exp of one branch equal scipy's routines."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((5, 32)); kv = rng.standard_normal((17, 32)); v = rng.standard_normal((17, 32))
    o, lse = attention.branch(q, kv, v, 0.3)
    logits = 0.3 * q @ kv.T
    assert np.allclose(lse, scipy.special.logsumexp(logits, axis=1), rtol=0, atol=1e-12)
    assert np.allclose(o, scipy.special.softmax(logits, axis=1) @ v, rtol=0, atol=1e-12)


def check_dense_equivalence():
    """Both branches merged equal one softmax attention over the concatenated
    keys/values (torch scaled_dot_product_attention in float64); with K = V in
    the sparse branch."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((8, 64)); rows = rng.standard_normal((30, 64))
    wk = rng.standard_normal((12, 64)); wv = rng.standard_normal((12, 64))
    scale = 1 / math.sqrt(64)
    out, lse = attention.attend(q, rows, wk, wv, scale)
    K = torch.from_numpy(np.concatenate([rows, wk]))[None]
    V = torch.from_numpy(np.concatenate([rows, wv]))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None], K, V, scale=scale)[0]
    assert np.allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(scale * q @ K[0].numpy().T, axis=1), atol=1e-12)


def check_attention_special_cases():
    """One row gives that row; equal logits give the mean; row order does not matter."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, 16)); r = rng.standard_normal((1, 16))
    o, lse = attention.branch(q, r, r, 0.5)
    assert np.allclose(o, np.repeat(r, 3, axis=0), atol=1e-15) and np.allclose(lse, 0.5 * q @ r[0])
    v = rng.standard_normal((9, 16))
    o, _ = attention.branch(np.zeros((2, 16)), rng.standard_normal((9, 16)), v, 1.0)
    assert np.allclose(o, v.mean(axis=0)[None].repeat(2, 0), atol=1e-15)
    rows = rng.standard_normal((11, 16)); perm = rng.permutation(11)
    a = attention.attend(q, rows, rows[:4], rows[4:8], 0.2)[0]
    b = attention.attend(q, rows[perm], rows[:4], rows[4:8], 0.2)[0]
    assert np.allclose(a, b, atol=1e-13)


def check_merge_asymmetric():
    """Merging a branch with a much heavier one is dominated by the heavier,
    and merging with an empty branch (lse = -inf) returns the other branch."""
    o1 = np.ones((2, 3)); o2 = 2 * np.ones((2, 3))
    out, lse = attention.merge(o1, np.array([0.0, 0.0]), o2, np.array([math.log(3.0), -np.inf]))
    assert np.allclose(out[0], 0.25 * 1 + 0.75 * 2) and np.allclose(out[1], 1.0)
    assert np.allclose(lse, [math.log(4.0), 0.0])


# ---------------------------------------------------------------- chain ----

def check_schedule():
    """The decoder schedule on the page: Full, then Reindex layers rescoring
    the Full layer's pool, Reuse layers copying the nearest Full/Reindex
    indices; the encoder groups each start with their own Full layer."""
    codes = {"F": chain.FULL, "I": chain.REINDEX, "R": chain.REUSE}
    for part in ("decoder", "encoder"):
        modes = [codes[c] for kind, g in golden_lines("csa2_schedule.txt") if kind == part for c in g]
        calls = []

        def full_fn(layer):
            calls.append(("F", layer))
            return np.array([layer]), np.array([100 + layer])

        def reindex_fn(layer, pool):
            calls.append(("I", layer, int(pool[0])))
            return np.array([200 + layer])

        res = chain.layer_indices(modes, full_fn, reindex_fn)
        last_full = last_sel = None
        for layer, mode in enumerate(modes):
            if mode == chain.FULL:
                last_full = layer; last_sel = 100 + layer
            elif mode == chain.REINDEX:
                assert ("I", layer, last_full) in calls
                last_sel = 200 + layer
            assert int(res[layer][1][0]) == last_sel, (part, layer)
            assert int(res[layer][0][0]) == last_full
        assert len(calls) == sum(m != chain.REUSE for m in modes)
    assert len(modes) == 18


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
