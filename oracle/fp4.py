"""FP4 main-KV codec: E2M1 values, an E4M3 scale per 16-channel group.

Follows [G] "FP4 main KV" paragraph and [N] "FP4 KV Quantization and Cache
Lifetime Management": main KV is E2M1 scaled by an E4M3 factor for every 16-channel group, the
NVFP4 layout without its second-level (global) scale. ([T] "Mechanism 3" calls
it MXFP4; two pages agree on E4M3 per 16, which is the reading taken.)

Storage per row of C channels: C/2 code bytes (channel 2j in the low nibble of
byte j, channel 2j+1 in the high nibble) and C/16 scale bytes.

Everything here is exact: decoded values have at most 5 significant bits, and
every comparison is between |x| (8 significant bits, bfloat16) and products of
at most 7 significant bits, all exact in float64.
"""
from __future__ import annotations

import numpy as np

GROUP = 16          # channels per E4M3 scale
SCALE_DIVISOR = 6.0  # the largest E2M1 magnitude: scale = amax / 6 before rounding


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                       # subnormal: 2^(1-1) * (m / 2)
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3FN code: 1 sign, 4 exponent bits (bias 7), 3 mantissa
    bits, no infinities; exponent 15 with mantissa 7 is NaN."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * 2.0 ** -6 * (m / 8.0)
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite E4M3 values, indexed by their code 0x00..0x7E (ascending).
_E4M3_POS = E4M3_TABLE[:127]
# Non-negative E2M1 magnitudes, indexed by their 3-bit code (ascending).
_E2M1_POS = E2M1_TABLE[:8]


def _nearest_even(dist: np.ndarray) -> np.ndarray:
    """Index of the smallest distance along the last axis; on a tie, the even index.

    The candidates are strictly increasing values indexed by consecutive codes,
    so at most two neighbours can tie, and exactly one of them is even.
    """
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    first = np.argmax(tied, axis=-1)
    nxt = np.minimum(first + 1, dist.shape[-1] - 1)
    next_ties = np.take_along_axis(tied, nxt[..., None], axis=-1)[..., 0] & (nxt != first)
    return np.where((first % 2 == 1) & next_ties, nxt, first)


def encode_scale(amax: np.ndarray) -> np.ndarray:
    """E4M3 code of the value nearest amax/6 (ties to the even code).

    Out-of-range values take the nearest finite value, i.e. saturate at 448;
    values at or below 2^-10 round to code 0. Compared as |amax - 6 v|. Above
    6*448 the nearest value is 448 whatever amax is, so amax is first clamped
    there; after that every difference is exact in float64 (a huge amax would
    otherwise swamp the small differences between candidates).
    """
    a = np.minimum(np.asarray(amax, dtype=np.float64), SCALE_DIVISOR * _E4M3_POS[-1])
    dist = np.abs(a[..., None] - SCALE_DIVISOR * _E4M3_POS)
    return _nearest_even(dist).astype(np.uint8)


def encode_values(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """4-bit codes of x given the decoded scale of its group (broadcastable).

    Magnitude: the E2M1 value m nearest |x|/scale (ties to the even code,
    saturating at 6), compared as ||x| - scale*m|. Above 6*scale the nearest
    value is 6, so |x| is first clamped there, which keeps every difference
    exact in float64. A zero scale gives magnitude code 0. Sign bit: the sign
    bit of x.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(scale, dtype=np.float64), x.shape)
    ax = np.minimum(np.abs(x), s * _E2M1_POS[-1])
    dist = np.abs(ax[..., None] - s[..., None] * _E2M1_POS)
    mag = _nearest_even(dist)
    mag = np.where(s == 0.0, 0, mag)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 3) | mag).astype(np.uint8)


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows x [R, C] (exact bfloat16 values as float64).

    Returns (codes uint8 [R, C/2], scales uint8 [R, C/16]).
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    assert C % GROUP == 0 and C % 2 == 0
    g = x.reshape(R, C // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    scode = encode_scale(amax)                       # [R, G]
    sval = E4M3_TABLE[scode]                         # [R, G]
    codes = encode_values(g, sval[..., None]).reshape(R, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scode


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode (codes [R, C/2], scales [R, C/16]) to float64 values [R, C]."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, half = codes.shape
    C = 2 * half
    nib = np.empty((R, C), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    s = np.repeat(E4M3_TABLE[np.asarray(scales, dtype=np.uint8)], GROUP, axis=1)
    return E2M1_TABLE[nib] * s


def bytes_per_row(C: int) -> int:
    """Main-KV bytes per token and source layer: C/2 code bytes + C/16 scale bytes."""
    return C // 2 + C // GROUP
