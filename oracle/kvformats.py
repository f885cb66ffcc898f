"""Main-KV format variants beside the FP4 codec with E4M3 scales per 16 channels.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this module; the product path never does.

Two readings the pages leave open are built as variants of the main-KV cache:

* MXFP4. [T] "Mechanism 3" calls the 4-bit KV format MXFP4, which in the OCP
  Microscaling format means E2M1 values sharing one power-of-two (E8M0) scale
  per 32 values. Per block: amax = max |x|; the shared exponent is
  floor(log2(amax)) - 2 (2 is the exponent of the largest E2M1 value, 6), clamped
  to [-127, 127], and -127 for an all-zero block; the scale byte is that
  exponent + 127. Each value is the E2M1 code nearest x / 2^e, ties to the even
  code, saturating at 6 (values in [6, 8) * 2^e saturate, as the format allows).
  Storage per row: C/2 code bytes (same nibble order as the FP4 codec) and C/32
  scale bytes.
* FP8. [G] "FP4 main KV" and [N] "FP4 KV Quantization and Cache Lifetime
  Management" say the FP4 cache takes roughly half the bytes of an FP8 one; the
  FP8 layout is not described. The plainest reading is taken: each value an
  E4M3FN code (the nearest finite value, ties to the even code, saturating at
  448; the sign bit is the sign bit of x), no scale, C bytes per row.

Everything is exact in float64: inputs are bfloat16 values, scales are powers of
two or absent, and the candidate grids have at most 4 significant bits.
"""
from __future__ import annotations

import numpy as np

from oracle import fp4

FMT_FP4 = 0       # E2M1 + an E4M3 scale for each 16-channel group (oracle/fp4.py)
FMT_MXFP4 = 1     # E2M1 + one E8M0 scale per 32 channels
FMT_FP8 = 2       # E4M3FN per value, no scale

MX_GROUP = 32
MX_ELEM_EMAX = 2          # the largest E2M1 value is 1.5 * 2^2
E8M0_BIAS = 127


def e8m0_value(code: int) -> float:
    """Value of an E8M0 scale code: 2^(code - 127); code 255 is NaN."""
    if code == 255:
        return float("nan")
    return 2.0 ** (int(code) - E8M0_BIAS)


E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def mx_shared_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 where amax is 0.

    np.frexp writes amax = m * 2^e with m in [0.5, 1), so floor(log2(amax)) = e - 1
    exactly, for normal and subnormal inputs alike.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)
    shared = (e.astype(np.int64) - 1) - MX_ELEM_EMAX
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    return np.where(a == 0.0, -E8M0_BIAS, shared)


def mxfp4_quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows x [R, C] (exact bfloat16 values as float64) to MXFP4.

    Returns (codes uint8 [R, C/2], scales uint8 [R, C/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    assert C % MX_GROUP == 0
    g = x.reshape(R, C // MX_GROUP, MX_GROUP)
    shared = mx_shared_exponent(np.abs(g).max(axis=2))            # [R, G]
    scale = np.ldexp(1.0, shared)                                  # exact powers of two
    codes = fp4.encode_values(g, scale[..., None]).reshape(R, C)   # nearest E2M1 of x / 2^e
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (shared + E8M0_BIAS).astype(np.uint8)


def mxfp4_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 (codes [R, C/2], scales [R, C/32]) to float64 values [R, C]."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, half = codes.shape
    C = 2 * half
    nib = np.empty((R, C), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    s = np.repeat(E8M0_TABLE[np.asarray(scales, dtype=np.uint8)], MX_GROUP, axis=1)
    return fp4.E2M1_TABLE[nib] * s


def fp8_encode(x: np.ndarray) -> np.ndarray:
    """E4M3FN code of each x: nearest finite value (ties to the even code,
    saturating at 448), sign bit = sign bit of x. |x| is clamped to 448 first
    (above it the nearest finite value is 448 whatever |x| is), which keeps every
    compared difference exact in float64."""
    x = np.asarray(x, dtype=np.float64)
    pos = fp4.E4M3_TABLE[:127]                         # codes 0x00..0x7E, ascending
    ax = np.minimum(np.abs(x), pos[-1])
    mag = fp4._nearest_even(np.abs(ax[..., None] - pos))
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 7) | mag).astype(np.uint8)


def fp8_quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows x [R, C] to E4M3FN codes [R, C]; the scale plane is empty [R, 0]."""
    x = np.asarray(x, dtype=np.float64)
    return fp8_encode(x), np.zeros((x.shape[0], 0), dtype=np.uint8)


def fp8_dequantize_rows(codes: np.ndarray, scales: np.ndarray | None = None) -> np.ndarray:
    """Decode E4M3FN codes [R, C] to float64 values."""
    return fp4.E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize_rows(fmt: int, x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    if fmt == FMT_FP4:
        return fp4.quantize_rows(x)
    if fmt == FMT_MXFP4:
        return mxfp4_quantize_rows(x)
    if fmt == FMT_FP8:
        return fp8_quantize_rows(x)
    raise ValueError(fmt)


def dequantize_rows(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    if fmt == FMT_FP4:
        return fp4.dequantize_rows(codes, scales)
    if fmt == FMT_MXFP4:
        return mxfp4_dequantize_rows(codes, scales)
    if fmt == FMT_FP8:
        return fp8_dequantize_rows(codes)
    raise ValueError(fmt)


def code_bytes(fmt: int, C: int) -> int:
    return C if fmt == FMT_FP8 else C // 2


def scale_bytes(fmt: int, C: int) -> int:
    return {FMT_FP4: C // fp4.GROUP, FMT_MXFP4: C // MX_GROUP, FMT_FP8: 0}[fmt]


def bytes_per_row(fmt: int, C: int) -> int:
    """Main-KV bytes per token and source layer."""
    return code_bytes(fmt, C) + scale_bytes(fmt, C)
