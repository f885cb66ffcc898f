"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers. It holds none of the method's arithmetic:
no quantisation, no scoring, no selection, no attention.

Every value is a pure function of (seed, stream name, element counter), built
from a 32-bit integer mixing function evaluated with int64 torch ops. All
products stay below 2**63, so the same code gives bit-identical results on the
CPU and on a GPU. That lets the oracle regenerate any subset of a tensor (for
example the 512 rows one query selects out of a 1M-row context) without
materialising the rest.

Distributions:
  * uniform integers in [lo, hi]: lo + floor(u * n / 2**32), n = hi - lo + 1;
  * standard normal: a 65,536-entry inverse-CDF table of float32 quantiles at
    (j + 0.5) / 65536, indexed by the top 16 bits of u;
  * outliers: an independent Bernoulli(0.01) stream; selected values are
    multiplied by 20 in float32 before rounding;
  * bfloat16: float32 rounded to nearest-even by integer bit operations.
"""
from __future__ import annotations

import zlib

import numpy as np
import torch

MASK32 = 0xFFFFFFFF
_OUTLIER_THRESHOLD = 42949673  # round(0.01 * 2**32)


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """32-bit avalanche mixer (xorshift-multiply, two odd constants < 2**31)."""
    x = x ^ (x >> 16)
    x = (x * 0x21F0AAAD) & MASK32
    x = x ^ (x >> 15)
    x = (x * 0x735A2D97) & MASK32
    x = x ^ (x >> 15)
    return x


def _mix32_int(x: int) -> int:
    x &= MASK32
    x ^= x >> 16
    x = (x * 0x21F0AAAD) & MASK32
    x ^= x >> 15
    x = (x * 0x735A2D97) & MASK32
    x ^= x >> 15
    return x


def stream_key(seed: int, name: str) -> tuple[int, int]:
    """Two 32-bit keys for the stream `name` under `seed`."""
    a = _mix32_int(_mix32_int(seed ^ 0x5BD1E995) ^ zlib.crc32(name.encode()))
    b = _mix32_int(a ^ 0x1B873593)
    return a, b


def uniform_u32(seed: int, name: str, counters: torch.Tensor) -> torch.Tensor:
    """u32 (held in int64) for each non-negative int64 counter."""
    ka, kb = stream_key(seed, name)
    lo = counters & MASK32
    hi = counters >> 32
    return _mix32(_mix32(lo ^ ka) ^ _mix32(hi ^ kb))


def randint(seed: int, name: str, counters: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    n = hi - lo + 1
    assert 0 < n < 2**31
    return lo + ((uniform_u32(seed, name, counters) * n) >> 32)


_TABLES: dict = {}


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    if key not in _TABLES:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLES[key] = torch.from_numpy(ndtri(p).astype(np.float32)).to(device)
    return _TABLES[key]


def normal_f32(seed: int, name: str, counters: torch.Tensor, outliers: bool) -> torch.Tensor:
    u = uniform_u32(seed, name, counters)
    z = _normal_table(counters.device)[u >> 16]
    if outliers:
        o = uniform_u32(seed, name + "/outlier", counters) < _OUTLIER_THRESHOLD
        z = torch.where(o, z * 20.0, z)
    return z


def f32_to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round finite float32 to bfloat16 (nearest, ties to even); returns int64 bit patterns."""
    b = x.contiguous().view(torch.int32).to(torch.int64) & MASK32
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF


def bits_to_bf16(bits: torch.Tensor) -> torch.Tensor:
    return bits.to(torch.int32).to(torch.int16).view(torch.bfloat16)


def bf16_to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bfloat16 tensor, as numpy."""
    return x.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def _counters(base: int, shape, device) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= s
    return (base + torch.arange(n, dtype=torch.int64, device=device)).reshape(shape)


# ---- named tensors --------------------------------------------------------
# Counter layout: (entity << 40) | element-within-entity, so any row can be
# regenerated on its own. An entity is a sequence, or a (layer, query) pair.

ENTITY_SHIFT = 40


def int_tensor_bf16(seed, name, entity, shape, lo, hi, device="cpu", offset=0):
    """Integers in [lo, hi] stored as bfloat16, for element offsets offset.. of an entity."""
    c = _counters((entity << ENTITY_SHIFT) + offset, shape, device)
    return randint(seed, name, c, lo, hi).to(torch.float32).to(torch.bfloat16)


def int_tensor_f32(seed, name, entity, shape, lo, hi, device="cpu", offset=0):
    c = _counters((entity << ENTITY_SHIFT) + offset, shape, device)
    return randint(seed, name, c, lo, hi).to(torch.float32)


def normal_bf16(seed, name, entity, shape, outliers, device="cpu", offset=0):
    c = _counters((entity << ENTITY_SHIFT) + offset, shape, device)
    return bits_to_bf16(f32_to_bf16_bits(normal_f32(seed, name, c, outliers)))


def normal_bf16_rows(seed, name, entity, rows: torch.Tensor, width: int, outliers: bool):
    """Rows `rows` (int64, any device) of a [*, width] normal bf16 tensor of one entity."""
    c = (entity << ENTITY_SHIFT) + rows.to(torch.int64)[:, None] * width + torch.arange(
        width, dtype=torch.int64, device=rows.device)[None, :]
    return bits_to_bf16(f32_to_bf16_bits(normal_f32(seed, name, c, outliers)))


def int_bf16_rows(seed, name, entity, rows: torch.Tensor, width: int, lo: int, hi: int):
    c = (entity << ENTITY_SHIFT) + rows.to(torch.int64)[:, None] * width + torch.arange(
        width, dtype=torch.int64, device=rows.device)[None, :]
    return randint(seed, name, c, lo, hi).to(torch.float32).to(torch.bfloat16)


def bernoulli_rows(seed, name, entity, rows: torch.Tensor, width: int, threshold_u32: int):
    c = (entity << ENTITY_SHIFT) + rows.to(torch.int64)[:, None] * width + torch.arange(
        width, dtype=torch.int64, device=rows.device)[None, :]
    return uniform_u32(seed, name, c) < threshold_u32


def uniform_f64_host(seed: int, name: str, n: int) -> np.ndarray:
    """n uniforms in (0, 1) on the host (for host-side scalars such as lengths)."""
    u = uniform_u32(seed, name, torch.arange(n, dtype=torch.int64)).numpy().astype(np.float64)
    return (u + 0.5) / 2.0**32
