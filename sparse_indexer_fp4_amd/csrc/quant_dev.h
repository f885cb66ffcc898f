// Main-KV quantize-append, one work item at a time: shared by the append
// kernels (quant.hip) and by the indexer scan, whose launch can carry a layer's
// append as extra workgroups (scan.hip). The FP4 cache: E2M1 values with an
// E4M3 scale for each 16-channel group ([G] FP4 main KV paragraph; [N] "FP4 KV
// Quantization and Cache Lifetime Management"). Two variants for the formats
// the pages compare it with: MXFP4, E2M1 with an E8M0 scale for each
// 32-channel block ([T] "Mechanism 3"), and an FP8 cache of E4M3FN codes ([G],
// [N]: FP4 is about half its bytes).
//
// Rounding decisions are taken by exact comparisons, never by rounding a
// quotient:
//   * scale: a first guess from amax * (1/6) is corrected against the exact
//     rounding thresholds 3*(v_c + v_{c+1}) of its neighbours (E4M3 values
//     have 4 significant bits, so every threshold is exact in fp32);
//   * values: |x| is compared with scale * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}
//     (<= 7 significant bits, exact); a tie moves to the even code.
#pragma once
#include "kernels.h"

namespace fp4kv {

// Rounding threshold between E4M3 codes c and c+1, times 6: 3 * (v_c + v_{c+1}).
__device__ __forceinline__ float scale_threshold(uint32_t c) {
  return 3.0f * (e4m3_value(c) + e4m3_value(c + 1));
}

// E4M3 code of the value nearest a/6 (a >= 0), ties to even, saturating at 448 (code 126).
__device__ __forceinline__ uint32_t encode_scale(float a) {
  if (!(a < 6.0f * 448.0f)) return 126u;
  // first guess: round-to-nearest of y ~= a/6 on the E4M3 grid by bit manipulation
  float y = a * (1.0f / 6.0f);
  uint32_t c;
  if (y < 0.015625f) {                       // below the smallest normal 2^-6: step 2^-9
    c = (uint32_t)__builtin_rintf(y * 512.0f);
  } else {
    uint32_t b = __float_as_uint(y);
    int e = (int)((b >> 23) & 0xFF) - 127;   // -6 .. 8
    uint32_t m = (b >> 20) & 7u;
    uint32_t rest = b & 0xFFFFFu;
    c = (uint32_t)((e + 7) << 3) + m + (rest >= 0x80000u ? 1u : 0u);
  }
  if (c > 126u) c = 126u;
  // exact correction: at most one step either way
  if (c < 126u) {
    float up = scale_threshold(c);
    if (a > up || (a == up && (c & 1u))) ++c;
  }
  if (c > 0u) {
    float lo = scale_threshold(c - 1u);
    if (a < lo || (a == lo && (c & 1u))) --c;
  }
  return c;
}

// 4-bit code of x given the group's decoded scale s (s >= 0).
__device__ __forceinline__ uint32_t encode_value(float x, float s) {
  float ax = fabsf(x);
  uint32_t m = 0;
  m += ax > s * 0.25f;
  m += ax > s * 0.75f;
  m += ax > s * 1.25f;
  m += ax > s * 1.75f;
  m += ax > s * 2.5f;
  m += ax > s * 3.5f;
  m += ax > s * 5.0f;
  // a tie at an odd threshold (between codes 1|2, 3|4, 5|6) goes up to the even code
  m += (ax == s * 0.75f) | (ax == s * 1.75f) | (ax == s * 3.5f);
  if (s == 0.0f) m = 0;
  return ((__float_as_uint(x) >> 28) & 8u) | m;
}

// Shared exponent of an MX block from the fp32 bits of its amax (a bf16 value):
// floor(log2 amax) - 2, clamped to [-127, 127]; -127 for amax = 0. Subnormal
// amax (value = bits * 2^-149) takes floor(log2) from its leading bit.
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits) {
  if (amax_bits == 0u) return -127;
  const int e = (int)(amax_bits >> 23);
  const int fl = e > 0 ? e - 127 : -149 + (31 - (int)__clz(amax_bits));
  const int sh = fl - 2;
  return sh < -127 ? -127 : (sh > 127 ? 127 : sh);
}

// E4M3FN code of x: the nearest finite value, ties to the even code, saturating
// at 448; sign bit = sign bit of x. x is a bf16 value (at most 8 significant
// bits), so the rounding is decided exactly on its bits.
__device__ __forceinline__ uint32_t encode_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float ax = fabsf(x);
  uint32_t c;
  if (ax > 448.0f) {
    c = 126u;
  } else if (ax < 0.015625f) {             // below 2^-6: subnormal step 2^-9 (the product is exact)
    c = (uint32_t)__builtin_rintf(ax * 512.0f);
  } else {
    const uint32_t b = __float_as_uint(ax);
    const uint32_t e = (b >> 23) - 120u;   // biased E4M3 exponent: (e32 - 127) + 7
    const uint32_t m = (b >> 20) & 7u, rest = b & 0xFFFFFu;
    const uint32_t up = (rest > 0x80000u) | ((rest == 0x80000u) & (m & 1u));
    c = (e << 3) + m + up;                 // a carry moves into the exponent; <= 126 since ax <= 448
  }
  return sign | c;
}

// One work item of an append: a 16-channel group (FP4, FP8) or a 32-channel
// block (MXFP4) of one source row, quantised and written at its destination
// row; rows whose destination lies outside [0, cap_rows) are skipped.
__device__ __forceinline__ int64_t append_items(const AppendJob& j) {
  return j.n_rows * (j.C >> (j.fmt == kKvMxfp4 ? 5 : 4));
}

__device__ __forceinline__ void append_item(const AppendJob& j, int64_t gid) {
  const int32_t C = j.C;
  if (j.fmt == kKvMxfp4) {
    const int32_t G = C >> 5;
    const int64_t row = gid / G;
    const int32_t g = (int32_t)(gid - row * G);
    const int64_t dst = append_dst(j.dd, row);
    if (dst < 0 || dst >= j.cap_rows) return;
    const uint4* p = reinterpret_cast<const uint4*>(j.src + row * C + g * 32);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = p[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax_bits = max(amax_bits, max((w[i] << 16) & 0x7FFF0000u, w[i] & 0x7FFF0000u));
    const int sh = mx_shared_exp(amax_bits);
    // 2^-sh is a normal float: sh <= 125 for any finite bf16 amax (< 2^128)
    const float inv = __uint_as_float((uint32_t)(127 - sh) << 23);
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // x * 2^-sh is exact (power of two; |result| < 8), and keeps the sign bit
      const uint32_t c0 = encode_value(__uint_as_float(w[i] << 16) * inv, 1.0f);
      const uint32_t c1 = encode_value(__uint_as_float(w[i] & 0xFFFF0000u) * inv, 1.0f);
      out[i >> 2] |= (c0 | (c1 << 4)) << (8 * (i & 3));
    }
    uint2* q = reinterpret_cast<uint2*>(j.codes + dst * (C >> 1) + g * 16);
    q[0] = make_uint2(out[0], out[1]);
    q[1] = make_uint2(out[2], out[3]);
    j.scales[dst * G + g] = (uint8_t)(sh + 127);
    return;
  }
  const int32_t G = C >> 4;
  const int64_t row = gid / G;
  const int32_t g = (int32_t)(gid - row * G);
  const int64_t dst = append_dst(j.dd, row);
  if (dst < 0 || dst >= j.cap_rows) return;
  const uint4* p = reinterpret_cast<const uint4*>(j.src + row * C + g * 16);
  const uint4 v0 = p[0], v1 = p[1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if (j.fmt == kKvFp8) {
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = encode_e4m3(__uint_as_float(w[2 * i] << 16));
      const uint32_t b = encode_e4m3(__uint_as_float(w[2 * i] & 0xFFFF0000u));
      const uint32_t c = encode_e4m3(__uint_as_float(w[2 * i + 1] << 16));
      const uint32_t d = encode_e4m3(__uint_as_float(w[2 * i + 1] & 0xFFFF0000u));
      out[i] = a | (b << 8) | (c << 16) | (d << 24);
    }
    uint2* q = reinterpret_cast<uint2*>(j.codes + dst * C + g * 16);
    q[0] = make_uint2(out[0], out[1]);
    q[1] = make_uint2(out[2], out[3]);
    return;
  }
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = (w[i] << 16) & 0x7FFF0000u, hi = w[i] & 0x7FFF0000u;
    amax_bits = max(amax_bits, max(lo, hi));
  }
  const uint32_t sc = encode_scale(__uint_as_float(amax_bits));
  const float s = e4m3_value(sc);
  uint32_t out0 = 0, out1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c0 = encode_value(__uint_as_float(w[i] << 16), s);
    const uint32_t c1 = encode_value(__uint_as_float(w[i] & 0xFFFF0000u), s);
    out0 |= (c0 | (c1 << 4)) << (8 * i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c0 = encode_value(__uint_as_float(w[4 + i] << 16), s);
    const uint32_t c1 = encode_value(__uint_as_float(w[4 + i] & 0xFFFF0000u), s);
    out1 |= (c0 | (c1 << 4)) << (8 * i);
  }
  *reinterpret_cast<uint2*>(j.codes + dst * (C >> 1) + g * 8) = make_uint2(out0, out1);
  j.scales[dst * G + g] = (uint8_t)sc;
}

}  // namespace fp4kv
