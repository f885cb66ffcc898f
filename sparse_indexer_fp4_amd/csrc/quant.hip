// FP4 quantize-append: E2M1 values with one E4M3 scale per 16 channels.
// [G] FP4 main KV paragraph; [N] "FP4 KV Quantization and Cache Lifetime Management".
//
// One thread per 16-channel group. Rounding decisions are taken by exact
// comparisons, never by rounding a quotient:
//   * scale: a first guess from amax * (1/6) is corrected against the exact
//     rounding thresholds 3*(v_c + v_{c+1}) of its neighbours (E4M3 values
//     have 4 significant bits, so every threshold is exact in fp32);
//   * values: |x| is compared with scale * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}
//     (<= 7 significant bits, exact); a tie moves to the even code.
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

__global__ __launch_bounds__(256) void quantize_append_kernel(
    const uint16_t* __restrict__ src, int64_t n_rows, int32_t C, const int64_t* __restrict__ dst_rows,
    int64_t dst_start, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t cap_rows) {
  const int32_t G = C >> 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_rows * G) return;
  const int64_t row = gid / G;
  const int32_t g = (int32_t)(gid - row * G);
  const int64_t dst = dst_rows ? dst_rows[row] : dst_start + row;
  if (dst < 0 || dst >= cap_rows) return;

  const uint4* p = reinterpret_cast<const uint4*>(src + row * C + g * 16);
  uint4 v0 = p[0], v1 = p[1];
  uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = (w[i] << 16) & 0x7FFF0000u, hi = w[i] & 0x7FFF0000u;
    amax_bits = max(amax_bits, max(lo, hi));
  }
  const uint32_t sc = encode_scale(__uint_as_float(amax_bits));
  const float s = e4m3_value(sc);
  uint32_t out0 = 0, out1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c0 = encode_value(__uint_as_float(w[i] << 16), s);
    uint32_t c1 = encode_value(__uint_as_float(w[i] & 0xFFFF0000u), s);
    out0 |= (c0 | (c1 << 4)) << (8 * i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c0 = encode_value(__uint_as_float(w[4 + i] << 16), s);
    uint32_t c1 = encode_value(__uint_as_float(w[4 + i] & 0xFFFF0000u), s);
    out1 |= (c0 | (c1 << 4)) << (8 * i);
  }
  *reinterpret_cast<uint2*>(codes + dst * (C >> 1) + g * 8) = make_uint2(out0, out1);
  scales[dst * G + g] = (uint8_t)sc;
}

hipError_t launch_quantize_append(const void* src, int64_t n_rows, int32_t C, const int64_t* dst_rows,
                                  int64_t dst_start, uint8_t* codes, uint8_t* scales, int64_t cap_rows,
                                  hipStream_t stream) {
  const int64_t n = n_rows * (C >> 4);
  const int64_t blocks = (n + 255) / 256;
  quantize_append_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      static_cast<const uint16_t*>(src), n_rows, C, dst_rows, dst_start, codes, scales, cap_rows);
  return hipGetLastError();
}

}  // namespace fp4kv
