// Internal helpers shared by the fp4kv kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4kv {

constexpr int kWave = 64;

// Operand and result types of v_mfma_f32_16x16x32_bf16.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

// max(x, 0) for finite x as one v_med3 (fmaxf would add a NaN-quieting step).
__device__ __forceinline__ float relu_f(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }

// bfloat16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Value of an E4M3FN code (bias 7, no infinities; 0x7F / 0xFF are NaN and never produced here).
__host__ __device__ constexpr float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e == 0 ? (float)m * (1.0f / 512.0f)
                     : (float)(8u + m) * (1.0f / 8.0f) * (e >= 7 ? (float)(1u << (e - 7)) : 1.0f / (float)(1u << (7 - e)));
  return (c & 0x80u) ? -mag : mag;
}

// Maximum over each aligned group of 8 lanes, left in every lane of the group
// (swap neighbours, swap pairs, then mirror the halves of each 8 lanes). Each
// step is one v_max_f32 whose first operand is read through DPP; the s_nop
// gives the two wait states a DPP read needs after a VALU write. The inputs
// are finite here (scores, or -FLT_MAX for a token that is not visible), so
// max has no NaN case to handle.
__device__ __forceinline__ float max8(float v) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(v) : "v"(r));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  return r;
}

}  // namespace fp4kv
