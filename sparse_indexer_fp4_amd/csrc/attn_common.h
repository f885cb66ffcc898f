// Pieces of the attention kernel (attn.hip) that do not depend on its
// workgroup layout: KV-row dequantisation and the per-query bookkeeping of the
// sparse and window rows.
#pragma once
#include "kernels.h"

namespace fp4kv {

constexpr int kAttnC = 512;       // channels (the kernels are written for 512)
constexpr int kChunk = 32;        // rows per chunk

// Half the value of an E4M3 scale code (sign bit never set): exact in fp32.
__device__ __forceinline__ float e4m3_half(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 119u) << 23) | (m << 20)) : (float)m * 0x1p-10f;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // exact here: dequantised values fit in bf16
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// bf16 pair (lo, hi) of two E4M3FN codes, exact: a normal code's fields move
// into an fp32, a subnormal one (m * 2^-9) is formed by a product. (The NaN
// codes 0x7F and 0xFF are never written by the append and decode as 480.)
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// Dequantised bf16 pairs d[r][0..3] (channels 8cg..8cg+7 of rows r = 0..3 of an
// item) from the raw code and scale words of format FMT; rows whose valid bit
// is clear come out as zeros. Exact: E2M1 x E4M3 (or E8M0, or E4M3 alone) has
// at most 6 significant bits.
template <int FMT>
__device__ __forceinline__ void dequant_item(const uint32_t (&code)[4], const uint32_t (&scale)[4], uint32_t valid,
                                             int cg, uint32_t (&d)[4][4]) {
  if constexpr (FMT == kKvFp8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool real = (valid >> r) & 1u;
      const uint32_t lo = real ? code[r] : 0u, hi = real ? scale[r] : 0u;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        d[r][j] = pack_bf16x2(e4m3_to_f32((lo >> (16 * j)) & 0xFFu), e4m3_to_f32((lo >> (16 * j + 8)) & 0xFFu));
        d[r][2 + j] = pack_bf16x2(e4m3_to_f32((hi >> (16 * j)) & 0xFFu), e4m3_to_f32((hi >> (16 * j + 8)) & 0xFFu));
      }
    }
  } else {
    // twice the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as bytes
    constexpr uint32_t lut_lo = 0x03020100u, lut_hi = 0x0C080604u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool real = (valid >> r) & 1u;
      const uint32_t cw = real ? code[r] : 0u;
      float sh2;   // half the block scale (the table holds twice the magnitudes)
      if constexpr (FMT == kKvMxfp4) {
        const uint32_t sc = (scale[r] >> (8 * ((cg >> 2) & 3))) & 0xFFu;
        sh2 = real ? __builtin_ldexpf(1.0f, (int)sc - 128) : 0.0f;   // 2^(sc - 127) / 2, exact
      } else {
        sh2 = e4m3_half(real ? (scale[r] >> (8 * ((cg >> 1) & 3))) & 0xFFu : 0u);
      }
      const uint32_t me = __builtin_amdgcn_perm(lut_hi, lut_lo, cw & 0x07070707u);         // even channels
      const uint32_t mo = __builtin_amdgcn_perm(lut_hi, lut_lo, (cw >> 4) & 0x07070707u);  // odd channels
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f0 = (float)((me >> (8 * j)) & 0xFFu) * sh2;
        float f1 = (float)((mo >> (8 * j)) & 0xFFu) * sh2;
        // sign bits of nibbles 2j (bit 8j+3) and 2j+1 (bit 8j+7)
        f0 = __uint_as_float(__float_as_uint(f0) | ((cw << (28 - 8 * j)) & 0x80000000u));
        f1 = __uint_as_float(__float_as_uint(f1) | ((cw << (24 - 8 * j)) & 0x80000000u));
        d[r][j] = pack_bf16x2(f0, f1);
      }
    }
  }
}

struct QueryInfo {
  int64_t kv_base;    // first main-KV row of the sequence (contiguous storage)
  int64_t seq;        // sequence of the query (paged storage)
  int64_t p;          // query position
  int n_s, n_w;       // sparse rows, window rows
  int cs, cw;         // chunks of each
  int64_t win_row0;   // window-buffer row holding the oldest used window row
  int64_t ring_base;  // window ring: first row of the query's W rows
};

__device__ __forceinline__ QueryInfo query_info(const AttnArgs& a, int qi) {
  QueryInfo r;
  r.kv_base = a.map.block_table ? 0 : (a.seq_start ? a.seq_start[qi] : a.seq_start_scalar);
  r.seq = a.map.block_table ? qi / a.page_q_per_seq : 0;
  int64_t p = a.q_pos ? (int64_t)a.q_pos[qi] : (int64_t)a.pos0 + qi;
  r.p = p;            // negative: the query sees no token
  int ns = a.n_idx[qi];
  r.n_s = ns < 0 ? 0 : (ns > a.k ? a.k : ns);
  if (!a.map.block_table && (r.kv_base < 0 || r.kv_base > a.total_rows)) r.n_s = 0;   // start outside the cache
  r.n_w = p < 0 ? 0 : (int)min<int64_t>(a.W, p + 1);
  r.cs = (r.n_s + kChunk - 1) / kChunk;
  r.cw = (r.n_w + kChunk - 1) / kChunk;
  r.win_row0 = (int64_t)qi * a.win_stride + (a.W - r.n_w);
  r.ring_base = (int64_t)qi * a.W;
  return r;
}

// Main-KV row of sparse slot j holding position `pos` at storage row `row`
// (already mapped), or -1 if the slot is not a usable row.
__device__ __forceinline__ int64_t sparse_row(const AttnArgs& a, const QueryInfo& qi_, int j, int64_t pos,
                                              int64_t row) {
  if (j >= qi_.n_s || pos < 0 || pos > qi_.p || row < 0) return -1;
  return row < a.total_rows ? row : -1;
}

}  // namespace fp4kv
