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

// Two floats as a bf16 pair (lo in the low half), rounded to nearest even;
// exact for dequantised values, which fit in bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));   // one v_cvt_pk_bf16_f32
}

// bf16 pair (lo, hi) of two E4M3FN codes, exact: a normal code's fields move
// into an fp32, a subnormal one (m * 2^-9) is formed by a product. (The NaN
// codes 0x7F and 0xFF are never written by the append and decode as 480.)
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// Eight channels of one row as four bf16 pairs, dequantised exactly: E2M1 x
// E4M3 (or E8M0, or E4M3 alone) has at most 6 significant bits. FP4 and
// MXFP4: cw holds the eight E2M1 nibbles (channel 2i in the low nibble of byte
// i) and sc the row's scale code for them in its low byte. FP8: cw and sc hold
// the E4M3 codes of channels 0-3 and 4-7. A row that is not real comes out as
// zeros.
template <int FMT>
__device__ __forceinline__ uint4 dequant8(uint32_t cw, uint32_t sc, bool real) {
  uint32_t d[4];
  if constexpr (FMT == kKvFp8) {
    const uint32_t lo = real ? cw : 0u, hi = real ? sc : 0u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      d[j] = pack_bf16x2(e4m3_to_f32((lo >> (16 * j)) & 0xFFu), e4m3_to_f32((lo >> (16 * j + 8)) & 0xFFu));
      d[2 + j] = pack_bf16x2(e4m3_to_f32((hi >> (16 * j)) & 0xFFu), e4m3_to_f32((hi >> (16 * j + 8)) & 0xFFu));
    }
  } else {
    // twice the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as bytes
    constexpr uint32_t lut_lo = 0x03020100u, lut_hi = 0x0C080604u;
    const uint32_t c = real ? cw : 0u;
    float sh2;   // half the block scale (the table holds twice the magnitudes)
    if constexpr (FMT == kKvMxfp4)
      sh2 = real ? __builtin_ldexpf(1.0f, (int)(sc & 0xFFu) - 128) : 0.0f;   // 2^(sc - 127) / 2, exact
    else
      sh2 = e4m3_half(real ? sc & 0xFFu : 0u);
    const uint32_t me = __builtin_amdgcn_perm(lut_hi, lut_lo, c & 0x07070707u);         // even channels
    const uint32_t mo = __builtin_amdgcn_perm(lut_hi, lut_lo, (c >> 4) & 0x07070707u);  // odd channels
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f0 = (float)((me >> (8 * j)) & 0xFFu) * sh2;
      float f1 = (float)((mo >> (8 * j)) & 0xFFu) * sh2;
      // sign bits of nibbles 2j (bit 8j+3) and 2j+1 (bit 8j+7)
      f0 = __uint_as_float(__float_as_uint(f0) | ((c << (28 - 8 * j)) & 0x80000000u));
      f1 = __uint_as_float(__float_as_uint(f1) | ((c << (24 - 8 * j)) & 0x80000000u));
      d[j] = pack_bf16x2(f0, f1);
    }
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// Dequantised bf16 pairs d[r][0..3] (channels 8cg..8cg+7 of rows r = 0..3 of an
// item) from the raw code and scale words of format FMT; FP4 and MXFP4 scale
// words are the row's aligned 4-byte word holding the scale byte of channel
// group cg. Rows whose valid bit is clear come out as zeros.
template <int FMT>
__device__ __forceinline__ void dequant_item(const uint32_t (&code)[4], const uint32_t (&scale)[4], uint32_t valid,
                                             int cg, uint32_t (&d)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t sc = scale[r];
    if constexpr (FMT == kKvMxfp4) sc >>= 8 * ((cg >> 2) & 3);
    else if constexpr (FMT == kKvFp4) sc >>= 8 * ((cg >> 1) & 3);
    const uint4 v = dequant8<FMT>(code[r], sc, (valid >> r) & 1u);
    d[r][0] = v.x; d[r][1] = v.y; d[r][2] = v.z; d[r][3] = v.w;
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
  int ring_first;     // window ring: slot of the oldest used window row, (p - n_w + 1) mod W
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
  r.ring_first = r.n_w > 0 ? (int)((uint32_t)(p - r.n_w + 1) % (uint32_t)a.W) : 0;   // p - n_w + 1 >= 0
  return r;
}

// Main-KV row of sparse slot j holding position `pos` at storage row `row`
// (already mapped), or -1 if the slot is not a usable row.
__device__ __forceinline__ int64_t sparse_row(const AttnArgs& a, const QueryInfo& qi_, int j, int64_t pos,
                                              int64_t row) {
  if (j >= qi_.n_s || pos < 0 || pos > qi_.p || row < 0) return -1;
  return row < a.total_rows ? row : -1;
}

// Storage row of window row wr (0 <= wr < n_w) of a query: the window buffer
// keeps a query's last n_w rows in order, a ring keeps position t in slot
// t mod W of the query's W rows.
__device__ __forceinline__ int64_t window_row(const AttnArgs& a, const QueryInfo& Q, int wr) {
  if (!a.ring) return Q.win_row0 + wr;
  const int slot = Q.ring_first + wr;              // both below W
  return Q.ring_base + (slot >= a.W ? slot - a.W : slot);
}

}  // namespace fp4kv
