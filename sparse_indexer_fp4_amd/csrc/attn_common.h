// Pieces of the attention kernel (attn.hip) that do not depend on its
// workgroup layout: KV-row dequantisation and the per-query bookkeeping of the
// sparse and window rows.
#pragma once
#include "kernels.h"

namespace fp4kv {

constexpr int kAttnC = 512;       // channels (the kernels are written for 512)
constexpr int kChunk = 32;        // rows per chunk

// Two floats as a bf16 pair (lo in the low half), rounded to nearest even;
// exact for dequantised values, which fit in bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));   // one v_cvt_pk_bf16_f32
}

// Channels 2j and 2j+1 (the low and high nibble of byte j of c) as E2M1 values
// times s, as a bf16 pair. The hardware converter decodes the two nibbles
// exactly into fp32; the product with an E4M3 or E8M0 scale has at most 6
// significant bits, so it and its bf16 rounding are exact. (The converter's
// own scale operand is not used: it applies only the exponent of its scale.)
template <int J>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t c, float s) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, J);
  return pack_bf16x2(v[0] * s, v[1] * s);
}

// Eight channels of one row as four bf16 pairs, dequantised exactly: E2M1 x
// E4M3 (or E8M0, or E4M3 alone) has at most 6 significant bits. FP4 and
// MXFP4: cw holds the eight E2M1 nibbles (channel 2i in the low nibble of byte
// i) and sc the row's scale code for them in its low byte. FP8: cw and sc hold
// the E4M3 codes of channels 0-3 and 4-7. A row that is not real comes out as
// zeros. E4M3 codes go through the hardware E4M3FN converter (exact; the NaN
// codes 0x7F and 0xFF, which the append never writes, give NaN).
template <int FMT>
__device__ __forceinline__ uint4 dequant8(uint32_t cw, uint32_t sc, bool real) {
  if constexpr (FMT == kKvFp8) {
    const uint32_t lo = real ? cw : 0u, hi = real ? sc : 0u;
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), e = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                      pack_bf16x2(e[0], e[1]));
  } else {
    const uint32_t c = real ? cw : 0u;
    float s;   // the block scale
    if constexpr (FMT == kKvMxfp4)
      s = real ? __builtin_ldexpf(1.0f, (int)(sc & 0xFFu) - 127) : 0.0f;   // 2^(sc - 127), exact
    else
      s = real ? __builtin_amdgcn_cvt_f32_fp8(sc, 0) : 0.0f;
    return make_uint4(e2m1_pair<0>(c, s), e2m1_pair<1>(c, s), e2m1_pair<2>(c, s), e2m1_pair<3>(c, s));
  }
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
