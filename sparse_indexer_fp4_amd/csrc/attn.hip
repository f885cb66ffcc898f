// Sparse attention over selected FP4 main-KV rows and a sliding-window branch,
// merged by log-sum-exp.
// [T] "Mechanism 4: the hierarchical sparse indexer" (attention runs over the
// selected candidates); [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (every layer has its own main Q and SWA KV) and "Causal
// Encoder-Decoder and Prefill Halving" (a window of the last 128 tokens);
// [G] FP4 main KV paragraph (E2M1 values, one E4M3 scale per 16 channels).
//
// The main KV is a shared latent (keys = values = the dequantised row) read by
// all Hq heads, so per query the work is two dense contractions:
// S = Q K^T ([Hq x 512] x [512 x rows]) and O = P V. They run on MFMA
// (v_mfma_f32_16x16x32_bf16): dequantised E2M1 x E4M3 values have at most 6
// significant bits and are exact in bf16; P is split into bf16 hi + lo parts
// so the P V product keeps ~16 bits of P; accumulation is fp32.
//
// The sparse rows and the window rows form one softmax over their union; by
// the log-sum-exp identity this equals merging the two branch softmaxes by
// their log-sum-exps. The running maximum is only moved (and O, l rescaled)
// when a chunk's maximum exceeds it by more than 2^8; otherwise P is formed
// against the old maximum (values up to 2^8, still exact after the hi/lo
// split), so the 128 accumulators per lane are normally touched by MFMA only.
//
// Workgroup = (query, split); two waves per group of 16 heads, each owning
// half of the 512 output channels (64 accumulators per lane, so that two waves
// fit on a SIMD and hide each other's LDS and MFMA latencies). Each wave forms
// the partial S over its channel half; the two partials are exchanged through
// LDS and added in the same order by both waves. A split takes every
// n_split-th 32-row chunk. Each chunk is dequantised once into LDS by the whole
// workgroup, one (4 rows x 8 channels) item per thread: the codes of a row are
// read as one coalesced 256-byte line per wave, E2M1 magnitudes come from a
// byte table (v_perm), and the item is written as a row-major copy (the K
// operand of S^T = K Q^T) and a channel-major copy (the V^T operand of
// O^T = V^T P^T), both padded so that the MFMA operand reads fall in distinct
// bank groups. The raw bytes of the next sparse chunk are loaded into registers
// while the current one is computed, and are not touched (masked) until the
// chunk is committed, so the loads stay in flight. Chunk rows 2j and 2j+1 are
// the j-th rows of the two 16-row MFMA tiles, so each lane's eight P values are
// exactly the eight rows its P^T operand needs. With one split the result is
// written directly; otherwise (m, l, O) partials go to the workspace and a
// combine kernel merges them.
#include "kernels.h"

namespace fp4kv {

constexpr int kAttnC = 512;       // channels (the kernels are written for 512)
constexpr int kChunk = 32;        // rows per chunk
constexpr int kItems = (kChunk / 4) * (kAttnC / 8);   // (4-row, 8-channel) items = 512

constexpr int kKbufUnits = kChunk * 64 + kChunk / 2;          // 64 units per row + 1 per row pair
constexpr int kVtUnits = kAttnC * 4 + kAttnC / 4;               // 4 units per channel + 1 per 4 channels

template <int NHG>
struct AttnShared {
  uint4 kbuf[kKbufUnits];                // row-major bf16 in 16-byte units: 33 KB
  uint4 vt[kVtUnits];                    // channel-major bf16, 8 rows per unit: 34 KB
  float sp[NHG][2][64][8];               // partial S of each head group's two channel halves
  uint32_t vb[kChunk / 4];               // bit r of word q: chunk row 4q+r is a real row
};

// 16-byte unit holding channels 8u..8u+7 of chunk row `row`. One unit of
// padding per row pair: the 16 rows of equal parity read by one MFMA tile fall
// in 16 distinct bank groups.
__device__ __forceinline__ int kbuf_unit(int row, int u) { return row * 64 + (row >> 1) + u; }
// 16-byte unit holding rows 8q..8q+7 of channel ch. One unit of padding per 4
// channels: the 16 consecutive channels read by one MFMA tile fall in 16
// distinct bank groups.
__device__ __forceinline__ int vt_unit(int ch, int q) { return ch * 4 + (ch >> 2) + q; }

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

// Raw FP4 bytes of one item: channels 8c..8c+7 of 4 consecutive rows.
struct RawItem {
  uint32_t code[4];   // 8 nibbles per row (loaded from a stand-in row when the row is not real)
  uint32_t scale[4];  // the row's scale byte for these channels (likewise)
  uint32_t valid;     // bit r: row r is real; the others are zeroed when committed
};

struct QueryInfo {
  int64_t kv_base;    // first main-KV row of the sequence
  int64_t p;          // query position
  int n_s, n_w;       // sparse rows, window rows
  int cs, cw;         // chunks of each
  int64_t win_row0;   // window-buffer row holding the oldest used window row
};

__device__ __forceinline__ QueryInfo query_info(const AttnArgs& a, int qi) {
  QueryInfo r;
  r.kv_base = a.seq_start ? a.seq_start[qi] : a.seq_start_scalar;
  int64_t p = a.q_pos ? (int64_t)a.q_pos[qi] : (int64_t)a.pos0 + qi;
  r.p = p;            // negative: the query sees no token
  int ns = a.n_idx[qi];
  r.n_s = ns < 0 ? 0 : (ns > a.k ? a.k : ns);
  r.n_w = p < 0 ? 0 : (int)min<int64_t>(a.W, p + 1);
  r.cs = (r.n_s + kChunk - 1) / kChunk;
  r.cw = (r.n_w + kChunk - 1) / kChunk;
  r.win_row0 = (int64_t)qi * a.win_stride + (a.W - r.n_w);
  return r;
}

// Main-KV row of sparse slot j, or -1 if the slot is not a usable row.
__device__ __forceinline__ int64_t sparse_row(const AttnArgs& a, const QueryInfo& qi_, int qi, int j) {
  if (j >= qi_.n_s) return -1;
  int64_t pos = a.idx[(int64_t)qi * a.k + j];
  if (pos < 0 || pos > qi_.p) return -1;
  int64_t row = qi_.kv_base + pos;
  return row < a.total_rows ? row : -1;
}

// Item `item` of a chunk: row group (4 rows) and channel group (8 channels).
// Row groups are wave-uniform: a wave covers whole rows.
__device__ __forceinline__ int item_rows(int item) { return __builtin_amdgcn_readfirstlane(item >> 6); }

// Prefetch the raw bytes of sparse chunk c (window chunks are read at commit time).
template <int NHG>
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const QueryInfo& Q, int qi, int c,
                                           RawItem (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
  if (c >= Q.cs) return;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = sparse_row(a, Q, qi, c * kChunk + 4 * rg + r);
      const int64_t rr = row < 0 ? 0 : row;
      // the loaded values are not touched until the chunk is committed, so
      // the loads stay in flight while the current chunk is computed
      raw[it].code[r] = *reinterpret_cast<const uint32_t*>(a.codes + rr * (kAttnC / 2) + 4 * cg);
      raw[it].scale[r] = a.scales[rr * (kAttnC / 16) + (cg >> 1)];
      bits |= (uint32_t)(row >= 0) << r;
    }
    raw[it].valid = bits;
  }
}

// Write one item (4 rows x 8 channels as bf16 pairs d[row][pair]): the rows
// into the row-major copy, and per channel the 4 rows as half of a unit of the
// channel-major copy.
template <int NHG>
__device__ __forceinline__ void store_item(AttnShared<NHG>& sh, int rg, int cg, const uint32_t (&d)[4][4], bool keys,
                                           bool values) {
  if (keys) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sh.kbuf[kbuf_unit(4 * rg + r, cg)] = make_uint4(d[r][0], d[r][1], d[r][2], d[r][3]);
  }
  if (values) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high / low bf16 of each pair
      const uint32_t w0 = __builtin_amdgcn_perm(d[1][e >> 1], d[0][e >> 1], sel);
      const uint32_t w1 = __builtin_amdgcn_perm(d[3][e >> 1], d[2][e >> 1], sel);
      uint2* u = reinterpret_cast<uint2*>(&sh.vt[vt_unit(8 * cg + e, rg >> 1)]);
      u[rg & 1] = make_uint2(w0, w1);
    }
  }
}

template <int NHG>
__device__ __forceinline__ void commit_chunk(AttnShared<NHG>& sh, const QueryInfo& Q, const AttnArgs& a, int c,
                                             const RawItem (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
  const bool sparse = c < Q.cs;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    uint32_t d[4][4];
    if (sparse) {
      if (cg == 0) sh.vb[rg] = raw[it].valid;
      // twice the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as bytes
      constexpr uint32_t lut_lo = 0x03020100u, lut_hi = 0x0C080604u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool real = (raw[it].valid >> r) & 1u;
        const uint32_t code = real ? raw[it].code[r] : 0u;
        const float sh2 = e4m3_half(real ? raw[it].scale[r] : 0u);
        const uint32_t me = __builtin_amdgcn_perm(lut_hi, lut_lo, code & 0x07070707u);         // even channels
        const uint32_t mo = __builtin_amdgcn_perm(lut_hi, lut_lo, (code >> 4) & 0x07070707u);  // odd channels
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float f0 = (float)((me >> (8 * j)) & 0xFFu) * sh2;
          float f1 = (float)((mo >> (8 * j)) & 0xFFu) * sh2;
          // sign bits of nibbles 2j (bit 8j+3) and 2j+1 (bit 8j+7)
          f0 = __uint_as_float(__float_as_uint(f0) | ((code << (28 - 8 * j)) & 0x80000000u));
          f1 = __uint_as_float(__float_as_uint(f1) | ((code << (24 - 8 * j)) & 0x80000000u));
          d[r][j] = pack_bf16x2(f0, f1);
        }
      }
      store_item<NHG>(sh, rg, cg, d, true, true);
    } else {
      uint32_t bits = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int wr = (c - Q.cs) * kChunk + 4 * rg + r;
        const bool ok = wr < Q.n_w;
        bits |= (uint32_t)ok << r;
        const int64_t row = Q.win_row0 + (ok ? wr : 0);
        const uint4 kv = ok ? *reinterpret_cast<const uint4*>(a.swa_k + row * kAttnC + 8 * cg) : make_uint4(0, 0, 0, 0);
        d[r][0] = kv.x; d[r][1] = kv.y; d[r][2] = kv.z; d[r][3] = kv.w;
      }
      if (cg == 0) sh.vb[rg] = bits;
      store_item<NHG>(sh, rg, cg, d, true, false);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int wr = (c - Q.cs) * kChunk + 4 * rg + r;
        const bool ok = wr < Q.n_w;
        const int64_t row = Q.win_row0 + (ok ? wr : 0);
        const uint4 vv = ok ? *reinterpret_cast<const uint4*>(a.swa_v + row * kAttnC + 8 * cg) : make_uint4(0, 0, 0, 0);
        d[r][0] = vv.x; d[r][1] = vv.y; d[r][2] = vv.z; d[r][3] = vv.w;
      }
      store_item<NHG>(sh, rg, cg, d, false, true);
    }
  }
}

// Workgroup = (query, split): two waves per group of 16 heads, each owning half
// of the 512 output channels (64 accumulators per lane, so two waves fit on a
// SIMD). The two waves of a head group each form S over their half of the
// channels and exchange the partial sums through LDS.
template <int NHG>
__global__ __launch_bounds__(128 * NHG) void attn_kernel(AttnArgs a) {
  constexpr int PER = kItems / (128 * NHG);
  __shared__ AttnShared<NHG> sh;
  const int split = blockIdx.x, qi = blockIdx.y;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int hg = wave >> 1, hc = wave & 1;          // head group, channel half
  const int g = lane / 16, hcol = lane % 16;
  const int head = hg * 16 + hcol;
  const QueryInfo Q = query_info(a, qi);
  const int nchunk = Q.cs + Q.cw;

  // Q^T operand over this wave's channel half: lane holds Q[head][256hc + 32kk + 8g .. +7]
  uint4 qv[8];
  const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.Hq + head) * kAttnC + 256 * hc);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qv[kk] = qp[4 * kk + g];

  v4f o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_use = -__builtin_inff(), l_run = 0.0f;   // P is formed as exp2(x - m_use)

  RawItem raw[PER];
  int c = split;
  if (c < nchunk) load_chunk<NHG>(a, Q, qi, c, raw);
  for (; c < nchunk; c += a.n_split) {
    __syncthreads();
    commit_chunk<NHG>(sh, Q, a, c, raw);
    __syncthreads();
    if (c + a.n_split < nchunk) load_chunk<NHG>(a, Q, qi, c + a.n_split, raw);

    // partial S^T over this channel half: A = even rows (tile 0) / odd rows (tile 1), B = Q^T
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 k0 = sh.kbuf[kbuf_unit(2 * hcol, 32 * hc + 4 * kk + g)];
      const uint4 k1 = sh.kbuf[kbuf_unit(2 * hcol + 1, 32 * hc + 4 * kk + g)];
      const v8bf b = __builtin_bit_cast(v8bf, qv[kk]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, k0), b, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, k1), b, s1, 0, 0, 0);
    }
    {
      float4* mine = reinterpret_cast<float4*>(&sh.sp[hg][hc][lane][0]);
      mine[0] = make_float4(s0[0], s0[1], s0[2], s0[3]);
      mine[1] = make_float4(s1[0], s1[1], s1[2], s1[3]);
    }
    __syncthreads();
    // full S: the two halves added in the same order in both waves
    const float4* h0 = reinterpret_cast<const float4*>(&sh.sp[hg][0][lane][0]);
    const float4* h1 = reinterpret_cast<const float4*>(&sh.sp[hg][1][lane][0]);
    const float4 a0 = h0[0], a1 = h0[1], b0 = h1[0], b1 = h1[1];
    const float sa[4] = {a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w};
    const float sb[4] = {a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w};
    // lane holds rows 8g+2i (sa[i]) and 8g+2i+1 (sb[i]) for its head
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < kChunk / 4; ++q) valid |= sh.vb[q] << (4 * q);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = ((valid >> (8 * g + 2 * i)) & 1u) ? sa[i] * a.scale_log2 : -__builtin_inff();
      x[2 * i + 1] = ((valid >> (8 * g + 2 * i + 1)) & 1u) ? sb[i] * a.scale_log2 : -__builtin_inff();
    }
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, x[i]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    if (cm == -__builtin_inff() && m_use == -__builtin_inff()) continue;   // nothing usable yet (per head)
    // move the reference maximum only when this chunk exceeds it by more than 2^8
    const bool move = cm > m_use + 8.0f;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float corr = move ? exp2f(m_use - cm) : 1.0f;
      if (move) m_use = cm;
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] *= corr;
    }
    float p[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { p[i] = exp2f(x[i] - m_use); psum += p[i]; }
    l_run += psum;
    v8bf phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)p[i];
      phi[i] = h;
      plo[i] = (__bf16)(p[i] - (float)h);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint4 vtile = sh.vt[vt_unit(256 * hc + 16 * t + hcol, g)];
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vtile), phi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vtile), plo, o[t], 0, 0, 0);
    }
  }

  // lane holds O^T[ch = 256hc + 16t + 4g + i][head]; l_run is this lane's share of the sum
  float l_all = l_run + __shfl_xor(l_run, 16);
  l_all += __shfl_xor(l_all, 32);
  if (a.n_split == 1) {
    const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
    float* op = a.out + ((int64_t)qi * a.Hq + head) * kAttnC + 256 * hc;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      *reinterpret_cast<float4*>(op + 16 * t + 4 * g) = make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (a.lse && g == 0 && hc == 0)
      a.lse[(int64_t)qi * a.Hq + head] = l_all > 0.0f ? m_use * 0.69314718055994531f + logf(l_all) : -__builtin_inff();
  } else {
    const int64_t slot = ((int64_t)qi * a.n_split + split) * a.Hq + head;
    float* op = a.part_o + slot * kAttnC + 256 * hc;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      *reinterpret_cast<float4*>(op + 16 * t + 4 * g) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    if (g == 0 && hc == 0) { a.part_ml[2 * slot] = l_all > 0.0f ? m_use : -__builtin_inff(); a.part_ml[2 * slot + 1] = l_all; }
  }
}

// Merge the splits of one (query, head): 128 threads x 4 channels.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int head = blockIdx.x, qi = blockIdx.y;
  const int S = a.n_split;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[2 * (((int64_t)qi * S + s) * a.Hq + head)]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const int64_t slot = ((int64_t)qi * S + s) * a.Hq + head;
    const float m = a.part_ml[2 * slot], l = a.part_ml[2 * slot + 1];
    const float f = (m == -__builtin_inff()) ? 0.0f : exp2f(m - M);
    L += f * l;
    const float4 v = reinterpret_cast<const float4*>(a.part_o + slot * kAttnC)[threadIdx.x];
    acc.x += f * v.x; acc.y += f * v.y; acc.z += f * v.z; acc.w += f * v.w;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  reinterpret_cast<float4*>(a.out + ((int64_t)qi * a.Hq + head) * kAttnC)[threadIdx.x] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)qi * a.Hq + head] = L > 0.0f ? M * 0.69314718055994531f + logf(L) : -__builtin_inff();
}

// Splits per query for nq queries of up to `chunks` chunks: enough workgroups
// to cover the CUs, at least two chunks per split.
int attn_splits(int nq, int chunks) {
  int s = 1;
  while (s < 16 && (int64_t)nq * s < 256 && chunks >= 4 * s) s *= 2;
  return s;
}

size_t attn_workspace_bytes(int nq, int Hq, int k, int W) {
  const int chunks = (k + kChunk - 1) / kChunk + (W + kChunk - 1) / kChunk;
  const int s = attn_splits(nq, chunks);
  if (s == 1) return 0;
  return (size_t)nq * s * Hq * (kAttnC + 2) * sizeof(float);
}

hipError_t launch_attn(AttnArgs a, void* ws, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  const int chunks = (a.k + kChunk - 1) / kChunk + (a.W + kChunk - 1) / kChunk;
  a.n_split = attn_splits(a.nq, chunks);
  if (a.n_split > 1) {
    a.part_o = static_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)a.nq * a.n_split * a.Hq * kAttnC;
  }
  const int nhg = a.Hq / 16;
  dim3 grid((uint32_t)a.n_split, (uint32_t)a.nq);
  switch (nhg) {
    case 1: attn_kernel<1><<<grid, dim3(128), 0, stream>>>(a); break;
    case 2: attn_kernel<2><<<grid, dim3(256), 0, stream>>>(a); break;
    case 4: attn_kernel<4><<<grid, dim3(512), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  attn_combine_kernel<<<dim3((uint32_t)a.Hq, (uint32_t)a.nq), dim3(128), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
