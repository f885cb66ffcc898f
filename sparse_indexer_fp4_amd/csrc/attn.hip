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
// Workgroup = (query, split); one wave per group of 16 heads. A split takes
// every n_split-th 32-row chunk. Each chunk is dequantised once into LDS by
// the whole workgroup, one (8 rows x 8 channels) item per thread: the codes of
// a row are read as one coalesced 256-byte line per wave, E2M1 magnitudes come
// from a byte table (v_perm), and the item is written as a row-major copy (the
// K operand of S^T = K Q^T) and a channel-major copy (the V^T operand of
// O^T = V^T P^T), both in 16-byte units placed to avoid bank conflicts. The
// raw bytes of the next sparse chunk are loaded into registers while the
// current one is computed. Chunk rows 2j and 2j+1 are the j-th rows of the two
// 16-row MFMA tiles, so each lane's eight P values are exactly the eight rows
// its P^T operand needs. With one split the result is written directly;
// otherwise (m, l, O) partials go to the workspace and a combine kernel merges
// them.
#include "kernels.h"

namespace fp4kv {

constexpr int kAttnC = 512;       // channels (the kernels are written for 512)
constexpr int kChunk = 32;        // rows per chunk
constexpr int kItems = (kChunk / 8) * (kAttnC / 8);   // (8-row, 8-channel) items = 256

struct AttnShared {
  uint4 kbuf[kChunk * kAttnC / 8];       // row-major bf16 in 16-byte units: 32 KB
  uint4 vt[kAttnC * kChunk / 8];         // channel-major bf16, 8 rows per unit: 32 KB
  uint32_t valid;                        // bit r: chunk row r is a real row
};

// 16-byte unit holding channels 8u..8u+7 of chunk row `row`. Rows of equal
// parity (one MFMA tile) spread over all 16 bank groups.
__device__ __forceinline__ int kbuf_unit(int row, int u) { return row * 64 + (u ^ ((row >> 1) & 15)); }
// 16-byte unit holding rows 8q..8q+7 of channel ch. Channels are permuted within
// aligned groups of 4 and the row quarter is flipped, so that both the 8 channels
// 8c+e (c = 0..7) written together and the 8 consecutive channels read together
// land in distinct bank groups.
__device__ __forceinline__ int vt_unit(int ch, int q) {
  const int pc = ch ^ ((ch >> 3) & 3);
  const int f = ((ch >> 2) ^ (ch >> 5)) & 1;
  return pc * 4 + (q ^ f);
}

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

// Raw FP4 bytes of one item: channels 8c..8c+7 of 8 consecutive rows.
struct RawItem {
  uint32_t code[8];   // 8 nibbles per row
  uint32_t scale[8];  // the row's scale byte for these channels
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

// Item `item` of a chunk: row group (8 rows) and channel group (8 channels).
// Row groups are wave-uniform: a wave covers whole rows.
__device__ __forceinline__ int item_rows(int item) { return __builtin_amdgcn_readfirstlane(item >> 6); }

// Prefetch the raw bytes of sparse chunk c (window chunks are read at commit time).
template <int NW>
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const QueryInfo& Q, int qi, int c,
                                           RawItem (&raw)[kItems / (64 * NW)]) {
  constexpr int PER = kItems / (64 * NW);
  if (c >= Q.cs) return;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 64 * NW;
    const int rg = item_rows(item), cg = item & 63;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = sparse_row(a, Q, qi, c * kChunk + 8 * rg + r);
      const int64_t rr = row < 0 ? 0 : row;
      const uint32_t code = *reinterpret_cast<const uint32_t*>(a.codes + rr * (kAttnC / 2) + 4 * cg);
      const uint32_t sc = a.scales[rr * (kAttnC / 16) + (cg >> 1)];
      raw[it].code[r] = row < 0 ? 0u : code;
      raw[it].scale[r] = row < 0 ? 0u : sc;
    }
  }
}

// Write one item (8 rows x 8 channels as bf16 pairs d[row][pair]) into both copies.
__device__ __forceinline__ void store_item(AttnShared& sh, int rg, int cg, const uint32_t (&d)[8][4]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) sh.kbuf[kbuf_unit(8 * rg + r, cg)] = make_uint4(d[r][0], d[r][1], d[r][2], d[r][3]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high / low bf16 of each pair
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_perm(d[2 * i + 1][e >> 1], d[2 * i][e >> 1], sel);
    sh.vt[vt_unit(8 * cg + e, rg)] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int NW>
__device__ __forceinline__ void commit_chunk(AttnShared& sh, const QueryInfo& Q, const AttnArgs& a, int qi, int c,
                                             const RawItem (&raw)[kItems / (64 * NW)]) {
  constexpr int PER = kItems / (64 * NW);
  const bool sparse = c < Q.cs;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 64 * NW;
    const int rg = item_rows(item), cg = item & 63;
    uint32_t d[8][4];
    if (sparse) {
      // twice the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as bytes
      constexpr uint32_t lut_lo = 0x03020100u, lut_hi = 0x0C080604u;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t code = raw[it].code[r];
        const float sh2 = e4m3_half(raw[it].scale[r]);
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
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int wr = (c - Q.cs) * kChunk + 8 * rg + r;
        const bool ok = wr < Q.n_w;
        const int64_t row = Q.win_row0 + (ok ? wr : 0);
        const uint4 kv = ok ? *reinterpret_cast<const uint4*>(a.swa_k + row * kAttnC + 8 * cg) : make_uint4(0, 0, 0, 0);
        d[r][0] = kv.x; d[r][1] = kv.y; d[r][2] = kv.z; d[r][3] = kv.w;
      }
      // keys: row-major copy only
#pragma unroll
      for (int r = 0; r < 8; ++r) sh.kbuf[kbuf_unit(8 * rg + r, cg)] = make_uint4(d[r][0], d[r][1], d[r][2], d[r][3]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int wr = (c - Q.cs) * kChunk + 8 * rg + r;
        const bool ok = wr < Q.n_w;
        const int64_t row = Q.win_row0 + (ok ? wr : 0);
        const uint4 vv = ok ? *reinterpret_cast<const uint4*>(a.swa_v + row * kAttnC + 8 * cg) : make_uint4(0, 0, 0, 0);
        d[r][0] = vv.x; d[r][1] = vv.y; d[r][2] = vv.z; d[r][3] = vv.w;
      }
      // values: channel-major copy only
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_perm(d[2 * i + 1][e >> 1], d[2 * i][e >> 1], sel);
        sh.vt[vt_unit(8 * cg + e, rg)] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      continue;
    }
    store_item(sh, rg, cg, d);
  }
  if (threadIdx.x < 64) {
    const int r = threadIdx.x;
    bool ok = false;
    if (r < kChunk) {
      if (sparse) ok = sparse_row(a, Q, qi, c * kChunk + r) >= 0;
      else ok = (c - Q.cs) * kChunk + r < Q.n_w;
    }
    const uint64_t b = __ballot(ok);
    if (r == 0) sh.valid = (uint32_t)b;
  }
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnArgs a) {
  constexpr int PER = kItems / (64 * NW);
  __shared__ AttnShared sh;
  const int split = blockIdx.x, qi = blockIdx.y;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int g = lane / 16, hcol = lane % 16;
  const int head = wave * 16 + hcol;
  const QueryInfo Q = query_info(a, qi);
  const int nchunk = Q.cs + Q.cw;

  // Q^T operand: lane holds Q[head][32kk + 8g .. +7] for kk = 0..15
  uint4 qv[16];
  const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.Hq + head) * kAttnC);
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) qv[kk] = qp[4 * kk + g];

  v4f o[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_use = -__builtin_inff(), l_run = 0.0f;   // P is formed as exp2(x - m_use)

  RawItem raw[PER];
  int c = split;
  if (c < nchunk) load_chunk<NW>(a, Q, qi, c, raw);
  for (; c < nchunk; c += a.n_split) {
    __syncthreads();
    commit_chunk<NW>(sh, Q, a, qi, c, raw);
    __syncthreads();
    if (c + a.n_split < nchunk) load_chunk<NW>(a, Q, qi, c + a.n_split, raw);

    // S^T tiles: A = even rows (tile 0) / odd rows (tile 1), B = Q^T
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint4 k0 = sh.kbuf[kbuf_unit(2 * hcol, 4 * kk + g)];
      const uint4 k1 = sh.kbuf[kbuf_unit(2 * hcol + 1, 4 * kk + g)];
      const v8bf b = __builtin_bit_cast(v8bf, qv[kk]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, k0), b, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, k1), b, s1, 0, 0, 0);
    }
    // lane holds rows 8g+2i (s0[i]) and 8g+2i+1 (s1[i]) for its head
    const uint32_t valid = sh.valid;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = ((valid >> (8 * g + 2 * i)) & 1u) ? s0[i] * a.scale_log2 : -__builtin_inff();
      x[2 * i + 1] = ((valid >> (8 * g + 2 * i + 1)) & 1u) ? s1[i] * a.scale_log2 : -__builtin_inff();
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
      for (int t = 0; t < 32; ++t) o[t] *= corr;
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
    for (int t = 0; t < 32; ++t) {
      const uint4 vtile = sh.vt[vt_unit(16 * t + hcol, g)];
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vtile), phi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vtile), plo, o[t], 0, 0, 0);
    }
  }

  // lane holds O^T[ch = 16t + 4g + i][head]; l_run is this lane's share of the sum
  float l_all = l_run + __shfl_xor(l_run, 16);
  l_all += __shfl_xor(l_all, 32);
  if (a.n_split == 1) {
    const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
    float* op = a.out + ((int64_t)qi * a.Hq + head) * kAttnC;
#pragma unroll
    for (int t = 0; t < 32; ++t)
      *reinterpret_cast<float4*>(op + 16 * t + 4 * g) = make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (a.lse && g == 0)
      a.lse[(int64_t)qi * a.Hq + head] = l_all > 0.0f ? m_use * 0.69314718055994531f + logf(l_all) : -__builtin_inff();
  } else {
    const int64_t slot = ((int64_t)qi * a.n_split + split) * a.Hq + head;
    float* op = a.part_o + slot * kAttnC;
#pragma unroll
    for (int t = 0; t < 32; ++t)
      *reinterpret_cast<float4*>(op + 16 * t + 4 * g) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    if (g == 0) { a.part_ml[2 * slot] = l_all > 0.0f ? m_use : -__builtin_inff(); a.part_ml[2 * slot + 1] = l_all; }
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
  const int nw = a.Hq / 16;
  dim3 grid((uint32_t)a.n_split, (uint32_t)a.nq);
  switch (nw) {
    case 1: attn_kernel<1><<<grid, dim3(64), 0, stream>>>(a); break;
    case 2: attn_kernel<2><<<grid, dim3(128), 0, stream>>>(a); break;
    case 4: attn_kernel<4><<<grid, dim3(256), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  attn_combine_kernel<<<dim3((uint32_t)a.Hq, (uint32_t)a.nq), dim3(128), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
