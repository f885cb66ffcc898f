// Sparse attention over selected FP4 main-KV rows and a sliding-window branch,
// merged by log-sum-exp.
// [T] "Mechanism 4: the hierarchical sparse indexer" (attention runs over the
// selected candidates); [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (each layer brings a main query and window keys/values of its own) and "Causal
// Encoder-Decoder and Prefill Halving" (a window of the last 128 tokens);
// [G] FP4 main KV paragraph (E2M1 values, an E4M3 scale for each 16-channel group).
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
// n_split-th 32-row chunk, its first window chunk first. Each chunk is
// dequantised once into LDS by the whole workgroup, one (4 rows x 8 channels)
// item per thread: the codes of a row are read as one coalesced 256-byte line
// per wave and decoded by the hardware FP4 and FP8 converters. Rows are stored
// row-major only, with an XOR swizzle of the 16-byte units that keeps the S
// reads, the P V reads and the commit writes free of bank conflicts; the V^T
// operand of O^T = V^T P^T is read from the same rows with the LDS transposing
// read (ds_read_b64_tr_b16), so no channel-major copy is made. Window values
// (which differ from their keys) get a second row-major buffer. The selected
// positions a split needs are read with one vector load at the start; the raw
// bytes of the next sparse chunk are loaded into registers while the current
// one is computed and are not touched until it is committed, so the loads stay
// in flight. Each step issues all of its LDS reads of K (and most of V) before
// the products that use them, so the products wait for the first read only. Chunk rows 2j and 2j+1 are the j-th rows of the two 16-row MFMA
// tiles, so each lane's eight P values are exactly the eight rows its P^T
// operand needs. With one split the result is written directly; otherwise
// (m, l, O) partials go to the workspace and a combine kernel merges them.
#include "attn_common.h"

namespace fp4kv {

constexpr int kItems = (kChunk / 4) * (kAttnC / 8);   // (4-row, 8-channel) items = 512

constexpr int kRowUnits = kChunk * 64;   // a chunk's rows in 16-byte units (64 per row)

template <int NHG>
struct AttnShared {
  uint4 kbuf[kRowUnits];                 // row-major bf16 keys (= values for sparse rows): 32 KB
  uint4 vbuf[kRowUnits];                 // row-major bf16 values of a window chunk: 32 KB
  float4 sp[NHG][2][2][64];              // partial S of each head group's two channel halves, [tile][lane]
  uint32_t vb[2][kChunk / 4];            // bit r of word q: chunk row 4q+r is a real row (by step parity)
};

// 16-byte unit holding channels 8u..8u+7 of chunk row `row`: the unit index is
// XOR-swizzled by a function of the row bits r0..r4, x = r2 | r1 << 1 |
// (r0 ^ r3) << 2 | (r0 ^ r4) << 3. With it the three access patterns fall in
// distinct LDS banks: the K-operand reads of S (16 rows of one parity, one
// unit column), the transposing V-operand reads of P V (4 consecutive rows x
// 32 bytes per 16 lanes, 8 rows per 32 lanes), and the row writes of a commit.
__device__ __forceinline__ int row_swizzle(int row) {
  return ((row >> 2) & 1) | (row & 2) | ((((row) ^ (row >> 3)) & 1) << 2) | ((((row) ^ (row >> 4)) & 1) << 3);
}
__device__ __forceinline__ int kbuf_unit(int row, int u) { return row * 64 + (u ^ row_swizzle(row)); }

// Raw bytes of one item, loaded one chunk ahead of its use. Sparse and
// window chunks have register slots of their own, so that no slot ever holds
// both kinds (merging the two would copy registers that are still being
// loaded, which waits for the loads).
struct RawSparse {
  // Channels 8c..8c+7 of row r (a stand-in row where row r is not real):
  //   FP4 and MXFP4: code = their 8 nibbles, scale = the row's aligned scale word
  //                  holding their scale byte;
  //   FP8:           code = the E4M3 bytes of channels 8c..8c+3, scale = of 8c+4..8c+7.
  uint32_t code[4];
  uint32_t scale[4];
  uint32_t valid;     // bit r: row r is real; the others are zeroed when committed
};
struct RawWindow {
  uint4 k[4], v[4];   // bf16 keys and values, channels 8c..8c+7 of row r
  uint32_t valid;
};

// Item `item` of a chunk: row group (4 rows) and channel group (8 channels).
// Row groups are wave-uniform: a wave covers whole rows.
__device__ __forceinline__ int item_rows(int item) { return __builtin_amdgcn_readfirstlane(item >> 6); }

// The selected positions a wave needs are read with one vector load when the
// workgroup starts: lane l takes the position of row 4*rg + (l & 3) of the
// m-th chunk of this split, where m = l / (4 PER) and rg is the row group of the
// wave's item (l / 4) % PER. The lane checks it once (slot within n_s, position
// within the query's causal range, row inside the cache; with paged storage it
// maps it through the block table first) and keeps the addresses of the row's
// codes and scale bytes, or of the stand-in (the query, always present) for a
// slot that is not a usable row; a ballot keeps which slots are rows. In the
// loop a row then costs four lane reads. Chunks past the 16/PER covered this
// way check their rows where they are loaded.
struct LanePos {
  uint32_t c_lo, c_hi;     // codes of the slot's row (or the stand-in)
  uint32_t s_lo, s_hi;     // scale bytes of the slot's row (or the stand-in)
  uint64_t real;           // wave-uniform: bit l set when lane l's slot is a row
};

template <int FMT>
__device__ __forceinline__ constexpr int64_t code_row_bytes() { return FMT == kKvFp8 ? kAttnC : kAttnC / 2; }
template <int FMT>
__device__ __forceinline__ constexpr int64_t scale_row_bytes() { return FMT == kKvMxfp4 ? kAttnC / 32 : kAttnC / 16; }

template <int NHG, int FMT, bool PAGED>
__device__ __forceinline__ LanePos idx_lane_load(const AttnArgs& a, const QueryInfo& Q, int qi, int split, int lane) {
  constexpr int PER = kItems / (128 * NHG);
  const int m = lane / (4 * PER), it = (lane / 4) % PER, r = lane & 3;
  const int rg = (int)(threadIdx.x >> 6) + it * 2 * NHG;   // item_rows of item threadIdx.x + it * 128 * NHG
  const int j = (split + m * a.n_split) * kChunk + 4 * rg + r;
  const int64_t pos = j < a.k ? a.idx[(int64_t)qi * a.k + j] : -1;
  const int64_t row = sparse_row(a, Q, j, pos, PAGED ? paged_row(a.map, Q.seq, pos) : Q.kv_base + pos);
  const uint8_t* stand_in = reinterpret_cast<const uint8_t*>(a.q);
  const uint64_t cb = reinterpret_cast<uint64_t>(row < 0 ? stand_in : a.codes + row * code_row_bytes<FMT>());
  const uint64_t sb = FMT == kKvFp8 ? cb   // (FP8 rows have no scale bytes)
                                    : reinterpret_cast<uint64_t>(row < 0 ? stand_in : a.scales + row * scale_row_bytes<FMT>());
  LanePos lp;
  lp.c_lo = (uint32_t)cb;
  lp.c_hi = (uint32_t)(cb >> 32);
  lp.s_lo = (uint32_t)sb;
  lp.s_hi = (uint32_t)(sb >> 32);
  lp.real = __builtin_amdgcn_ballot_w64(row >= 0);
  return lp;
}

// Storage row of sparse slot j of a chunk past the preloaded ones, or -1 if
// the slot is not a usable row.
template <bool PAGED>
__device__ __forceinline__ int64_t late_chunk_row(const AttnArgs& a, const QueryInfo& Q, int qi, int j) {
  const int64_t pos = j < a.k ? a.idx[(int64_t)qi * a.k + j] : -1;
  return sparse_row(a, Q, j, pos, PAGED ? paged_row(a.map, Q.seq, pos) : Q.kv_base + pos);
}

// Issue the loads of chunk c, the m-th chunk of this split: FP4 codes and
// scales of a sparse chunk, or bf16 keys and values of a window chunk. The
// registers are not read until the chunk is committed, so the loads stay in
// flight while the current chunk is computed.
template <int NHG, int FMT, bool PAGED>
__device__ __forceinline__ void load_sparse(const AttnArgs& a, const QueryInfo& Q, int qi, int c, int m,
                                            const LanePos& lp, RawSparse (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // the addresses of the row's code and scale bytes, or of the stand-in
      // for a slot without a row (zeroed at commit)
      uint64_t cb, sb;
      bool real;
      if (m < 16 / PER) {
        const int l = (m * PER + it) * 4 + r;
        cb = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lp.c_hi, l) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)lp.c_lo, l);
        sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lp.s_hi, l) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)lp.s_lo, l);
        real = (lp.real >> l) & 1u;
      } else {
        const int64_t row = late_chunk_row<PAGED>(a, Q, qi, c * kChunk + 4 * rg + r);
        const uint8_t* stand_in = reinterpret_cast<const uint8_t*>(a.q);
        real = row >= 0;
        cb = reinterpret_cast<uint64_t>(real ? a.codes + row * code_row_bytes<FMT>() : stand_in);
        sb = FMT == kKvFp8 ? cb : reinterpret_cast<uint64_t>(real ? a.scales + row * scale_row_bytes<FMT>() : stand_in);
      }
      // (global pointers: the addresses are device memory, so the loads are
      // global rather than flat loads)
      typedef const __attribute__((address_space(1))) uint32_t* gptr32;
      if constexpr (FMT == kKvFp8) {
        raw[it].code[r] = reinterpret_cast<gptr32>(cb + 8 * cg)[0];
        raw[it].scale[r] = reinterpret_cast<gptr32>(cb + 8 * cg)[1];
      } else {
        constexpr int kGroupShift = FMT == kKvMxfp4 ? 2 : 1;     // items (8 channels) per scale byte: 4 or 2
        raw[it].code[r] = reinterpret_cast<gptr32>(cb + 4 * cg)[0];
        raw[it].scale[r] = reinterpret_cast<gptr32>(sb + 4 * (cg >> (kGroupShift + 2)))[0];
      }
      bits |= (uint32_t)real << r;
    }
    raw[it].valid = bits;
  }
}

template <int NHG>
__device__ __forceinline__ void load_window(const AttnArgs& a, const QueryInfo& Q, int c,
                                            RawWindow (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int wr = (c - Q.cs) * kChunk + 4 * rg + r;
      const bool ok = wr < Q.n_w;
      bits |= (uint32_t)ok << r;
      const int64_t row = window_row(a, Q, ok ? wr : 0);
      raw[it].k[r] = *reinterpret_cast<const uint4*>(a.swa_k + row * kAttnC + 8 * cg);
      raw[it].v[r] = *reinterpret_cast<const uint4*>(a.swa_v + row * kAttnC + 8 * cg);
    }
    raw[it].valid = bits;
  }
}

// Write one item (4 rows x 8 channels as bf16 pairs d[row][pair]) into a
// row-major buffer.
__device__ __forceinline__ void store_rows(uint4* buf, int rg, int cg, const uint32_t (&d)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) buf[kbuf_unit(4 * rg + r, cg)] = make_uint4(d[r][0], d[r][1], d[r][2], d[r][3]);
}

// Maximum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48)
// by the two lane-swap permutes: register-to-register, no LDS round trip.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

template <int NHG, int FMT>
__device__ __forceinline__ void commit_sparse(AttnShared<NHG>& sh, int vbi, const RawSparse (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    const uint32_t valid = raw[it].valid;
    if (cg == 0) sh.vb[vbi][rg] = valid;
    uint32_t d[4][4];
    dequant_item<FMT>(raw[it].code, raw[it].scale, valid, cg, d);
    store_rows(sh.kbuf, rg, cg, d);
  }
}

template <int NHG>
__device__ __forceinline__ void commit_window(AttnShared<NHG>& sh, int vbi, const RawWindow (&raw)[kItems / (128 * NHG)]) {
  constexpr int PER = kItems / (128 * NHG);
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int item = threadIdx.x + it * 128 * NHG;
    const int rg = item_rows(item), cg = item & 63;
    const uint32_t valid = raw[it].valid;
    if (cg == 0) sh.vb[vbi][rg] = valid;
    uint32_t d[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 kv = ((valid >> r) & 1u) ? raw[it].k[r] : make_uint4(0, 0, 0, 0);
      d[r][0] = kv.x; d[r][1] = kv.y; d[r][2] = kv.z; d[r][3] = kv.w;
    }
    store_rows(sh.kbuf, rg, cg, d);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 vv = ((valid >> r) & 1u) ? raw[it].v[r] : make_uint4(0, 0, 0, 0);
      d[r][0] = vv.x; d[r][1] = vv.y; d[r][2] = vv.z; d[r][3] = vv.w;
    }
    store_rows(sh.vbuf, rg, cg, d);
  }
}

// A tail window chunk (one that follows the sparse ones) straight from HBM
// into the chunk buffers, with no registers in between: one 16-byte
// global_load_lds per lane and row fills a whole 1 KB row, lane L writing
// unit slot L, so lane L loads the unit that the row's swizzle puts there.
// With 8 waves, wave w loads rows 4w .. 4w+3 of keys and values. A row past
// the query's window reads window row 0 instead: its products are masked and
// its values multiply a zero P. The valid bits are written by the caller.
template <int NHG>
__device__ __forceinline__ void window_to_lds(const AttnArgs& a, const QueryInfo& Q, AttnShared<NHG>& sh, int c,
                                              int wave, int lane) {
  static_assert(NHG == 4, "8 waves x 4 rows cover a chunk");
  const int w = __builtin_amdgcn_readfirstlane(wave);   // rows, and so their addresses, are wave-uniform
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr;
    const int wr = (c - Q.cs) * kChunk + r;
    const int64_t row = window_row(a, Q, wr < Q.n_w ? wr : 0);
    const uint32_t ofs = 16u * (uint32_t)(lane ^ row_swizzle(r));
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(a.swa_k + row * kAttnC) + ofs),
                                     (__attribute__((address_space(3))) void*)&sh.kbuf[r * 64], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(a.swa_v + row * kAttnC) + ofs),
                                     (__attribute__((address_space(3))) void*)&sh.vbuf[r * 64], 16, 0, 0);
  }
}

// V^T operand of channel tile t (channels 256hc + 16t .. +15, chunk rows
// 8g .. 8g+7) by two transposing reads: lane 4a+b of a 16-lane group gets
// element b of the 8-byte words addressed by lanes a, 4+a, 8+a, 12+a, so lane
// i addresses row 8g + 4h + i/4, channels 16t + 4(i%4) .. +3 (h = 0, 1 for
// the two reads). vt_byte gives the byte offset of a lane's word for tile 0;
// tile t only XORs t into bits 5-8 (its 16-byte unit is 2t above tile 0's,
// bits 1-4 of the unit index, which the row swizzle leaves alone apart from
// its own XOR), so read_vt needs one XOR per read.
__device__ __forceinline__ uint32_t vt_byte(int hc, int hcol, int row) {
  return (uint32_t)(kbuf_unit(row, 32 * hc + ((hcol & 3) >> 1)) * 16 + 8 * (hcol & 1));
}
template <int NHG>
__device__ __forceinline__ v8bf read_vt(const AttnShared<NHG>& sh, uint32_t lo0, uint32_t hi0, int t) {
  const char* base = reinterpret_cast<const char*>(&sh);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(base + (lo0 ^ ((uint32_t)t << 5))));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(base + (hi0 ^ ((uint32_t)t << 5))));
  return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup = (query, split): two waves per group of 16 heads, each owning half
// of the 512 output channels (64 accumulators per lane, so two waves fit on a
// SIMD). The two waves of a head group each form S over their half of the
// channels and exchange the partial sums through LDS.
template <int NHG, int FMT, bool PAGED>
__global__ __launch_bounds__(128 * NHG) void attn_kernel(AttnArgs a) {
  constexpr int PER = kItems / (128 * NHG);
  __shared__ AttnShared<NHG> sh;
  // The query index is the fastest grid dimension: workgroups are dealt to the
  // eight XCDs round-robin in launch order, so all splits of one query (and its
  // combine below) run on one XCD and meet its partials in that XCD's L2.
  const int qi = blockIdx.x, split = blockIdx.y;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int hg = wave >> 1, hc = wave & 1;          // head group, channel half
  const int g = lane / 16, hcol = lane % 16;
  const int head = ((int)blockIdx.z * NHG + hg) * 16 + hcol;   // z: this block's group of NHG head groups
  const QueryInfo Q = query_info(a, qi);
  const LanePos lp = idx_lane_load<NHG, FMT, PAGED>(a, Q, qi, split, lane);
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

  // This split's chunks are split + i * n_split: nS sparse ones, then nW window
  // ones. The first window chunk is loaded in the prologue and computed first;
  // the sparse chunks follow, each loaded a step before its commit (the first
  // one during the window step); further window chunks (only with few splits)
  // go straight into LDS a step ahead (with several items per thread, they are
  // loaded when they are committed).
  const int ns_ = a.n_split;
  const int nS = split < Q.cs ? (Q.cs - split + ns_ - 1) / ns_ : 0;
  const int nT = split < nchunk ? (nchunk - split + ns_ - 1) / ns_ : 0;
  const int nW = nT - nS, w0 = nW > 0 ? 1 : 0;
  // With a window chunk first, the first sparse chunk is loaded after that
  // chunk's commit (it is committed at the end of the window step, like every
  // later one a step after its load), so that the prologue waits for one round
  // of loads only.
  RawSparse rs[PER] = {};
  RawWindow rw[PER];
  if (nS > 0 && w0 == 0) load_sparse<NHG, FMT, PAGED>(a, Q, qi, split, 0, lp, rs);
  // (with several items per thread the window slot would not fit in registers
  // beside the accumulators: the first window chunk is then loaded at commit)
  if constexpr (PER == 1) {
    if (nW > 0) load_window<NHG>(a, Q, split + nS * ns_, rw);
  }
  // Take delivery of everything loaded so far, once, here (the prologue's
  // loads were issued together and the first commit needs them anyway): a
  // register still counted as in flight at the loop head would make every
  // iteration wait for the loads issued after it (the counter is in order),
  // which includes the prefetched chunk.
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qv[kk])));
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    asm volatile("" ::"v"(rs[it].code[0]), "v"(rs[it].code[1]), "v"(rs[it].code[2]), "v"(rs[it].code[3]));
    asm volatile("" ::"v"(rs[it].scale[0]), "v"(rs[it].scale[1]), "v"(rs[it].scale[2]), "v"(rs[it].scale[3]));
    if constexpr (PER == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        asm volatile("" ::"v"(__builtin_bit_cast(u32x4, rw[it].k[r])), "v"(__builtin_bit_cast(u32x4, rw[it].v[r])));
    }
  }
  // Step 0's chunk is committed here. Every step then ends by committing the
  // next step's chunk: all of its own LDS reads of the chunk buffers are done
  // before its exchange barrier, so the buffers are free from there on, and a
  // step needs two barriers, one that publishes its chunk and one for the S
  // exchange. (The valid bits alternate between two slots, since a wave that
  // commits may run ahead of one still forming this step's P.)
  if (w0) {
    if constexpr (PER == 1) {
      commit_window<NHG>(sh, 0, rw);
    } else {
      RawWindow tw[PER];
      load_window<NHG>(a, Q, split + nS * ns_, tw);
      commit_window<NHG>(sh, 0, tw);
    }
    if (nS > 0) load_sparse<NHG, FMT, PAGED>(a, Q, qi, split, 0, lp, rs);
  } else if (nS > 0) {
    commit_sparse<NHG, FMT>(sh, 0, rs);
    if (nS > 1) load_sparse<NHG, FMT, PAGED>(a, Q, qi, split + ns_, 1, lp, rs);
  }
  // Tail window chunks go straight into LDS, issued one step ahead.
  constexpr bool kWinToLds = PER == 1;
  for (int step = 0; step < nT; ++step) {
    const int i = step - w0;              // sparse ordinal when i < nS
    const bool window = step < w0 || i >= nS;
    const int vbi = step & 1;
    __syncthreads();

    // partial S^T over this channel half: A = even rows (tile 0) / odd rows (tile 1), B = Q^T
    // (all 16 K reads are issued before the first product, so that the
    // products wait for the first read only)
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    uint4 kr0[8], kr1[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kr0[kk] = sh.kbuf[kbuf_unit(2 * hcol, 32 * hc + 4 * kk + g)];
      kr1[kk] = sh.kbuf[kbuf_unit(2 * hcol + 1, 32 * hc + 4 * kk + g)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const v8bf b = __builtin_bit_cast(v8bf, qv[kk]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kr0[kk]), b, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kr1[kk]), b, s1, 0, 0, 0);
    }
    // V^T operands of all 16 channel tiles, read now (before the exchange
    // barrier, which then also ends this step's use of the chunk buffers), so
    // that the reads overlap the S products, the exchange and the softmax.
    // Values: the latent rows themselves (kbuf), or the window's (vbuf); the
    // buffer's offset in the shared block is added before the XORs, which leave
    // its bits alone. (The bases are made opaque per step so that the compiler
    // does not keep 32 tile addresses live across the loop.)
    const uint32_t vofs = window ? (uint32_t)offsetof(AttnShared<NHG>, vbuf) : (uint32_t)offsetof(AttnShared<NHG>, kbuf);
    uint32_t vlo = vofs + vt_byte(hc, hcol, 8 * g + (hcol >> 2)), vhi = vofs + vt_byte(hc, hcol, 8 * g + (hcol >> 2) + 4);
    asm volatile("" : "+v"(vlo), "+v"(vhi));
    v8bf vt[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) vt[t] = read_vt(sh, vlo, vhi, t);
    __builtin_amdgcn_sched_barrier(0);
    {
      sh.sp[hg][hc][0][lane] = make_float4(s0[0], s0[1], s0[2], s0[3]);
      sh.sp[hg][hc][1][lane] = make_float4(s1[0], s1[1], s1[2], s1[3]);
    }
    __syncthreads();
    if constexpr (kWinToLds) {
      // every wave has read this step's buffers: the next step's chunk, when it
      // is a tail window chunk (window ordinal i - nS + 2), starts loading
      if (step + 1 < nT && i + 1 >= nS) window_to_lds<NHG>(a, Q, sh, split + (i + 2) * ns_, wave, lane);
    }
    // full S: the two halves added in the same order in both waves
    const float4 a0 = sh.sp[hg][0][0][lane], a1 = sh.sp[hg][0][1][lane];
    const float4 b0 = sh.sp[hg][1][0][lane], b1 = sh.sp[hg][1][1][lane];
    const float sa[4] = {a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w};
    const float sb[4] = {a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w};
    // lane holds rows 8g+2i (sa[i]) and 8g+2i+1 (sb[i]) for its head
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < kChunk / 4; ++q) valid |= sh.vb[vbi][q] << (4 * q);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = ((valid >> (8 * g + 2 * i)) & 1u) ? sa[i] * a.scale_log2 : -__builtin_inff();
      x[2 * i + 1] = ((valid >> (8 * g + 2 * i + 1)) & 1u) ? sb[i] * a.scale_log2 : -__builtin_inff();
    }
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, x[i]);
    cm = max_over_rows(cm);
    // move the reference maximum only when this chunk exceeds it by more than
    // 2^8 (always at a head's first usable row: m_use starts at -inf)
    const bool move = cm > m_use + 8.0f;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float corr = move ? __builtin_amdgcn_exp2f(m_use - cm) : 1.0f;
      if (move) m_use = cm;
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] *= corr;
    }
    // m_use stays -inf while a head has seen no usable row; its x are all -inf
    // then, and so are its P zeros (its rows are zeros too: rows that are not
    // real are committed as zeros, or multiply a zero P)
    const float m_sub = m_use == -__builtin_inff() ? 0.0f : m_use;
    float p[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { p[i] = __builtin_amdgcn_exp2f(x[i] - m_sub); psum += p[i]; }
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
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[t], phi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[t], plo, o[t], 0, 0, 0);
    }

    // the next step's chunk: a sparse chunk from the registers loaded a step
    // ago (whose slot then takes the loads of the sparse chunk after it); a
    // tail window chunk, already on its way into the buffers, gets its valid
    // bits and this wave waits for its share of the rows
    if (step + 1 < nT) {
      const int i1 = i + 1;
      if (i1 < nS) {
        commit_sparse<NHG, FMT>(sh, vbi ^ 1, rs);
        if (i1 + 1 < nS) load_sparse<NHG, FMT, PAGED>(a, Q, qi, split + (i1 + 1) * ns_, i1 + 1, lp, rs);
      } else if constexpr (kWinToLds) {
        if (threadIdx.x < kChunk / 4) {
          const int wr0 = (split + (i1 + 1) * ns_ - Q.cs) * kChunk + 4 * (int)threadIdx.x;
          uint32_t bits = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) bits |= (uint32_t)(wr0 + r < Q.n_w) << r;
          sh.vb[vbi ^ 1][threadIdx.x] = bits;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        RawWindow tw[PER];
        load_window<NHG>(a, Q, split + (i1 + 1) * ns_, tw);   // window ordinal i1 - nS + 1
        commit_window<NHG>(sh, vbi ^ 1, tw);
      }
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
      __builtin_nontemporal_store(v4f{o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv},
                                  reinterpret_cast<v4f*>(op + 16 * t + 4 * g));
    if (a.lse && g == 0 && hc == 0)
      a.lse[(int64_t)qi * a.Hq + head] = l_all > 0.0f ? m_use * 0.69314718055994531f + logf(l_all) : -__builtin_inff();
  } else {
    // Split partials are written and read back once, non-temporally, like the
    // outputs: dirty lines left in the caches were written back during the next
    // indexer scan and slowed it (decode step at 128K: scan 204 -> 196 us with
    // partials and outputs non-temporal).
    const int64_t slot = ((int64_t)qi * a.n_split + split) * a.Hq + head;
    float* op = a.part_o + slot * kAttnC + 256 * hc;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      __builtin_nontemporal_store(v4f{o[t][0], o[t][1], o[t][2], o[t][3]}, reinterpret_cast<v4f*>(op + 16 * t + 4 * g));
    if (g == 0 && hc == 0) { a.part_ml[2 * slot] = l_all > 0.0f ? m_use : -__builtin_inff(); a.part_ml[2 * slot + 1] = l_all; }
  }
}

// Merge the splits of one (query, head): 128 threads x 4 channels. Every
// split's (m, l) and O slice are loaded before any is used, so the S loads of
// a thread are in flight together.
template <int S>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int qi = blockIdx.x, head = blockIdx.y;   // query fastest, as in attn_kernel
  float2 ml[S];
  float4 v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t slot = ((int64_t)qi * S + s) * a.Hq + head;
    ml[s] = reinterpret_cast<const float2*>(a.part_ml)[slot];
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.part_o + slot * kAttnC) + threadIdx.x);
    v[s] = make_float4(t[0], t[1], t[2], t[3]);
  }
  float M = ml[0].x;
#pragma unroll
  for (int s = 1; s < S; ++s) M = fmaxf(M, ml[s].x);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float f = (ml[s].x == -__builtin_inff()) ? 0.0f : exp2f(ml[s].x - M);
    L += f * ml[s].y;
    acc.x += f * v[s].x; acc.y += f * v[s].y; acc.z += f * v[s].z; acc.w += f * v[s].w;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  __builtin_nontemporal_store(v4f{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv},
                              reinterpret_cast<v4f*>(a.out + ((int64_t)qi * a.Hq + head) * kAttnC) + threadIdx.x);
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)qi * a.Hq + head] = L > 0.0f ? M * 0.69314718055994531f + logf(L) : -__builtin_inff();
}

// Splits per query for nq queries of up to `chunks` chunks: enough workgroups
// to cover the CUs, at least one chunk per split.
// Launch plan for nq queries of Hq heads and `chunks` chunks: head groups of
// 16 per block (nhg), blocks across the heads (hb = Hq / 16 / nhg) and splits
// of the rows (n_split).
struct AttnPlan {
  int nhg, hb, n_split;
};

AttnPlan attn_plan(int nq, int Hq, int chunks) {
  AttnPlan p;
  p.nhg = Hq / 16;
  p.hb = 1;
  int s = 1;
  while (s < 16 && (int64_t)nq * s < 256 && chunks >= 2 * s) s *= 2;
  p.n_split = s;
  return p;
}

size_t attn_workspace_bytes(int nq, int Hq, int k, int W) {
  const int chunks = (k + kChunk - 1) / kChunk + (W + kChunk - 1) / kChunk;
  const AttnPlan p = attn_plan(nq, Hq, chunks);
  if (p.n_split == 1) return 0;
  return (size_t)nq * p.n_split * Hq * (kAttnC + 2) * sizeof(float);
}

hipError_t launch_attn(AttnArgs a, void* ws, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  const int chunks = (a.k + kChunk - 1) / kChunk + (a.W + kChunk - 1) / kChunk;
  const AttnPlan plan = attn_plan(a.nq, a.Hq, chunks);
  a.n_split = plan.n_split;
  if (a.n_split > 1) {
    a.part_o = static_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)a.nq * a.n_split * a.Hq * kAttnC;
  }
  if (a.kv_fmt < kKvFp4 || a.kv_fmt > kKvFp8) return hipErrorInvalidValue;
  const int nhg = plan.nhg;
  dim3 grid((uint32_t)a.nq, (uint32_t)a.n_split, (uint32_t)plan.hb);
  const bool paged = a.map.block_table != nullptr;
#define FP4KV_ATTN_CASE(NH, FM)                                                                  \
  if (nhg == NH && a.kv_fmt == FM) {                                                             \
    if (paged) attn_kernel<NH, FM, true><<<grid, dim3(128 * NH), 0, stream>>>(a);                 \
    else attn_kernel<NH, FM, false><<<grid, dim3(128 * NH), 0, stream>>>(a);                      \
  } else
  FP4KV_ATTN_CASE(1, kKvFp4) FP4KV_ATTN_CASE(2, kKvFp4) FP4KV_ATTN_CASE(4, kKvFp4)
  FP4KV_ATTN_CASE(1, kKvMxfp4) FP4KV_ATTN_CASE(2, kKvMxfp4) FP4KV_ATTN_CASE(4, kKvMxfp4)
  FP4KV_ATTN_CASE(1, kKvFp8) FP4KV_ATTN_CASE(2, kKvFp8) FP4KV_ATTN_CASE(4, kKvFp8)
  return hipErrorInvalidValue;
#undef FP4KV_ATTN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const dim3 cgrid((uint32_t)a.nq, (uint32_t)a.Hq);
  switch (a.n_split) {
    case 2: attn_combine_kernel<2><<<cgrid, dim3(128), 0, stream>>>(a); break;
    case 4: attn_combine_kernel<4><<<cgrid, dim3(128), 0, stream>>>(a); break;
    case 8: attn_combine_kernel<8><<<cgrid, dim3(128), 0, stream>>>(a); break;
    case 16: attn_combine_kernel<16><<<cgrid, dim3(128), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp4kv
