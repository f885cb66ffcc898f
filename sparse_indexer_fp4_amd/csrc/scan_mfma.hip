// Indexer scan for many queries of one sequence (a prefill chunk) on the
// matrix cores: the same token score s_t = sum_h w_h * max(0, q_h . k_t) and
// 8-token block maximum as the decode scan.
// [G] hierarchical sparse indexer paragraph; [T] "Mechanism 4: the hierarchical
// sparse indexer"; [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (the Full layer scores every visible context token).
//
// Queries of one sequence share every key, so the q_h . k_t of a wave's four
// queries over 16 tokens are v_mfma_f32_16x16x32_bf16 tiles per 32 channels:
// rows = (query, head) pairs (the query fragments, resident in VGPRs), columns =
// tokens (the key fragment, read from LDS). The rows are arranged so that a
// result lane holds 4 heads of one query at one token, and the four products
// over the four groups of 4 heads leave all 16 heads of that query and token
// in the lane: ReLU, the head weights and the sum over the heads are applied
// there, with no exchange between lanes, and lane l ends with the score of
// query l/16 at token l%16 of a 16-token tile.
//
// Workgroup = 32 queries of one sequence x one range of tokens: 8 compute waves
// (4 queries each) and one copy wave. The copy wave streams 128-token key tiles
// HBM -> LDS with global_load_lds into a 3-deep ring, XOR-swizzled so that the
// compute waves' 16-byte fragment reads are free of bank conflicts. It is the
// only wave that loads, so its vmcnt waits count its tile loads alone (the
// compute waves' score stores never hold them up). One barrier per tile:
// before it the copy wave has waited for the next tile and the compute waves
// have finished the current one; the tile after next is then loaded into the
// slot the finished tile leaves free. Within a tile, each 32-token part's
// 32 products (both 16-token tiles) are issued before either tile's weighted
// ReLU sums, so that one tile's vector work overlaps the other's products.
//
// Work items (query block, token range) are laid out so that the workgroups
// an XCD runs together share one token range, which then streams through that
// XCD's L2 once.
//
// Integer-valued bf16 inputs make every product and partial sum exact in fp32
// while below 2^24, so the scores equal the decode scan's bit for bit.
#include "kernels.h"

namespace fp4kv {

constexpr int kMQ = 32;                       // queries per workgroup
constexpr int kMWaves = 8;                    // compute waves, 4 queries each
constexpr int kMThreads = (kMWaves + 1) * 64; // + the copy wave
constexpr int kMTile = 128;                   // tokens per LDS tile
constexpr int kMRing = 3;                     // tiles in the ring

__device__ __forceinline__ int64_t mq_visible(const ScanArgs& a, int q, int64_t base) {
  int64_t p = a.q_pos[q];
  if (p < 0 || base < 0 || base > a.total_rows) return 0;   // sees no token (also a start outside the keys)
  p = p >= a.max_ctx ? a.max_ctx - 1 : p;
  int64_t n = p + 1;
  const int64_t avail = a.total_rows - base;
  if (avail < n) n = avail;
  return n < 0 ? 0 : n;
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kMThreads) void scan_mfma_kernel(ScanArgs a, MfmaScanGrid g) {
  constexpr int NCH = D / 8;                  // 16-byte chunks per key row
  constexpr int KS = D / 32;                  // 32-channel MFMA k-steps
  constexpr int NL = kMTile * NCH / 64;       // copy instructions per tile
  __shared__ __attribute__((aligned(16))) uint4 ring[kMRing][kMTile * NCH];
  __shared__ int32_t nvis[kMQ];

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wi = (blockIdx.x % 8) * g.per_xcd + blockIdx.x / 8;
  const int r = wi / g.n_qblocks, qb = wi % g.n_qblocks;
  if (r >= g.n_ranges) return;                // padding item (uniform)
  const int s = qb / g.qblocks_per_seq;
  const int q0 = s * a.q_per_seq + (qb % g.qblocks_per_seq) * kMQ;
  const int q1 = min(min(q0 + kMQ, (s + 1) * a.q_per_seq), g.n_q);
  const int64_t base = a.seq_start[s];

  if (threadIdx.x < kMQ) {
    const int q = q0 + threadIdx.x;
    nvis[threadIdx.x] = q < q1 ? (int32_t)mq_visible(a, q, base) : 0;
  }
  __syncthreads();
  int32_t maxv = 0;
#pragma unroll
  for (int i = 0; i < kMQ; ++i) maxv = max(maxv, nvis[i]);
  const int64_t r0 = (int64_t)r * g.range_tokens;
  const int64_t r1 = min(r0 + g.range_tokens, (int64_t)maxv);
  if (r0 >= r1) return;                       // nothing visible in this range (uniform)
  const int nsteps = (int)((r1 - r0 + kMTile - 1) / kMTile);

  if (wave == kMWaves) {
    // ---------------- copy wave
    const char* kseq = reinterpret_cast<const char*>(a.idx_k + base * D);
    const int64_t last = maxv - 1;            // rows past every query's visibility are never read back
    // Byte offset within a tile of this lane's 16-byte chunk of each copy
    // instruction: the same for every tile, so a whole tile's loads are a
    // uniform tile base plus these (only the last, partial tile clamps rows).
    uint32_t off[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int slot = i * 64 + lane, tok = slot / NCH, c = (slot % NCH) ^ (tok % NCH);
      off[i] = (uint32_t)(tok * (D * 2) + c * 16);
    }
    auto issue = [&](int st) {
      const int64_t t0 = r0 + (int64_t)st * kMTile;
      uint4* dst = ring[st % kMRing];
      if (t0 + kMTile - 1 <= last) {
        const char* tb = kseq + t0 * (D * 2);
#pragma unroll
        for (int i = 0; i < NL; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(tb + off[i]),
                                           (__attribute__((address_space(3))) void*)&dst[i * 64], 16, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int slot = i * 64 + lane, tok = slot / NCH, c = (slot % NCH) ^ (tok % NCH);
          int64_t t = t0 + tok;
          t = t > last ? last : t;
          __builtin_amdgcn_global_load_lds((const void*)(kseq + t * (D * 2) + c * 16),
                                           (__attribute__((address_space(3))) void*)&dst[i * 64], 16, 0, 0);
        }
      }
    };
    issue(0);
    if (nsteps > 1) { issue(1); wait_vm<NL>(); } else { wait_vm<0>(); }
    tile_barrier();
    for (int st = 0; st < nsteps; ++st) {
      if (st + 2 < nsteps) { issue(st + 2); wait_vm<NL>(); } else { wait_vm<0>(); }
      tile_barrier();
    }
    return;
  }

  // ---------------- compute waves: queries q0 + 4*wave + j, j = 0..3.
  // Product m of a 16-token tile has rows (query j, head 4m + i) at row 4j + i,
  // so result register i of lane l holds head 4m + i of query l/16 at token
  // l%16: after the four products m = 0..3 a lane holds all 16 heads of its
  // query and token, and the weighted ReLU sum over the heads stays inside it.
  const int g4 = lane / 16, col = lane % 16;
  uint4 qa[4][KS];                            // A operand of product m: Q[q0+4w+col/4][4m + col%4][32ks + 8g4 .. +7]
  float wv[16];                               // w[query q0+4w+g4][h]
  {
    const int qr = q0 + 4 * wave + col / 4;   // this lane's A row query
    const bool qvalid = qr < q1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int h = 4 * m + col % 4;
      const bool valid = qvalid && h < g.H;
      const uint4* qp = reinterpret_cast<const uint4*>(a.idx_q + ((int64_t)(valid ? qr : q0) * g.H + (valid ? h : 0)) * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 v = qp[4 * ks + g4];
        qa[m][ks] = valid ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    const int qw4 = q0 + 4 * wave + g4;       // this lane's result query
#pragma unroll
    for (int h = 0; h < 16; ++h) wv[h] = (qw4 < q1 && h < g.H) ? a.w[(int64_t)qw4 * g.H + h] : 0.0f;
  }
  // This lane's token of each 16-token tile tt of part `part` is t0 + 32 part +
  // 16 tt + lane % 16, its score belongs to query lane/16 of the wave. The wave's
  // four score and block-maximum rows start at uniform bases; carried from tile
  // to tile are 32-bit byte offsets from them to that token's score and block
  // maximum in part 0, tile 0 (parts and tiles add immediate offsets; four rows
  // of max_ctx < 2^28 tokens keep them below 2^32) and how many of the query's
  // visible tokens lie at or past it.
  const int qw = q0 + 4 * __builtin_amdgcn_readfirstlane(wave);
  char* const sbase = reinterpret_cast<char*>(a.scores + (int64_t)qw * a.max_ctx);
  char* const bbase = reinterpret_cast<char*>(a.blockmax + (int64_t)qw * a.nblk_max);
  uint32_t so, bo;
  int32_t rem;
  {
    const int64_t tb = r0 + col;              // r0 is a multiple of 128: tb / 8 is the lane's block
    so = (uint32_t)((g4 * a.max_ctx + tb) * 4);
    bo = (uint32_t)((g4 * a.nblk_max + (tb >> 3)) * 4);
    rem = (int32_t)(nvis[4 * wave + g4] - tb);
  }
  tile_barrier();

  for (int st = 0; st < nsteps; ++st) {
    const uint4* tile = ring[st % kMRing];
#pragma unroll
    for (int part = 0; part < kMTile / 32; ++part) {
      uint4 bf[2][KS];                        // B operand: K[token col of tile tt][32ks + 8g4 .. +7]
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tok = 32 * part + 16 * tt + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bf[tt][ks] = tile[tok * NCH + ((4 * ks + g4) ^ (tok % NCH))];
      }
      v4f acc[2][4];                          // [16-token tile][head group m]
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[tt][m] = v4f{0.f, 0.f, 0.f, 0.f};
      // A wave raises its priority while it issues its products, so that the
      // matrix core is fed first and the other waves' vector work fills in
      // around it (measured 2-3% faster than equal priority).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[tt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[m][ks]),
                                                                 __builtin_bit_cast(v8bf, bf[tt][ks]),
                                                                 acc[tt][m], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        // lane: all 16 heads of query lane/16 at token col; weighted ReLU sum over them
        float y = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) y = fmaf(wv[4 * m + i], relu_f(acc[tt][m][i]), y);
        const bool vis = 32 * part + 16 * tt < rem;
        if (vis) reinterpret_cast<float*>(sbase + so)[32 * part + 16 * tt] = y;
        const float bm = max8(vis ? y : -3.402823466e38f);
        if ((lane & 7) == 0 && vis) reinterpret_cast<float*>(bbase + bo)[4 * part + 2 * tt] = bm;
      }
    }
    so += kMTile * 4;
    bo += kMTile / 8 * 4;
    rem -= kMTile;
    tile_barrier();
  }
}

bool scan_mfma_supported(int H, int D, int q_per_seq, int64_t max_ctx) {
  return q_per_seq >= 16 && H <= 16 && (D == 64 || D == 128) && max_ctx < (int64_t(1) << 28) - 1024;
}

hipError_t launch_scan_mfma(ScanArgs a, int H, int D, int n_q, hipStream_t stream) {
  if (n_q == 0 || a.max_ctx == 0) return hipSuccess;
  MfmaScanGrid g{};
  g.H = H;
  g.n_q = n_q;
  const int n_seq = (n_q + a.q_per_seq - 1) / a.q_per_seq;
  g.qblocks_per_seq = (a.q_per_seq + kMQ - 1) / kMQ;
  g.n_qblocks = n_seq * g.qblocks_per_seq;
  // About 8,192 tokens per range; shorter ranges when there are few query
  // blocks, so that the launch still spans the chip several times.
  int64_t n_ranges = (a.max_ctx + 4095) / 8192;
  const int64_t want = (1024 + g.n_qblocks - 1) / g.n_qblocks;
  if (n_ranges < want) n_ranges = want;
  const int64_t max_ranges = (a.max_ctx + 511) / 512;
  if (n_ranges > max_ranges) n_ranges = max_ranges;
  if (n_ranges < 1) n_ranges = 1;
  const int64_t per = (a.max_ctx + n_ranges - 1) / n_ranges;
  g.range_tokens = (per + kMTile - 1) / kMTile * kMTile;
  g.n_ranges = (int32_t)((a.max_ctx + g.range_tokens - 1) / g.range_tokens);
  const int64_t items = (int64_t)g.n_ranges * g.n_qblocks;
  g.per_xcd = (int32_t)((items + 7) / 8);
  const dim3 grid((uint32_t)(8 * (int64_t)g.per_xcd));
  if (D == 128)
    scan_mfma_kernel<128><<<grid, dim3(kMThreads), 0, stream>>>(a, g);
  else if (D == 64)
    scan_mfma_kernel<64><<<grid, dim3(kMThreads), 0, stream>>>(a, g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fp4kv
