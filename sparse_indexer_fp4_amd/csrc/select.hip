// Exact top-k selection for the hierarchical indexer: the best P blocks by
// block score (the candidate pool), then the best k positions inside the pool.
// [G] hierarchical sparse indexer paragraph (the context narrowed to 2,048
// eight-token blocks, then to 512 tokens per query); [N] "CSA2: Sharing Main
// KV, Indexer K, and Top-K Indices Across Layers" (Full builds the pool and a
// fresh top-512; Reindex re-selects within the inherited pool).
//
// Ranking: score descending, ties to the lower block id / position. Output:
// ascending ids, -1 after the count.
//
// One 1024-thread workgroup per query and role (Full: one writes the pool, one
// the positions, in parallel; Reindex: one). Scores map to order-preserving 32-bit
// keys (0 = not a candidate). Each thread owns a contiguous run of 16 keys,
// held in registers. A longer block list is re-read from global memory in
// each pass, in chunks of 16,384 keys where each thread again owns 16
// consecutive keys (coalesced), and is compacted chunk by chunk. A selection of kk of the candidates is
//   1. a radix search for the threshold key T: 11-bit digits from the highest
//      bit where the candidates differ down to the lowest (bits common to all
//      candidates cost no pass, and the first pass spreads over many bins);
//      per pass, LDS atomics into one 2,048-bin histogram; each thread then
//      takes and clears two bins, one block-wide prefix sum (DPP within the
//      wave, one barrier across waves) finds the bin that reaches rank kk, and
//      its thread broadcasts it; the search stops early when that bin holds
//      exactly the keys still needed;
//   2. an ordered compaction: each run counts keys > T and == T; one
//      block-wide prefix sum of both counts gives each run its output offset
//      (the ties taken before a run are the lesser of the ties before it and
//      the ties to take, since ties go to lower indices); the runs write their
//      selected ids in index order into LDS, and the result is copied out with
//      its -1 padding in one coalesced pass.
// Wave-level scans and reductions use DPP row shifts and row broadcasts; the
// block-level ones cost one barrier. Nothing depends on the order of atomic
// updates: results are deterministic.
#include "kernels.h"

namespace fp4kv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kKPT = 16;                     // keys per thread held in registers
constexpr int kRegKeys = kSelThreads * kKPT; // 16384
constexpr int kSelWideQueries = 256;         // workgroups that fit one per CU on MI355X's 256 CUs
constexpr int kDigitBits = 11;               // radix digit: 2,048 bins
constexpr int kBins = 1 << kDigitBits;
static_assert(kBins == 2 * kSelThreads, "each thread owns two histogram bins");

struct alignas(16) SelShared {
  union {
    uint32_t hist[kBins];                    // digit histogram, zero between passes
    int32_t out[kRegKeys];                   // selected positions, ascending: written only
                                             // after the last radix pass
  };
  int32_t pool[kRegKeys / 8];                // selected blocks, ascending
  uint32_t red[kSelWaves][4];                // per-wave partial results
  uint32_t wsum[kSelWaves];                  // per-wave histogram counts of a radix pass
  uint32_t bc[4];                            // broadcast of the chosen bin
};

// Inclusive scan of x over the 64 lanes of a wave with a commutative,
// associative op of identity `ident`: DPP row shifts by 1, 2, 4, 8 within each
// 16-lane row, then row broadcasts of lane 15 and lane 31 across rows.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, uint32_t ident, Op op) {
  const int id = (int)ident;
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xF, 0xF, false));   // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xF, 0xF, false));   // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xF, 0xF, false));   // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xF, 0xF, false));   // row_shr:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x) {
  return wave_incl_scan(x, 0u, [](uint32_t p, uint32_t q) { return p + q; });
}
__device__ __forceinline__ uint32_t lane63(uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 63); }

// Keys of the calling thread's run: either 16 registers or a global-memory run.
struct RegKeys {
  static constexpr int kRun = kKPT;
  uint32_t k[kKPT];
  template <typename F> __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int j = 0; j < kKPT; ++j) f(j, k[j]);
  }
};

// Keys of two pool slots held by the calling thread (2,048 slots at most).
struct PairKeys {
  static constexpr int kRun = 2;
  uint32_t k[2];
  template <typename F> __device__ __forceinline__ void each(F f) const { f(0, k[0]); f(1, k[1]); }
};

// Keys of the calling thread's run of 16 consecutive block maxima (coalesced
// across the wave), key 0 past the end n.
__device__ __forceinline__ void load_run(const float* bm, int64_t n, int64_t i0, uint32_t (&k)[kKPT]) {
  // A block-maximum row starts 16-byte aligned only when the row length is a
  // multiple of 4 (e.g. not for 131,096 tokens = 16,387 blocks). The row's
  // misalignment m (in floats) is the same for the whole workgroup: with m != 0
  // the run is read as two halves of three aligned 16-byte loads, each starting
  // m floats early, if that window lies inside the row's visible blocks (else
  // one value at a time).
  const int m = (int)(((uintptr_t)bm >> 2) & 3);
  if (m == 0 && i0 + kKPT <= n) {
    const float4* v = reinterpret_cast<const float4*>(bm + i0);
#pragma unroll
    for (int j = 0; j < kKPT / 4; ++j) {
      const float4 f = v[j];
      k[4 * j] = float_key(f.x); k[4 * j + 1] = float_key(f.y);
      k[4 * j + 2] = float_key(f.z); k[4 * j + 3] = float_key(f.w);
    }
  } else if (m != 0 && i0 >= m && i0 - m + kKPT + 4 <= n) {
    // two halves of 8 keys, each from three aligned loads (few live registers)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4* v = reinterpret_cast<const float4*>(bm + i0 + 8 * h - m);
      const float4 f0 = v[0], f1 = v[1], f2 = v[2];
      const float w[12] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w, f2.x, f2.y, f2.z, f2.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        k[8 * h + j] = float_key(m == 1 ? w[j + 1] : (m == 2 ? w[j + 2] : w[j + 3]));
    }
  } else {
#pragma unroll
    for (int j = 0; j < kKPT; ++j) k[j] = i0 + j < n ? float_key(bm[i0 + j]) : 0u;
  }
}

// Block maxima of a long context (more than 16,384 blocks), re-read from
// global memory in each pass: chunk c of 16,384 keys gives thread t the run
// c*16384 + 16t .. +15.
struct GlobalKeys {
  static constexpr int kRun = 1 << 30;     // no register run
  const float* bm;
  int64_t n;
  template <typename F> __device__ __forceinline__ void each(F f) const {
    for (int64_t c0 = 0; c0 < n; c0 += kRegKeys) {
      uint32_t k[kKPT];
      load_run(bm, n, c0 + (int64_t)threadIdx.x * kKPT, k);
#pragma unroll
      for (int j = 0; j < kKPT; ++j) f(j, k[j]);
    }
  }
};

// OR and AND of the candidate keys (key 0 is not a candidate) and the number
// of candidates, over the workgroup.
template <typename Keys>
__device__ void candidate_summary(SelShared& sh, const Keys& keys, uint32_t& vor, uint32_t& vand, int& count) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t o = 0, n = 0xFFFFFFFFu, c = 0;
  keys.each([&](int, uint32_t v) { if (v) { o |= v; n &= v; ++c; } });
  o = lane63(wave_incl_scan(o, 0u, [](uint32_t p, uint32_t q) { return p | q; }));
  n = lane63(wave_incl_scan(n, 0xFFFFFFFFu, [](uint32_t p, uint32_t q) { return p & q; }));
  c = lane63(wave_incl_add(c));
  if (lane == 0) { sh.red[wave][0] = o; sh.red[wave][1] = n; sh.red[wave][2] = c; }
  __syncthreads();
  vor = 0; vand = 0xFFFFFFFFu; count = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) { vor |= sh.red[w][0]; vand &= sh.red[w][1]; count += (int)sh.red[w][2]; }
}

// Threshold key T of a top-kk selection among the candidates, and how many
// keys equal to T to take (INT_MAX when every key equal to T is selected).
// sh.hist is zero on entry and on return.
template <typename Keys>
__device__ void radix_threshold(SelShared& sh, const Keys& keys, int kk, uint32_t vor, uint32_t vand, uint32_t& T,
                                int& take_eq) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t diff = vor ^ vand;
  if (diff == 0) { T = vand; take_eq = kk; __syncthreads(); return; }  // all candidates equal: the first kk
  // Only bits lo..hi differ between candidates: digits of up to kDigitBits
  // bits cover them from the top, so the first pass already spreads over many
  // bins (integer scores below 2^20 differ in about 22 bits: two passes).
  const int hi = 31 - __clz(diff), lo = __builtin_ctz(diff);
  // bits above hi: every candidate agrees (2u << 31 wraps to 0, so hi = 31 gives an empty mask)
  uint32_t mask = ~((2u << hi) - 1u);
  uint32_t prefix = vand & mask;
  int kr = kk;
  take_eq = -1;
  for (int top = hi; top >= lo; top -= kDigitBits) {
    const int shift = top - (kDigitBits - 1) > lo ? top - (kDigitBits - 1) : lo;
    const int width = top - shift + 1;
    const uint32_t dmask = (1u << width) - 1u;
    keys.each([&](int, uint32_t v) {
      if (v && (v & mask) == prefix) atomicAdd(&sh.hist[(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    // Thread t owns bins 2t and 2t+1 (higher threads own higher digits): it
    // takes their counts and clears them, and the keys ranked above its bins
    // are those of the higher lanes of its wave plus those of the higher waves.
    const uint2 c = reinterpret_cast<const uint2*>(sh.hist)[threadIdx.x];
    reinterpret_cast<uint2*>(sh.hist)[threadIdx.x] = make_uint2(0u, 0u);
    const uint32_t t = c.x + c.y;
    const uint32_t incl = wave_incl_add(t);
    const uint32_t wtot = lane63(incl);
    if (lane == 63) sh.wsum[wave] = wtot;
    __syncthreads();
    uint32_t above = wtot - incl;
#pragma unroll
    for (int w = kSelWaves - 1; w > 0; --w)
      if (w > wave) above += sh.wsum[w];
    if (above < (uint32_t)kr && above + t >= (uint32_t)kr) {   // one thread: its bins hold rank kr
      const bool upper = above + c.y >= (uint32_t)kr;
      sh.bc[0] = 2u * threadIdx.x + (upper ? 1u : 0u);
      sh.bc[1] = upper ? above : above + c.y;
      sh.bc[2] = upper ? c.y : c.x;
    }
    __syncthreads();
    const uint32_t bin = sh.bc[0];
    kr -= (int)sh.bc[1];
    const int in_bin = (int)sh.bc[2];
    prefix |= bin << shift;
    mask |= dmask << shift;
    if (in_bin == kr) {           // every key left in the bin is selected
      take_eq = 0x7FFFFFFF;
      break;
    }
  }
  // bits below the last digit: all candidates share them (common low bits)
  T = prefix | (vand & ~mask);
  if (take_eq < 0) take_eq = kr;
}

// Ordered compaction; out(slot, local index j) for selected keys of this run.
// One scan of (count > T, count == T): the ties taken before a run are
// min(ties before it, take_eq), because ties are taken from the lowest index.
template <typename Keys, typename Out>
__device__ int compact_selected(SelShared& sh, const Keys& keys, uint32_t T, int take_eq, Out out) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t gt = 0, eq = 0;
  keys.each([&](int, uint32_t v) { gt += v > T; eq += (v == T) & (v != 0u); });
  const uint32_t igt = wave_incl_add(gt), ieq = wave_incl_add(eq);
  if (lane == 63) { sh.red[wave][0] = igt; sh.red[wave][1] = ieq; }
  __syncthreads();
  int gt_before = (int)(igt - gt), eq_before = (int)(ieq - eq), gt_total = 0, eq_total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int u = (int)sh.red[w][0], v = (int)sh.red[w][1];
    if (w < wave) { gt_before += u; eq_before += v; }
    gt_total += u; eq_total += v;
  }
  const int taken_before = min(eq_before, take_eq);
  int take = take_eq - eq_before;
  take = take < 0 ? 0 : (take > (int)eq ? (int)eq : take);
  int slot = gt_before + taken_before;
  int taken = 0;
  if constexpr (Keys::kRun <= 32) {
    // register run: collect the selected indices, then write only those
    uint32_t selmask = 0;
    keys.each([&](int j, uint32_t v) {
      bool sel = v > T;
      if (!sel && v == T && v != 0u && taken < take) { sel = true; ++taken; }
      selmask |= (uint32_t)sel << j;
    });
    while (selmask) {
      const int j = __builtin_ctz(selmask);
      selmask &= selmask - 1u;
      out(slot++, j);
    }
  } else {
    keys.each([&](int j, uint32_t v) {
      bool sel = v > T;
      if (!sel && v == T && v != 0u && taken < take) { sel = true; ++taken; }
      if (sel) out(slot++, j);
    });
  }
  return gt_total + min(eq_total, take_eq);
}

// Ordered compaction of a long block list, chunk by chunk: within a chunk as
// compact_selected; the ties taken so far and the slots filled so far carry
// from one chunk to the next. out(slot, block id).
template <typename Out>
__device__ int compact_chunks(SelShared& sh, const GlobalKeys& keys, uint32_t T, int take_eq, Out out) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int filled = 0, ties_left = take_eq;
  for (int64_t c0 = 0; c0 < keys.n; c0 += kRegKeys) {
    const int64_t i0 = c0 + (int64_t)threadIdx.x * kKPT;
    uint32_t k[kKPT];
    load_run(keys.bm, keys.n, i0, k);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kKPT; ++j) { gt += k[j] > T; eq += (k[j] == T) & (k[j] != 0u); }
    const uint32_t igt = wave_incl_add(gt), ieq = wave_incl_add(eq);
    if (lane == 63) { sh.red[wave][0] = igt; sh.red[wave][1] = ieq; }
    __syncthreads();
    int gt_before = (int)(igt - gt), eq_before = (int)(ieq - eq), gt_total = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int u = (int)sh.red[w][0], v = (int)sh.red[w][1];
      if (w < wave) { gt_before += u; eq_before += v; }
      gt_total += u; eq_total += v;
    }
    __syncthreads();                         // sh.red is rewritten by the next chunk
    const int ties_here = min(eq_total, ties_left);
    int take = ties_here - eq_before;
    take = take < 0 ? 0 : (take > (int)eq ? (int)eq : take);
    int slot = filled + gt_before + min(eq_before, ties_here);
    int taken = 0;
    uint32_t selmask = 0;
#pragma unroll
    for (int j = 0; j < kKPT; ++j) {
      bool sel = k[j] > T;
      if (!sel && k[j] == T && k[j] != 0u && taken < take) { sel = true; ++taken; }
      selmask |= (uint32_t)sel << j;
    }
    while (selmask) {
      const int j = __builtin_ctz(selmask);
      selmask &= selmask - 1u;
      out(slot++, i0 + j);
    }
    filled += gt_total + ties_here;
    ties_left -= ties_here;
  }
  return filled;
}

// Keys of KPT consecutive token candidates per thread.
template <int KPT>
struct TokenKeys {
  static constexpr int kRun = KPT;
  uint32_t k[KPT];
  template <typename F> __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int j = 0; j < KPT; ++j) f(j, k[j]);
  }
};

// Top-k positions among the positions of the npool blocks in sh.pool
// (ascending), dropping those whose key is below tmin. Candidate c (< npool*8)
// is position pool[c/8]*8 + c%8; thread t holds candidates KPT t .. KPT t +
// KPT - 1, so candidates, and with them ties, run in ascending position order
// over the threads.
template <bool REINDEX, int KPT>
__device__ void token_search(SelShared& sh, const SelectArgs& a, int qi, int npool, uint32_t tmin, int64_t n_vis) {
  static_assert(KPT % 4 == 0 && KPT <= kKPT, "candidate runs of whole 4-position groups");
  const int tid = threadIdx.x;
  TokenKeys<KPT> keys;
#pragma unroll
  for (int g = 0; g < KPT / 4; ++g) {
    const int c = tid * KPT + 4 * g;                   // first candidate of this group of 4
    const int jb = c >> 3, e0 = c & 7;                 // pool slot, position in its block (0 or 4)
    const int64_t b = jb < npool ? (int64_t)sh.pool[jb] : -1;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if (REINDEX) {
      if (jb < npool) {
        const float4 f = *reinterpret_cast<const float4*>(a.scores + ((int64_t)qi * a.P + jb) * 8 + e0);
        s[0] = f.x; s[1] = f.y; s[2] = f.z; s[3] = f.w;
      }
    } else if (b >= 0 && b * 8 + e0 + 4 <= n_vis && ((a.max_ctx & 3) == 0)) {
      const float4 f = *reinterpret_cast<const float4*>(a.scores + (int64_t)qi * a.max_ctx + b * 8 + e0);
      s[0] = f.x; s[1] = f.y; s[2] = f.z; s[3] = f.w;
    } else if (b >= 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[e] = b * 8 + e0 + e < n_vis ? a.scores[(int64_t)qi * a.max_ctx + b * 8 + e0 + e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = b >= 0 && b * 8 + e0 + e < n_vis;
      const uint32_t key = ok ? float_key(s[e]) : 0u;
      keys.k[4 * g + e] = key >= tmin ? key : 0u;
    }
  }
  // float_key never gives 0 for a finite score, so the candidates are the visible
  // positions (those scoring >= tmin)
  uint32_t vor, vand; int nvalid;
  candidate_summary(sh, keys, vor, vand, nvalid);
  const int kk = min(a.k, nvalid);
  int32_t* out = a.idx_out + (int64_t)qi * a.k;
  int nsel = 0;
  if (kk > 0) {
    uint32_t T; int take_eq;
    radix_threshold(sh, keys, kk, vor, vand, T, take_eq);
    nsel = compact_selected(sh, keys, T, take_eq, [&](int slot, int j) {
      const int c = tid * KPT + j;
      sh.out[slot] = sh.pool[c >> 3] * 8 + (c & 7);
    });
  }
  __syncthreads();
  for (int i = tid; i < a.k; i += kSelThreads) out[i] = i < nsel ? sh.out[i] : -1;
  if (tid == 0) a.n_idx[qi] = nsel;
}

// WIDE: at most one workgroup per CU is wanted (few queries), so the kernel
// may use up to 128 VGPRs; otherwise it is held to 64, so that two 1,024-thread
// workgroups share a CU (measured: 32 queries 18.9 against 19.7 us, 4,096
// queries 405 against 309 us).
template <bool REINDEX, bool WIDE>
__global__ __launch_bounds__(kSelThreads, WIDE ? 4 : 8) void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int qi = blockIdx.x, tid = threadIdx.x;
  // histograms start at zero (the first barrier comes before any count)
  if (tid < kBins / 4) reinterpret_cast<uint4*>(sh.hist)[tid] = make_uint4(0u, 0u, 0u, 0u);

  const int64_t base = a.seq_start ? a.seq_start[qi / a.q_per_seq] : 0;   // paged storage: no base
  int64_t p = a.q_pos[qi];
  p = p >= a.max_ctx ? a.max_ctx - 1 : p;
  int64_t n_vis = p < 0 ? 0 : p + 1;                    // a negative position sees no token
  if (base < 0 || base > a.total_rows) n_vis = 0;       // as the scan: a start outside the keys sees nothing
  else if (a.total_rows - base < n_vis) n_vis = a.total_rows - base;

  int npool;
  int32_t* pool_row = a.pool + (int64_t)qi * a.P;
  // Lowest token key that can be selected (0: every visible pool position). A
  // selected token's score is at least the k-th best pool block maximum, which is
  // at least the pool's threshold key T; so when the pool holds >= k blocks, the
  // positions scoring below T can be dropped before the token search (each pool
  // block keeps its best token, so >= k candidates remain, and the selection is
  // unchanged, ties included).
  uint32_t tmin = 0u;
  if (!REINDEX) {
    // ---- blocks -> pool. When the pool holds >= k blocks, the position search
    // needs only the k best blocks, not the whole pool: every position of the
    // global top-k over all visible positions lies in one of them (each block
    // ranked ahead of its block holds a distinct position ranked ahead of it:
    // its best one, ahead on score or, on a tie, on the lower position), and
    // that global top-k is then the pool's top-k.
    // With two workgroups per query (grid y = 2: few queries) they run side by
    // side: role 0 (blockIdx.y == 0) selects and writes the pool; role 1 ranks
    // the blocks for a pool of min(k, blocks) and searches those 8k positions.
    // With one (grid y = 1: more queries than the chip runs two workgroups of
    // at once) a workgroup writes the pool and then narrows it to its k best
    // blocks: the pool is the first P blocks in the order (maximum descending,
    // index ascending) and the k best blocks are the first k, so ranking the
    // pool's blocks gives role 1's blocks, ties included, without a second
    // search over every block maximum.
    const bool split_roles = gridDim.y == 2;
    const bool idx_role = !split_roles || blockIdx.y == 1;
    const bool pool_role = !split_roles || blockIdx.y == 0;
    const int64_t nblk = (n_vis + 7) / 8;
    const float* bm = a.blockmax + (int64_t)qi * a.nblk_max;
    const int kk = (int)min<int64_t>(split_roles && idx_role && a.P >= a.k ? a.k : a.P, nblk);
    npool = 0;
    if (kk > 0 && nblk <= kRegKeys) {
      RegKeys keys;
      const int64_t i0 = (int64_t)tid * kKPT;
      load_run(bm, nblk, i0, keys.k);
      uint32_t vor, vand, T; int cnt, take_eq;
      candidate_summary(sh, keys, vor, vand, cnt);
      radix_threshold(sh, keys, kk, vor, vand, T, take_eq);
      npool = compact_selected(sh, keys, T, take_eq, [&](int slot, int j) { sh.pool[slot] = (int32_t)(i0 + j); });
      tmin = T;
    } else if (kk > 0) {
      GlobalKeys keys{bm, nblk};
      uint32_t vor, vand, T; int cnt, take_eq;
      candidate_summary(sh, keys, vor, vand, cnt);
      radix_threshold(sh, keys, kk, vor, vand, T, take_eq);
      npool = compact_chunks(sh, keys, T, take_eq, [&](int slot, int64_t b) { sh.pool[slot] = (int32_t)b; });
      tmin = T;
    }
    __syncthreads();
    if (pool_role) {
      for (int i = tid; i < a.P; i += kSelThreads) pool_row[i] = i < npool ? sh.pool[i] : -1;
      if (tid == 0) a.n_pool[qi] = npool;
      if (!idx_role) return;
    }
    if (!split_roles && a.P >= a.k && npool > a.k) {
      // narrow the pool (at most 2,048 slots: two per thread) to its k best
      // blocks, in place and in pool order; the keys come back from the block
      // maxima. Every slot is read here, before the barrier in
      // candidate_summary, and written only by the compaction after it.
      PairKeys pk;
      int32_t pb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int jb = 2 * tid + h;
        pb[h] = jb < npool ? sh.pool[jb] : 0;
        pk.k[h] = jb < npool ? float_key(bm[pb[h]]) : 0u;
      }
      uint32_t vor, vand, T; int cnt, take_eq;
      candidate_summary(sh, pk, vor, vand, cnt);
      radix_threshold(sh, pk, a.k, vor, vand, T, take_eq);
      npool = compact_selected(sh, pk, T, take_eq, [&](int slot, int j) { sh.pool[slot] = pb[j]; });
      tmin = T;
      __syncthreads();
    }
    if (npool < a.k) tmin = 0u;
  } else {
    npool = a.n_pool[qi];
    npool = npool < 0 ? 0 : (npool > a.P ? a.P : npool);
    for (int i = tid; i < npool; i += kSelThreads) sh.pool[i] = pool_row[i];
    __syncthreads();
  }

  // ---- pool positions -> top-k: 4 candidates per thread when they fit (a
  // pool narrowed to k <= 512 blocks), else 16, so that no thread runs its
  // passes over a run of empty keys
  if (npool <= kSelThreads / 2) token_search<REINDEX, 4>(sh, a, qi, npool, tmin, n_vis);
  else token_search<REINDEX, 16>(sh, a, qi, npool, tmin, n_vis);
}

hipError_t launch_select(const SelectArgs& a, int n_q, bool reindex, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  // Full: two workgroups per query (pool, positions), the query index fastest
  // so that both land on the same XCD, while every workgroup fits on the chip
  // at once (two per CU); beyond that one per query does both in turn, which
  // searches the block maxima once instead of twice. Reindex: one (the pool is
  // given).
  const int roles = reindex || n_q > kSelWideQueries ? 1 : 2;
  const bool wide = (int64_t)n_q * roles <= kSelWideQueries;
  const dim3 grid((uint32_t)n_q, (uint32_t)roles);
  if (reindex && wide)
    select_kernel<true, true><<<grid, dim3(kSelThreads), 0, stream>>>(a);
  else if (reindex)
    select_kernel<true, false><<<grid, dim3(kSelThreads), 0, stream>>>(a);
  else if (wide)
    select_kernel<false, true><<<grid, dim3(kSelThreads), 0, stream>>>(a);
  else
    select_kernel<false, false><<<grid, dim3(kSelThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
