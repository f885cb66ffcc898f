// Exact top-k selection for the hierarchical indexer: the best P blocks by
// block score (the candidate pool), then the best k positions inside the pool.
// [G] hierarchical sparse indexer paragraph (2,048 blocks of 8 tokens; each
// query keeps its best 512); [N] "CSA2: Sharing Main KV, Indexer K, and Top-K
// Indices Across Layers" (Full builds the pool and a fresh top-512; Reindex
// re-selects within the inherited pool).
//
// Ranking: score descending, ties to the lower block id / position. Output:
// ascending ids, -1 after the count.
//
// One 1024-thread workgroup per query. A selection of kk out of n keys is a
// radix select on order-preserving 32-bit keys: digits of 8 bits from the most
// significant, skipping bits all candidates share, with per-wave histograms in
// LDS; it ends with the exact threshold key T and how many keys equal to T
// must be taken. Then an ordered compaction: every thread owns a contiguous
// run of keys, counts (> T) and (== T) in it, a block-wide prefix sum gives
// each run the number of ties before it (ties go to lower indices) and its
// output offset, and each thread writes its selected ids in index order.
// Nothing depends on the order of atomic updates, so results are deterministic.
#include "kernels.h"

namespace fp4kv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelLdsKeys = 16384;          // keys held in LDS (64 KB)


struct SelShared {
  uint32_t keys[kSelLdsKeys];
  uint32_t hist[kSelWaves][256];
  int32_t pool[kSelLdsKeys / 8];
  uint32_t red[kSelWaves][2];
  int32_t scan[kSelWaves][2];
  uint32_t bcast[4];
};

// Block-wide exclusive prefix sums of two ints; also returns the totals.
__device__ __forceinline__ void block_scan2(SelShared& sh, int a, int b, int& ea, int& eb, int& ta, int& tb) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int xa = __shfl_up(ia, d), xb = __shfl_up(ib, d);
    if (lane >= d) { ia += xa; ib += xb; }
  }
  if (lane == kWave - 1) { sh.scan[wave][0] = ia; sh.scan[wave][1] = ib; }
  __syncthreads();
  int pa = 0, pb = 0, sa = 0, sb = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    int va = sh.scan[w][0], vb = sh.scan[w][1];
    if (w < wave) { pa += va; pb += vb; }
    sa += va; sb += vb;
  }
  ea = pa + ia - a; eb = pb + ib - b; ta = sa; tb = sb;
  __syncthreads();
}

// Threshold of a top-kk selection over n keys (key 0 = not a candidate; every
// candidate key is nonzero). Returns T and the number of keys equal to T to take.
template <typename KeyFn>
__device__ void radix_threshold(SelShared& sh, KeyFn key, int64_t n, int kk, uint32_t& T, int& take_eq) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // bits shared by all candidates
  uint32_t vor = 0, vand = 0xFFFFFFFFu;
  for (int64_t i = tid; i < n; i += kSelThreads) {
    uint32_t v = key(i);
    if (v) { vor |= v; vand &= v; }
  }
  for (int d = 1; d < kWave; d <<= 1) {
    vor |= __shfl_xor(vor, d);
    vand &= __shfl_xor(vand, d);
  }
  if (lane == 0) { sh.red[wave][0] = vor; sh.red[wave][1] = vand; }
  __syncthreads();
  vor = 0; vand = 0xFFFFFFFFu;
  for (int w = 0; w < kSelWaves; ++w) { vor |= sh.red[w][0]; vand &= sh.red[w][1]; }
  __syncthreads();
  const uint32_t diff = vor ^ vand;
  uint32_t prefix, mask;
  int kr = kk;
  if (diff == 0) {                      // all candidates equal
    T = vand; take_eq = kk;
    return;
  }
  const int top = 31 - __clz(diff);     // highest bit that differs
  int shift = (top / 8) * 8;
  mask = shift + 8 >= 32 ? 0u : ~((1u << (shift + 8)) - 1u);
  prefix = vand & mask;
  for (; shift >= 0; shift -= 8) {
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kSelThreads) {
      uint32_t v = key(i);
      if (v && (v & mask) == prefix) atomicAdd(&sh.hist[wave][(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3; suffix sums from the top bin down
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t t = 0;
        for (int w = 0; w < kSelWaves; ++w) t += sh.hist[w][4 * lane + j];
        c[j] = t; s += t;
      }
      uint32_t above = 0;  // keys in bins of higher lanes
      uint32_t incl = s;
      for (int d = 1; d < kWave; d <<= 1) {
        uint32_t x = __shfl_down(incl, d);
        if (lane + d < kWave) incl += x;
      }
      above = incl - s;
      // find the bin where the count from the top reaches kr
      uint32_t run = above;
      int found = -1; uint32_t before = 0;
      for (int j = 3; j >= 0; --j) {
        if (found < 0 && run < (uint32_t)kr && run + c[j] >= (uint32_t)kr) { found = 4 * lane + j; before = run; }
        run += c[j];
      }
      if (found >= 0) { sh.bcast[0] = (uint32_t)found; sh.bcast[1] = before; }
    }
    __syncthreads();
    const uint32_t bin = sh.bcast[0];
    kr -= (int)sh.bcast[1];
    prefix |= bin << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
  take_eq = kr;
}

// Ordered compaction: write out(slot, i) for the selected indices i in
// increasing order. Thread t owns indices [t*per, (t+1)*per).
template <typename KeyFn, typename OutFn>
__device__ int compact_selected(SelShared& sh, KeyFn key, int64_t n, uint32_t T, int take_eq, OutFn out) {
  const int tid = threadIdx.x;
  const int64_t per = (n + kSelThreads - 1) / kSelThreads;
  const int64_t lo = min((int64_t)tid * per, n), hi = min(lo + per, n);
  int gt = 0, eq = 0;
  for (int64_t i = lo; i < hi; ++i) {
    uint32_t v = key(i);
    gt += v > T;
    eq += (v == T) & (v != 0u);
  }
  int eq_before, d0, d1, d2;
  block_scan2(sh, eq, 0, eq_before, d0, d1, d2);
  int take = take_eq - eq_before;
  take = take < 0 ? 0 : (take > eq ? eq : take);
  int slot, total, d3, d4;
  block_scan2(sh, gt + take, 0, slot, d3, total, d4);
  int taken = 0;
  for (int64_t i = lo; i < hi; ++i) {
    uint32_t v = key(i);
    bool sel = v > T;
    if (!sel && v == T && v != 0u && taken < take) { sel = true; ++taken; }
    if (sel) out(slot++, i);
  }
  return total;
}

template <bool REINDEX>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem);
  const int qi = blockIdx.x, tid = threadIdx.x;

  const int64_t base = a.seq_start[qi / a.q_per_seq];
  int64_t p = a.q_pos[qi];
  p = p < 0 ? 0 : (p >= a.max_ctx ? a.max_ctx - 1 : p);
  int64_t n_vis = p + 1;
  if (a.total_rows - base < n_vis) n_vis = a.total_rows - base;
  if (n_vis < 0) n_vis = 0;

  int npool;
  int32_t* pool_row = a.pool + (int64_t)qi * a.P;
  if (!REINDEX) {
    // ---- blocks -> pool
    const int64_t nblk = (n_vis + 7) / 8;
    const float* bm = a.blockmax + (int64_t)qi * a.nblk_max;
    const int kk = (int)min<int64_t>(a.P, nblk);
    const bool in_lds = nblk <= kSelLdsKeys;
    if (in_lds) {
      for (int64_t i = tid; i < nblk; i += kSelThreads) sh.keys[i] = float_key(bm[i]);
      __syncthreads();
    }
    auto bkey = [&](int64_t i) -> uint32_t { return in_lds ? sh.keys[i] : float_key(bm[i]); };
    uint32_t T = 0; int take_eq = 0;
    if (kk > 0) radix_threshold(sh, bkey, nblk, kk, T, take_eq);
    npool = kk > 0 ? compact_selected(sh, bkey, nblk, T, take_eq, [&](int slot, int64_t i) {
      sh.pool[slot] = (int32_t)i;
      pool_row[slot] = (int32_t)i;
    }) : 0;
    for (int i = npool + tid; i < a.P; i += kSelThreads) pool_row[i] = -1;
    if (tid == 0) a.n_pool[qi] = npool;
    __syncthreads();
  } else {
    npool = a.n_pool[qi];
    npool = npool < 0 ? 0 : (npool > a.P ? a.P : npool);
    for (int i = tid; i < npool; i += kSelThreads) sh.pool[i] = pool_row[i];
    __syncthreads();
  }

  // ---- pool positions -> top-k (keys for slot j = block pool[j/8], token j%8)
  const int64_t nslot = (int64_t)npool * 8;
  const float* sc = REINDEX ? a.scores + (int64_t)qi * a.P * 8 : a.scores + (int64_t)qi * a.max_ctx;
  int nvalid = 0;
  for (int64_t j = tid; j < nslot; j += kSelThreads) {
    const int64_t b = sh.pool[j >> 3];
    const int64_t t = b * 8 + (j & 7);
    const bool ok = b >= 0 && t < n_vis;
    sh.keys[j] = ok ? float_key(REINDEX ? sc[j] : sc[t]) : 0u;
    nvalid += ok;
  }
  int d0, d1, d2;
  block_scan2(sh, nvalid, 0, d0, d1, nvalid, d2);
  const int kk = min(a.k, nvalid);
  auto tkey = [&](int64_t j) -> uint32_t { return sh.keys[j]; };
  uint32_t T = 0; int take_eq = 0;
  if (kk > 0) radix_threshold(sh, tkey, nslot, kk, T, take_eq);
  int32_t* out = a.idx_out + (int64_t)qi * a.k;
  const int nsel = kk > 0 ? compact_selected(sh, tkey, nslot, T, take_eq, [&](int slot, int64_t j) {
    out[slot] = sh.pool[j >> 3] * 8 + (int32_t)(j & 7);
  }) : 0;
  for (int i = nsel + tid; i < a.k; i += kSelThreads) out[i] = -1;
  if (tid == 0) a.n_idx[qi] = nsel;
}

size_t select_lds_bytes() { return sizeof(SelShared); }

hipError_t launch_select(const SelectArgs& a, int n_q, bool reindex, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const size_t lds = sizeof(SelShared);
  // More than 64 KB of dynamic LDS must be requested per kernel (once per process).
  static const hipError_t attr = [&] {
    hipError_t e1 = hipFuncSetAttribute((const void*)select_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipError_t e2 = hipFuncSetAttribute((const void*)select_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return e1 != hipSuccess ? e1 : e2;
  }();
  if (attr != hipSuccess) return attr;
  if (reindex)
    select_kernel<true><<<dim3(n_q), dim3(kSelThreads), lds, stream>>>(a);
  else
    select_kernel<false><<<dim3(n_q), dim3(kSelThreads), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
