// Indexer scan: score(t) = sum_h w_h * max(0, q_h . k_t), fp32, plus the 8-token
// block maximum.
// [G] hierarchical sparse indexer paragraph; [T] "Mechanism 4: the hierarchical
// sparse indexer"; [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (Full scores the context; Reindex rescores the pool).
//
// Layout of the work: one wave per workgroup, 64 tokens per step, 16 steps
// per workgroup. The q . k products of a step run on the matrix cores: one
// v_mfma_f32_16x16x32_bf16 per 32 channels and 16-token tile, with the query
// (16 heads x D, held in VGPRs for the whole workgroup) as the A operand and
// 16 tokens' keys as the B operand. The B operand is loaded straight from HBM
// into VGPRs (each load takes 64 contiguous bytes of 16 key rows); the next
// step's loads are issued before the current step is computed, so two steps
// of keys are in flight per wave. A lane of an MFMA result holds 4 heads of one
// token; ReLU and the head weights are applied there, and the four 16-lane
// groups of four tiles are reduce-scattered with v_permlane32_swap and
// v_permlane16_swap so that lane l ends with the score of token l of the step.
// Products and partial sums of integer-valued inputs are exact in fp32 while
// below 2^24.
//
// Scores stay in LDS until the workgroup's last step and are stored together,
// so the loop issues loads only and the compiler's partial vmcnt waits cover
// exactly the keys a step needs.
#include "quant_dev.h"

namespace fp4kv {

constexpr int kScanSteps = 16;              // 64-token steps per workgroup

// Visible rows of query qi: positions 0 .. n_vis-1 of its sequence. Paged
// storage bounds them by max_ctx only (the block table maps every position).
template <bool PAGED>
__device__ __forceinline__ int64_t visible_rows(const ScanArgs& a, int qi, int64_t& base) {
  base = PAGED ? 0 : a.seq_start[qi / a.q_per_seq];
  int64_t p = a.q_pos[qi];
  if (p < 0) return 0;                                  // sees no token
  if (!PAGED && (base < 0 || base > a.total_rows)) {    // a start outside the keys: no visible row
    base = 0;
    return 0;
  }
  p = p >= a.max_ctx ? a.max_ctx - 1 : p;
  int64_t n = p + 1;
  if (!PAGED) {
    int64_t avail = a.total_rows - base;
    if (avail < n) n = avail;
  }
  return n < 0 ? 0 : n;
}

// Scores (and block maxima) of slots first .. first + steps*64 - 1 of query qi,
// whose visible rows are positions 0 .. n_vis-1 starting at key row base (one
// wave; res holds the range's scores until they are stored).
template <int H, int D, bool REINDEX, bool PAGED>
__device__ __forceinline__ void scan_range(const ScanArgs& a, int qi, int64_t first, int64_t n_vis, int64_t base,
                                           float* res) {
  constexpr int MAXSTEPS = kScanSteps;
  constexpr int PD = 2;                       // steps of loads in flight
  constexpr int KS = D / 32;
  const int lane = threadIdx.x;
  int64_t limit;
  int32_t npool = 0;
  const int32_t* pool = nullptr;
  if (REINDEX) {
    npool = a.n_pool[qi];
    npool = npool < 0 ? 0 : (npool > a.P ? a.P : npool);
    limit = (int64_t)npool * 8;
    pool = a.pool + (int64_t)qi * a.P;
  } else {
    limit = n_vis;
  }
  if (n_vis == 0 || first >= limit) return;
  const int nsteps = (int)min<int64_t>(a.steps, (limit - first + 63) / 64);

  auto position = [&](int64_t j) -> int64_t {
    if (!REINDEX) return j < n_vis ? j : -1;
    if (j >= limit) return -1;
    int64_t b = pool[j >> 3];
    int64_t t = b * 8 + (j & 7);
    return (b >= 0 && t < n_vis) ? t : -1;
  };

  const int g = lane >> 4, col = lane & 15;
  const char* seq_k = reinterpret_cast<const char*>(a.idx_k + base * D);
  const int64_t seq = qi / a.q_per_seq;
  // Paged Full scan: the 64 tokens of a step lie in one page (pages are >= 64
  // rows and steps 64-aligned), so lane st holds the physical page of step st,
  // read once here; an unmapped page reads row 0 (the block table must map
  // every visible position).
  int32_t step_page = -1;
  if (PAGED && !REINDEX && lane < MAXSTEPS) {
    const int64_t page = (first + 64 * (int64_t)lane) >> a.map.log2_page;
    if (page < a.map.max_pages) step_page = a.map.block_table[seq * a.map.max_pages + page];
  }
  // B operand of tile tt, k-step ks: K[token 16tt + col][32ks + 8g .. +7], loaded
  // straight into registers (64 contiguous bytes of each of 16 rows per load)
  auto load_step = [&](uint4 (&b)[4][KS], int st) {
    const int64_t s0 = first + (int64_t)st * 64;
    int64_t prow0 = 0;
    if (PAGED && !REINDEX) {
      const int64_t gp = __builtin_amdgcn_readlane(step_page, st);
      prow0 = (gp >= 0 && gp < a.map.n_pages) ? (gp << a.map.log2_page) + (s0 & ((int64_t(1) << a.map.log2_page) - 1))
                                               : 0;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      int64_t t = position(s0 + 16 * tt + col);
      if (t < 0) t = 0;                       // any in-bounds row; its score is not used
      if (PAGED) {
        if (REINDEX) {
          t = paged_row(a.map, seq, t);
          if (t < 0) t = 0;
        } else {
          t = prow0 + 16 * tt + col;           // the step's rows are consecutive in its page
        }
      }
      const uint4* rp = reinterpret_cast<const uint4*>(seq_k + t * (D * 2));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[tt][ks] = rp[4 * ks + g];
    }
  };

  uint4 qa[KS];
  float wv[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.idx_q + ((int64_t)qi * H + (col < H ? col : 0)) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = qp[4 * ks + g];
      qa[ks] = col < H ? v : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = 4 * g + i < H ? a.w[(int64_t)qi * H + 4 * g + i] : 0.0f;
  }

  auto compute_step = [&](const uint4 (&bf)[4][KS], int st) {
    v4f acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[ks]),
                                                          __builtin_bit_cast(v8bf, bf[tt][ks]), acc[tt], 0, 0, 0);
    float p[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float v = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(wv[i], relu_f(acc[tt][i]), v);
      p[tt] = v;
    }
    const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
    const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
    const float s02 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
    const float s13 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
    res[st * 64 + lane] = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  };

  uint4 buf[PD][4][KS];
#pragma unroll
  for (int i = 0; i < PD - 1; ++i)
    if (i < nsteps) load_step(buf[i], i);
  for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      const int st = s0 + i;
      if (st < nsteps) {
        if (st + PD - 1 < nsteps) load_step(buf[(i + PD - 1) % PD], st + PD - 1);
        compute_step(buf[i], st);
      }
    }
  }

  // Store the workgroup's results: scores (and block maxima) of nsteps*64
  // slots. All scores are read from LDS first (one wait), the block maxima come
  // from DPP exchanges inside each group of 8 lanes, and the stores are issued
  // back to back, so the workgroup leaves its slot soon after its last load.
  float sv[MAXSTEPS];
#pragma unroll
  for (int step = 0; step < MAXSTEPS; ++step) sv[step] = step < nsteps ? res[step * 64 + lane] : 0.0f;
#pragma unroll
  for (int step = 0; step < MAXSTEPS; ++step) {
    if (step < nsteps) {
      const int64_t j = first + (int64_t)step * 64 + lane;
      const int64_t t = position(j);
      if (REINDEX) {
        if (j < (int64_t)a.P * 8) a.pool_scores[(int64_t)qi * a.P * 8 + j] = t >= 0 ? sv[step] : 0.0f;
      } else {
        if (t >= 0) a.scores[(int64_t)qi * a.max_ctx + t] = sv[step];
        const float bm = max8(t >= 0 ? sv[step] : -__builtin_inff());
        if ((lane & 7) == 0 && t >= 0) a.blockmax[(int64_t)qi * a.nblk_max + (t >> 3)] = bm;
      }
    }
  }
}

// The work list of a Full scan over queries of different lengths: items are
// (query, range of steps*64 slots) over each query's visible rows only, in
// query order. A persistent grid of list_wgs one-wave workgroups (as many as
// the GPU holds at once) walks it, item i taken by workgroup i mod list_wgs, so
// no workgroup is spent on a range past a short query's end. Each workgroup builds the list's prefix (first item of
// every query) itself from q_pos and seq_start: no extra launch.
constexpr int kListMaxQueries = 512;

__device__ __forceinline__ int32_t wave_incl_sum(int32_t x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o);
    if ((int)threadIdx.x >= o) x += y;
  }
  return x;
}

template <int H, int D, bool PAGED>
__device__ __forceinline__ void scan_list(const ScanArgs& a, float* res) {
  __shared__ int32_t item0[kListMaxQueries + 1];   // first item of each query (queries past 64)
  const int lane = threadIdx.x;
  const int64_t R = (int64_t)a.steps * 64;
  int32_t carry = 0;
  int32_t my_first = 0, my_end = 0;                // items of query `lane` (first 64 queries)
  int64_t my_vis = 0, my_base = 0;
  for (int c = 0; c < a.n_q; c += 64) {
    const int q = c + lane;
    int64_t b = 0, nv = 0;
    if (q < a.n_q) nv = visible_rows<PAGED>(a, q, b);
    const int32_t cnt = (int32_t)((nv + R - 1) / R);
    const int32_t incl = wave_incl_sum(cnt);
    if (q < a.n_q) item0[q] = carry + incl - cnt;
    if (c == 0) {
      my_first = carry + incl - cnt;
      my_end = carry + incl;
      my_vis = nv;
      my_base = b;
    }
    carry += __shfl(incl, 63);
  }
  __syncthreads();
  const int32_t total = carry;
  for (int32_t item = blockIdx.x; item < total; item += a.list_wgs) {
    int q;
    int64_t n_vis, base;
    if (a.n_q <= 64) {                     // the lane whose query holds the item
      const uint64_t m = __builtin_amdgcn_ballot_w64(lane < a.n_q && my_first <= item && item < my_end);
      if (m == 0) break;                   // (never: the queries' items partition [0, total))
      q = (int)__builtin_ctzll(m);
      n_vis = ((int64_t)__builtin_amdgcn_readlane((int)(my_vis >> 32), q) << 32) |
              (uint32_t)__builtin_amdgcn_readlane((int)my_vis, q);
      base = ((int64_t)__builtin_amdgcn_readlane((int)(my_base >> 32), q) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)my_base, q);
    } else {                               // binary search: the last query whose first item is <= item
      int lo = 0, hi = a.n_q;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (item0[mid] <= item) lo = mid;
        else hi = mid;
      }
      q = __builtin_amdgcn_readfirstlane(lo);
      n_vis = visible_rows<PAGED>(a, q, base);
    }
    const int32_t first_item = a.n_q <= 64 ? __builtin_amdgcn_readlane(my_first, q) : item0[q];
    scan_range<H, D, false, PAGED>(a, q, (int64_t)(item - first_item) * R, n_vis, base, res);
  }
}

template <int H, int D, bool REINDEX, bool PAGED>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs a) {
  __shared__ float res[kScanSteps * 64];        // scores of the current range, stored at its end
  if constexpr (!REINDEX) {
    if (a.list_wgs > 0) {
      if ((int)blockIdx.x >= a.list_wgs) {      // workgroups of the append carried by this launch
        if constexpr (!PAGED) {
          const int64_t gid = (int64_t)(blockIdx.x - a.list_wgs) * 64 + threadIdx.x;
          if (gid < append_items(a.app)) append_item(a.app, gid);
        }
        return;
      }
      scan_list<H, D, PAGED>(a, res);
      return;
    }
    if constexpr (!PAGED) {
      if (a.app_rows > 0 && (int)blockIdx.y >= a.n_q) {   // a row of the append carried by this launch
        const int64_t gid = ((int64_t)(blockIdx.y - a.n_q) * gridDim.x + blockIdx.x) * 64 + threadIdx.x;
        if (gid < append_items(a.app)) append_item(a.app, gid);
        return;
      }
    }
  }
  const int qi = blockIdx.y;
  int64_t base;
  const int64_t n_vis = visible_rows<PAGED>(a, qi, base);
  scan_range<H, D, REINDEX, PAGED>(a, qi, (int64_t)blockIdx.x * a.steps * 64, n_vis, base, res);
}

// Workgroups of a Full scan instance that the GPU holds resident at once
// (occupancy per CU x CUs), asked of the runtime once per instance; the
// work-list scan's persistent grid is that large, so every workgroup runs from
// the start and none waits for a slot.
template <int H, int D, bool PAGED>
static int64_t resident_scan_wgs() {
  static const int64_t n = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return (int64_t)2048;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&scan_kernel<H, D, false, PAGED>), 64, 0) != hipSuccess ||
        per_cu < 1)
      return (int64_t)2048;
    return (int64_t)cus * per_cu;
  }();
  return n;
}

template <int H, int D>
static hipError_t launch_scan_hd(ScanArgs a, int n_q, int64_t slots, bool reindex, hipStream_t stream) {
  const int64_t per_wg = (int64_t)a.steps * 64;
  const int64_t gx = (slots + per_wg - 1) / per_wg;
  dim3 grid((uint32_t)gx, (uint32_t)(n_q + a.app_rows));
  if (a.list_wgs > 0) {                     // work-list scan: a persistent grid of resident workgroups
    const int64_t upper = (int64_t)n_q * gx;
    const int64_t res = a.map.block_table ? resident_scan_wgs<H, D, true>() : resident_scan_wgs<H, D, false>();
    a.list_wgs = (int32_t)(upper < res ? upper : res);
    grid = dim3((uint32_t)(a.list_wgs + a.app_wgs), 1u);
  }
  const bool paged = a.map.block_table != nullptr;
  if (reindex) {
    if (paged) scan_kernel<H, D, true, true><<<grid, dim3(64), 0, stream>>>(a);
    else scan_kernel<H, D, true, false><<<grid, dim3(64), 0, stream>>>(a);
  } else {
    if (paged) scan_kernel<H, D, false, true><<<grid, dim3(64), 0, stream>>>(a);
    else scan_kernel<H, D, false, false><<<grid, dim3(64), 0, stream>>>(a);
  }
  return hipGetLastError();
}

bool scan_supported(int H, int D) {
  return (H == 4 || H == 8 || H == 16) && (D == 64 || D == 128);
}

// slots: max_ctx for a Full scan, P*8 for a Reindex scan.
hipError_t launch_scan(ScanArgs a, int H, int D, int n_q, int64_t slots, bool reindex, hipStream_t stream,
                       const AppendJob* app) {
  const int64_t app_items = app ? app->n_rows * (app->C >> (app->fmt == kKvMxfp4 ? 5 : 4)) : 0;
  auto separate_append = [&]() {
    return launch_quantize_append(app->fmt, app->src, app->n_rows, app->C, app->dd, app->codes, app->scales,
                                  app->cap_rows, stream);
  };
  if (n_q == 0 || slots == 0) return app_items > 0 ? separate_append() : hipSuccess;
  // Long runs per wave (16 steps of 64 tokens) while that still gives >= 2,048
  // one-wave workgroups; fewer queries or slots (a Reindex over a few queries'
  // pools, a short context) take shorter runs, down to 2 steps, so that enough
  // waves keep loads in flight.
  const int64_t steps_total = (slots + 63) / 64;
  int steps = kScanSteps;
  while (steps > 2 && (int64_t)n_q * ((steps_total + steps - 1) / steps) < 2048) steps /= 2;
  a.steps = steps;
  a.n_q = n_q;
  a.app_rows = 0;
  a.app_wgs = 0;
  // A Full scan of up to kListMaxQueries queries walks a work list (see
  // scan_list) with a persistent grid sized in launch_scan_hd; 1 marks it
  // here. An append it carries runs in workgroups after that grid.
  a.list_wgs = (!reindex && n_q >= 2 && n_q <= kListMaxQueries && slots <= INT32_MAX) ? 1 : 0;
  if (a.list_wgs > 0 && app_items > 0 && a.map.block_table == nullptr) {
    a.app = *app;
    a.app_wgs = (int32_t)((app_items + 63) / 64);
  } else if (app_items > 0) {
    // A contiguous Full scan carries the append in extra grid rows of 64-thread
    // workgroups, one item per thread (the scan never reads the main KV); other
    // scans, or a grid that would pass 65,535 rows, launch it on its own first.
    const int64_t gx = (slots + (int64_t)steps * 64 - 1) / ((int64_t)steps * 64);
    const int64_t rows = (app_items + gx * 64 - 1) / (gx * 64);
    if (a.list_wgs == 0 && !reindex && a.map.block_table == nullptr && n_q + rows <= 65535) {
      a.app = *app;
      a.app_rows = (int32_t)rows;
    } else {
      hipError_t e = separate_append();
      if (e != hipSuccess) return e;
    }
  }
#define FP4KV_SCAN_CASE(HH, DD) \
  if (H == HH && D == DD) return launch_scan_hd<HH, DD>(a, n_q, slots, reindex, stream);
  FP4KV_SCAN_CASE(4, 64) FP4KV_SCAN_CASE(8, 64) FP4KV_SCAN_CASE(16, 64)
  FP4KV_SCAN_CASE(4, 128) FP4KV_SCAN_CASE(8, 128) FP4KV_SCAN_CASE(16, 128)
#undef FP4KV_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace fp4kv
