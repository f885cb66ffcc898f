// Indexer scan: score(t) = sum_h w_h * max(0, q_h . k_t), fp32, plus the 8-token
// block maximum.
// [G] hierarchical sparse indexer paragraph; [T] "Mechanism 4: the hierarchical
// sparse indexer"; [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (Full scores the context; Reindex rescores the pool).
//
// Layout of the work: one wave per workgroup, one token per lane, 64 tokens
// per step. The 64 indexer-key rows of a step (64 x D bf16, contiguous in HBM
// for a Full scan, 8-row blocks for a Reindex scan) are copied into LDS by
// asynchronous global->LDS loads, 1 KB per instruction (fully coalesced). The
// chunk order is XOR-swizzled so that, when every lane then reads its own row,
// the 16-byte reads of a quarter-wave fall in distinct LDS banks. Each lane
// copies its row into registers, the next step's copy is issued, and the dot
// products run on v_dot2_f32_bf16 with the query's indexer Q as a
// wave-uniform (scalar) operand. Products and partial sums of integer-valued
// inputs are exact in fp32 while below 2^24.
#include "kernels.h"

namespace fp4kv {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
// Pointer into the constant address space: wave-uniform loads through it become
// scalar (SMEM) loads into SGPRs.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
typedef const __attribute__((address_space(4))) float* const_f32_ptr;


// Visible rows of query qi: positions 0 .. n_vis-1 of its sequence.
__device__ __forceinline__ int64_t visible_rows(const ScanArgs& a, int qi, int64_t& base) {
  base = a.seq_start[qi / a.q_per_seq];
  int64_t p = a.q_pos[qi];
  p = p < 0 ? 0 : (p >= a.max_ctx ? a.max_ctx - 1 : p);
  int64_t n = p + 1;
  int64_t avail = a.total_rows - base;
  if (avail < n) n = avail;
  return n < 0 ? 0 : n;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int H, int D, bool REINDEX>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs a) {
  constexpr int NCH = D / 8;                  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint4 tile[64 * NCH];

  const int qi = blockIdx.y;
  const int lane = threadIdx.x;
  int64_t base;
  const int64_t n_vis = visible_rows(a, qi, base);
  // token (Full) or pool-candidate (Reindex) index of this workgroup's first step
  const int64_t first = (int64_t)blockIdx.x * a.steps * 64;
  int64_t limit;                              // number of candidate slots
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

  // Position of candidate slot j, or -1 if not visible.
  auto position = [&](int64_t j) -> int64_t {
    if (!REINDEX) return j < n_vis ? j : -1;
    if (j >= limit) return -1;
    int64_t b = pool[j >> 3];
    int64_t t = b * 8 + (j & 7);
    return (b >= 0 && t < n_vis) ? t : -1;
  };

  // Asynchronous copy of 64 rows (slots s0 .. s0+63) into `tile`.
  auto issue_copy = [&](int64_t s0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int slot = i * 64 + lane;         // LDS 16-byte slot this lane fills
      const int tok = slot / NCH;             // row within the step
      const int chunk = (slot % NCH) ^ (tok % NCH);
      int64_t t = position(s0 + tok);
      if (t < 0) t = 0;                       // any in-bounds row; its score is not used
      const uint16_t* src = a.idx_k + (base + t) * D + chunk * 8;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tile[i * 64], 16, 0, 0);
    }
  };

  const_u32_ptr qw = (const_u32_ptr)(reinterpret_cast<const uint32_t*>(a.idx_q) + (int64_t)qi * H * (D / 2));
  const_f32_ptr wq = (const_f32_ptr)(a.w + (int64_t)qi * H);

  int64_t s0 = first;
  issue_copy(s0);
  for (int step = 0; step < a.steps && s0 < limit; ++step, s0 += 64) {
    wait_vmem();
    uint4 row[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) row[c] = tile[lane * NCH + (c ^ (lane % NCH))];
    wait_lds();
    if (step + 1 < a.steps && s0 + 64 < limit) issue_copy(s0 + 64);

    float score = 0.0f;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const_u32_ptr qh = qw + h * (D / 2) + c * 4;
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, row[c].x), __builtin_bit_cast(v2bf, qh[0]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, row[c].y), __builtin_bit_cast(v2bf, qh[1]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, row[c].z), __builtin_bit_cast(v2bf, qh[2]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, row[c].w), __builtin_bit_cast(v2bf, qh[3]), acc, false);
      }
      score = fmaf(wq[h], fmaxf(acc, 0.0f), score);
    }

    const int64_t j = s0 + lane;
    const int64_t t = position(j);
    if (REINDEX) {
      if (j < (int64_t)a.P * 8) a.pool_scores[(int64_t)qi * a.P * 8 + j] = t >= 0 ? score : 0.0f;
    } else {
      if (t >= 0) a.scores[(int64_t)qi * a.max_ctx + t] = score;
      float bm = t >= 0 ? score : -__builtin_inff();
      bm = fmaxf(bm, __shfl_xor(bm, 1));
      bm = fmaxf(bm, __shfl_xor(bm, 2));
      bm = fmaxf(bm, __shfl_xor(bm, 4));
      if ((lane & 7) == 0 && t >= 0) a.blockmax[(int64_t)qi * a.nblk_max + (t >> 3)] = bm;
    }
  }
}

template <int H, int D>
static hipError_t launch_scan_hd(const ScanArgs& a, int n_q, int64_t slots, bool reindex, hipStream_t stream) {
  const int64_t per_wg = (int64_t)a.steps * 64;
  const int64_t gx = (slots + per_wg - 1) / per_wg;
  dim3 grid((uint32_t)gx, (uint32_t)n_q);
  if (reindex)
    scan_kernel<H, D, true><<<grid, dim3(64), 0, stream>>>(a);
  else
    scan_kernel<H, D, false><<<grid, dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

bool scan_supported(int H, int D) {
  return (H == 4 || H == 8 || H == 16) && (D == 64 || D == 128);
}

// slots: max_ctx for a Full scan, P*8 for a Reindex scan.
hipError_t launch_scan(ScanArgs a, int H, int D, int n_q, int64_t slots, bool reindex, hipStream_t stream) {
  if (n_q == 0 || slots == 0) return hipSuccess;
  // Enough workgroups to fill 256 CUs several times over, with long runs per wave.
  const int64_t steps_total = (slots + 63) / 64;
  int steps = 16;
  while (steps > 1 && steps_total * n_q / steps < 4096) steps /= 2;
  a.steps = steps;
#define FP4KV_SCAN_CASE(HH, DD) \
  if (H == HH && D == DD) return launch_scan_hd<HH, DD>(a, n_q, slots, reindex, stream);
  FP4KV_SCAN_CASE(4, 64) FP4KV_SCAN_CASE(8, 64) FP4KV_SCAN_CASE(16, 64)
  FP4KV_SCAN_CASE(4, 128) FP4KV_SCAN_CASE(8, 128) FP4KV_SCAN_CASE(16, 128)
#undef FP4KV_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace fp4kv
