// Indexer scan: score(t) = sum_h w_h * max(0, q_h . k_t), fp32, plus the 8-token
// block maximum.
// [G] hierarchical sparse indexer paragraph; [T] "Mechanism 4: the hierarchical
// sparse indexer"; [N] "CSA2: Sharing Main KV, Indexer K, and Top-K Indices
// Across Layers" (Full scores the context; Reindex rescores the pool).
//
// Layout of the work: one wave per workgroup, one token per lane, 64 tokens
// per step, 8 steps per workgroup. The 64 indexer-key rows of a step
// (64 x D bf16, contiguous in HBM for a Full scan, 8-row blocks for a Reindex
// scan) are copied into LDS by asynchronous global->LDS loads, 1 KB per
// instruction (fully coalesced). The chunk order is XOR-swizzled so that, when
// every lane then reads its own row, the 16-byte reads of a quarter-wave fall
// in distinct LDS banks. Each lane copies its row into registers and the next
// step's copy is issued before the dot products, so one tile is always in
// flight per wave.
//
// The dot products run on v_dot2_f32_bf16. The indexer query is held in
// registers: lane j of every 16-lane row holds head j's query, and each
// v_dot2 takes its query operand by a DPP row broadcast from lane h. This keeps
// the scalar memory path (and its waits) out of the inner loop. Products and
// partial sums of integer-valued inputs are exact in fp32 while below 2^24.
//
// Scores stay in LDS until the workgroup's last step and are stored together:
// a store issued inside the loop would count in the vmcnt that the next step's
// wait for its tile uses.
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
  if (p < 0) return 0;                                  // sees no token
  p = p >= a.max_ctx ? a.max_ctx - 1 : p;
  int64_t n = p + 1;
  int64_t avail = a.total_rows - base;
  if (avail < n) n = avail;
  return n < 0 ? 0 : n;
}


// Sixteen v_dot2c_f32_bf16 with the q operand broadcast (DPP row_newbcast)
// from lane 4G+i of each 16-lane row: acc[i] += q(lane 4G+i)[d] . k[d] for
// four consecutive bf16 pairs d and the four heads of group G. The compiler
// neither folds a DPP move into v_dot2c nor sees DPP inside inline asm, so the
// block protects itself: "s_nop 1" gives the two wait states a DPP read needs
// after a VALU write of any register it reads, and inside the block every
// accumulator is read three instructions after it was written.
template <int G>
__device__ __forceinline__ void dot16_bcast(float (&acc)[4], uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3,
                                            uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %4, %8 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %4, %8 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %4, %8 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %5, %9 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %5, %9 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %5, %9 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %6, %10 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %6, %10 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %6, %10 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %7, %11 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %7, %11 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %7, %11 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
      : "v"(q0), "v"(q1), "v"(q2), "v"(q3), "v"(k0), "v"(k1), "v"(k2), "v"(k3),
        "i"(4 * G), "i"(4 * G + 1), "i"(4 * G + 2), "i"(4 * G + 3));
}

// acc[i] = q(head 4G+i) . k over D dims (bf16), for the four heads of group G.
template <int G, int D>
__device__ __forceinline__ void four_heads(float (&acc)[4], const uint32_t (&qv)[D / 2], const uint32_t (&kd)[D / 2]) {
  acc[0] = acc[1] = acc[2] = acc[3] = 0.0f;
  // five wait states for an EXEC write by a VALU instruction before the DPP reads
  asm volatile("s_nop 4");
#pragma unroll
  for (int d = 0; d < D / 2; d += 4)
    dot16_bcast<G>(acc, qv[d], qv[d + 1], qv[d + 2], qv[d + 3], kd[d], kd[d + 1], kd[d + 2], kd[d + 3]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int H, int D, bool REINDEX>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs a) {
  constexpr int NCH = D / 8;                  // 16-byte chunks per row
  constexpr int MAXSTEPS = 8;
  __shared__ __attribute__((aligned(16))) uint4 tile[64 * NCH];
  __shared__ float res[MAXSTEPS * 64];        // scores of this workgroup, stored at the end

  const int qi = blockIdx.y;
  const int lane = threadIdx.x;
  int64_t base;
  const int64_t n_vis = visible_rows(a, qi, base);
  const int64_t first = (int64_t)blockIdx.x * a.steps * 64;
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

  // Per-lane byte offset, within a 64-row tile, of the chunk this lane copies
  // in copy instruction i (token tok_i, chunk chunk_i): fixed for all steps.
  uint32_t off[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int slot = i * 64 + lane, tok = slot / NCH, chunk = (slot % NCH) ^ (tok % NCH);
    off[i] = (uint32_t)(tok * D * 2 + chunk * 16);
  }
  const char* seq_k = reinterpret_cast<const char*>(a.idx_k + base * D);

  auto issue_copy = [&](int64_t s0) {
    const bool full_tile = !REINDEX && s0 + 64 <= n_vis;
    if (full_tile) {
      const char* tb = seq_k + s0 * (D * 2);
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(tb + off[i]), (__attribute__((address_space(3))) void*)&tile[i * 64], 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int slot = i * 64 + lane, tok = slot / NCH, chunk = (slot % NCH) ^ (tok % NCH);
        int64_t t = position(s0 + tok);
        if (t < 0) t = 0;                       // any in-bounds row; its score is not used
        __builtin_amdgcn_global_load_lds((const void*)(seq_k + t * (D * 2) + chunk * 16),
                                         (__attribute__((address_space(3))) void*)&tile[i * 64], 16, 0, 0);
      }
    }
  };

  // lane j of each 16-lane row holds head j's indexer query (D/2 bf16 pairs);
  // lanes j >= H hold head 0's, which no broadcast reads
  uint32_t qv[D / 2];
  {
    const int h = (lane & 15) < H ? (lane & 15) : 0;
    const uint4* qp = reinterpret_cast<const uint4*>(a.idx_q + ((int64_t)qi * H + h) * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const uint4 v = qp[i];
      qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
    }
  }
  const_f32_ptr wq = (const_f32_ptr)(a.w + (int64_t)qi * H);

  issue_copy(first);
  for (int step = 0; step < nsteps; ++step) {
    wait_vmem();
    uint4 row[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) row[c] = tile[lane * NCH + (c ^ (lane % NCH))];
    wait_lds();
    if (step + 1 < nsteps) issue_copy(first + (int64_t)(step + 1) * 64);

    uint32_t kd[D / 2];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      kd[4 * c] = row[c].x; kd[4 * c + 1] = row[c].y; kd[4 * c + 2] = row[c].z; kd[4 * c + 3] = row[c].w;
    }
    float score = 0.0f;
    {
      float acc[4];
      four_heads<0, D>(acc, qv, kd);
#pragma unroll
      for (int i = 0; i < 4; ++i) score = fmaf(wq[i], fmaxf(acc[i], 0.0f), score);
    }
    if constexpr (H >= 8) {
      float acc[4];
      four_heads<1, D>(acc, qv, kd);
#pragma unroll
      for (int i = 0; i < 4; ++i) score = fmaf(wq[4 + i], fmaxf(acc[i], 0.0f), score);
    }
    if constexpr (H >= 16) {
#pragma unroll
      for (int gg = 2; gg < 4; ++gg) {
        float acc[4];
        if (gg == 2) four_heads<2, D>(acc, qv, kd); else four_heads<3, D>(acc, qv, kd);
#pragma unroll
        for (int i = 0; i < 4; ++i) score = fmaf(wq[4 * gg + i], fmaxf(acc[i], 0.0f), score);
      }
    }

    res[step * 64 + lane] = score;
  }

  // Store the workgroup's results: scores (and block maxima) of nsteps*64 slots.
  wait_lds();
  for (int step = 0; step < nsteps; ++step) {
    const int64_t j = first + (int64_t)step * 64 + lane;
    const float score = res[step * 64 + lane];
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
  const int steps = 8;   // at most MAXSTEPS of scan_kernel
  a.steps = steps;
#define FP4KV_SCAN_CASE(HH, DD) \
  if (H == HH && D == DD) return launch_scan_hd<HH, DD>(a, n_q, slots, reindex, stream);
  FP4KV_SCAN_CASE(4, 64) FP4KV_SCAN_CASE(8, 64) FP4KV_SCAN_CASE(16, 64)
  FP4KV_SCAN_CASE(4, 128) FP4KV_SCAN_CASE(8, 128) FP4KV_SCAN_CASE(16, 128)
#undef FP4KV_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace fp4kv
