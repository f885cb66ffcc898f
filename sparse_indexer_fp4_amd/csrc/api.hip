// C ABI of libfp4kv: argument checks, workspace sizing, grid sizing from host
// scalars, and kernel launches on the caller's stream. The declarations and
// their contracts are in include/fp4kv.h.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "fp4kv.h"
#include "kernels.h"


namespace {

thread_local std::string g_error;

fp4kv_status fail(fp4kv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

fp4kv_status ok() {
  g_error.clear();
  return FP4KV_OK;
}

fp4kv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FP4KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t nblk_of(int64_t max_ctx, int block) { return (max_ctx + block - 1) / block; }

// Largest max_ctx the indexer entry points accept (keeps every size and index
// product in range).
constexpr int64_t kMaxCtx = int64_t(1) << 40;

// Index workspace bytes (scores, then block maxima), or 0 when the size does
// not fit size_t.
size_t index_ws_bytes(int32_t n_q, int64_t max_ctx, int32_t block) {
  size_t scores = 0, bmax = 0, total = 0;
  if (__builtin_mul_overflow((size_t)n_q, (size_t)max_ctx, &scores) ||
      __builtin_mul_overflow(scores, sizeof(float), &scores) || scores > SIZE_MAX - kAlign)
    return 0;
  bmax = (size_t)n_q * (size_t)nblk_of(max_ctx, block) * sizeof(float);   // no larger than scores
  if (__builtin_add_overflow(align_up(scores), align_up(bmax), &total)) return 0;
  return total;
}

fp4kv_status check_max_ctx(const char* fn, int64_t max_ctx) {
  if (max_ctx < 1 || max_ctx > kMaxCtx)
    return fail(FP4KV_ERR_SHAPE, "%s: max_ctx=%lld must be in [1, 2^40]", fn, (long long)max_ctx);
  return FP4KV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Workspace of fp4kv_index_full_noalloc: a device array of fixed size in this
// code object. Each GPU the library runs on holds its own copy until the
// process ends. Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not a device address): the device address comes
// from hipGetSymbolAddress, taken once per device below.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};   // device address of `scratch` on each device

// Address of the calling device's copy of `scratch`, looked up on the first
// call made with that device current. The stream must belong to that device.
fp4kv_status scratch_address(const char* fn, hipStream_t s, void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(FP4KV_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  if (s) {
    int sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (sdev != dev)
      return fail(FP4KV_ERR_SHAPE, "%s: the stream belongs to device %d, device %d is current", fn, sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, fn);
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return FP4KV_OK;
}

}  // namespace

extern "C" {

int32_t fp4kv_abi_version(void) { return FP4KV_ABI_VERSION; }

const char* fp4kv_last_error(void) { return g_error.c_str(); }

static bool valid_fmt(int32_t fmt) { return fmt >= FP4KV_KV_FP4 && fmt <= FP4KV_KV_FP8; }

int64_t fp4kv_kv_code_bytes(int32_t fmt, int32_t C) {
  if (!valid_fmt(fmt) || C <= 0 || C % 32 != 0) return -1;
  return fmt == FP4KV_KV_FP8 ? C : C / 2;
}

int64_t fp4kv_kv_scale_bytes(int32_t fmt, int32_t C) {
  if (!valid_fmt(fmt) || C <= 0 || C % 32 != 0) return -1;
  return fmt == FP4KV_KV_FP4 ? C / 16 : (fmt == FP4KV_KV_MXFP4 ? C / 32 : 0);
}

static fp4kv_status check_append(const char* fn, int32_t fmt, const void* src, int64_t n_rows, int32_t C,
                                 const int64_t* dst_rows, int64_t dst_start, const uint8_t* codes,
                                 const uint8_t* scales, int64_t cap_rows) {
  if (!valid_fmt(fmt)) return fail(FP4KV_ERR_UNSUPPORTED, "%s: format %d (0, 1 or 2 implemented)", fn, fmt);
  if (n_rows == 0) return FP4KV_OK;        // nothing is read or written: the buffers may be NULL
  if (!src || !codes || (fmt != FP4KV_KV_FP8 && !scales))
    return fail(FP4KV_ERR_NULL, "%s: src, codes and (except for FP8) scales must be non-NULL", fn);
  if (C <= 0 || C % 32 != 0) return fail(FP4KV_ERR_SHAPE, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (n_rows < 0 || cap_rows < 0) return fail(FP4KV_ERR_SHAPE, "%s: n_rows and cap_rows must be >= 0", fn);
  if (!dst_rows && (dst_start < 0 || dst_start > cap_rows || n_rows > cap_rows - dst_start))
    return fail(FP4KV_ERR_SHAPE, "%s: %lld rows from row %lld do not fit the cache of %lld rows", fn,
                (long long)n_rows, (long long)dst_start, (long long)cap_rows);
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(codes) & 7u))
    return fail(FP4KV_ERR_SHAPE, "%s: src must be 16-byte and codes 8-byte aligned", fn);
  return FP4KV_OK;
}

fp4kv_status fp4kv_kv_append(int32_t fmt, const void* src, int64_t n_rows, int32_t C, const int64_t* dst_rows,
                             int64_t dst_start, uint8_t* codes, uint8_t* scales, int64_t cap_rows, void* stream) {
  fp4kv_status st = check_append("kv_append", fmt, src, n_rows, C, dst_rows, dst_start, codes, scales, cap_rows);
  if (st != FP4KV_OK) return st;
  if (n_rows == 0) return ok();
  fp4kv::AppendDst dd{};
  dd.dst_rows = dst_rows;
  dd.dst_start = dst_start;
  return hip_status(fp4kv::launch_quantize_append(fmt, src, n_rows, C, dd, codes, scales, cap_rows,
                                                  static_cast<hipStream_t>(stream)),
                    "kv_append");
}

fp4kv_status fp4kv_quantize_append(const void* src, int64_t n_rows, int32_t C, const int64_t* dst_rows,
                                   int64_t dst_start, uint8_t* codes, uint8_t* scales, int64_t cap_rows,
                                   void* stream) {
  return fp4kv_kv_append(FP4KV_KV_FP4, src, n_rows, C, dst_rows, dst_start, codes, scales, cap_rows, stream);
}

size_t fp4kv_index_workspace_bytes(int32_t n_q, int64_t max_ctx, int32_t block) {
  if (n_q <= 0 || max_ctx <= 0 || max_ctx > kMaxCtx || block <= 0) return 0;
  return index_ws_bytes(n_q, max_ctx, block);
}

size_t fp4kv_reindex_workspace_bytes(int32_t n_q, int32_t P, int32_t block) {
  if (n_q <= 0 || P <= 0 || block <= 0) return 0;
  return align_up((size_t)n_q * (size_t)P * (size_t)block * sizeof(float));   // < 2^95 / 2^31: fits
}

size_t fp4kv_attn_workspace_bytes(int32_t n_q, int32_t Hq, int32_t C, int32_t k, int32_t W) {
  if (n_q <= 0 || Hq <= 0 || C != 512 || k <= 0 || W <= 0) return 0;
  return fp4kv::attn_workspace_bytes(n_q, Hq, k, W);
}

static fp4kv_status check_indexer_common(const char* fn, const void* idx_q, const float* w, const void* idx_k,
                                         int64_t total_rows, const int64_t* seq_start, const int32_t* q_pos,
                                         int32_t n_q, int32_t q_per_seq, int32_t H, int32_t D, int32_t block,
                                         int32_t P, int32_t k, const int32_t* idx_out, const int32_t* n_idx) {
  if (!idx_q || !w || !idx_k || !seq_start || !q_pos || !idx_out || !n_idx)
    return fail(FP4KV_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (n_q < 0 || q_per_seq < 1 || total_rows < 0) return fail(FP4KV_ERR_SHAPE, "%s: n_q >= 0, q_per_seq >= 1 and total_rows >= 0 required", fn);
  if (H <= 0 || D <= 0 || D % 8 != 0) return fail(FP4KV_ERR_SHAPE, "%s: H=%d, D=%d (D must be a positive multiple of 8)", fn, H, D);
  if (!fp4kv::scan_supported(H, D)) return fail(FP4KV_ERR_UNSUPPORTED, "%s: H=%d, D=%d not implemented (H in {4,8,16}, D in {64,128})", fn, H, D);
  if (block != 8) return fail(FP4KV_ERR_UNSUPPORTED, "%s: block=%d (only 8 is implemented)", fn, block);
  if (P < 1 || k < 1) return fail(FP4KV_ERR_SHAPE, "%s: P=%d and k=%d must be >= 1", fn, P, k);
  if ((int64_t)P * block > 16384) return fail(FP4KV_ERR_UNSUPPORTED, "%s: P*block=%lld exceeds 16384", fn, (long long)P * block);
  if (k > P * block) return fail(FP4KV_ERR_SHAPE, "%s: k=%d exceeds P*block=%d", fn, k, P * block);
  if (!aligned16(idx_k) || !aligned16(idx_q)) return fail(FP4KV_ERR_SHAPE, "%s: idx_q and idx_k must be 16-byte aligned", fn);
  return FP4KV_OK;
}

static fp4kv_status launch_scores(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                  const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                  int32_t H, int32_t D, int64_t max_ctx, int32_t block, float* scores,
                                  float* blockmax, hipStream_t s, const fp4kv::PageMap* map = nullptr,
                                  const fp4kv::AppendJob* app = nullptr) {
  fp4kv::ScanArgs sa{};
  if (map) sa.map = *map;
  sa.idx_q = static_cast<const uint16_t*>(idx_q);
  sa.w = w;
  sa.idx_k = static_cast<const uint16_t*>(idx_k);
  sa.total_rows = total_rows;
  sa.seq_start = seq_start;
  sa.q_pos = q_pos;
  sa.q_per_seq = q_per_seq;
  sa.max_ctx = max_ctx;
  sa.scores = scores;
  sa.blockmax = blockmax;
  sa.nblk_max = nblk_of(max_ctx, block);
  // Many queries per sequence share every key: the scan is a dense product on the matrix cores
  // (contiguous storage only; a paged cache is scanned query by query).
  if (!map && fp4kv::scan_mfma_supported(H, D, q_per_seq, max_ctx)) {
    if (app && app->n_rows > 0) {          // the matrix-core scan does not carry an append: it goes first
      hipError_t e = fp4kv::launch_quantize_append(app->fmt, app->src, app->n_rows, app->C, app->dd, app->codes,
                                                   app->scales, app->cap_rows, s);
      if (e != hipSuccess) return hip_status(e, "quantize-append");
    }
    return hip_status(fp4kv::launch_scan_mfma(sa, H, D, n_q, s), "index scan (matrix cores)");
  }
  return hip_status(fp4kv::launch_scan(sa, H, D, n_q, max_ctx, false, s, app), "index scan");
}

static fp4kv_status launch_select_full(const float* scores, const float* blockmax, int64_t total_rows,
                                       const int64_t* seq_start, const int32_t* q_pos, int32_t n_q,
                                       int32_t q_per_seq, int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                                       int32_t* pool_out, int32_t* n_pool, int32_t* idx_out, int32_t* n_idx,
                                       hipStream_t s) {
  fp4kv::SelectArgs se{};
  se.seq_start = seq_start;
  se.q_pos = q_pos;
  se.q_per_seq = q_per_seq;
  se.total_rows = total_rows;
  se.max_ctx = max_ctx;
  se.scores = scores;
  se.blockmax = blockmax;
  se.nblk_max = nblk_of(max_ctx, block);
  se.P = P;
  se.k = k;
  se.pool = pool_out;
  se.n_pool = n_pool;
  se.idx_out = idx_out;
  se.n_idx = n_idx;
  return hip_status(fp4kv::launch_select(se, n_q, false, s), "index select");
}

// Full indexer with its workspace (scores, then block maxima) at `workspace`,
// already known to hold fp4kv_index_workspace_bytes(n_q, max_ctx, block) bytes.
static fp4kv_status index_full_into(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                    const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                    int32_t H, int32_t D, int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                                    int32_t* pool_out, int32_t* n_pool, int32_t* idx_out, int32_t* n_idx,
                                    void* workspace, hipStream_t s, const fp4kv::AppendJob* app = nullptr) {
  float* scores = static_cast<float*>(workspace);
  float* blockmax = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up((size_t)n_q * max_ctx * sizeof(float)));
  fp4kv_status st = launch_scores(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block,
                                  scores, blockmax, s, nullptr, app);
  if (st != FP4KV_OK) return st;
  return launch_select_full(scores, blockmax, total_rows, seq_start, q_pos, n_q, q_per_seq, max_ctx, block, P, k,
                            pool_out, n_pool, idx_out, n_idx, s);
}

fp4kv_status fp4kv_index_full(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                              const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                              int32_t H, int32_t D, int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                              int32_t* pool_out, int32_t* n_pool, int32_t* idx_out, int32_t* n_idx,
                              void* workspace, size_t ws_bytes, void* stream) {
  fp4kv_status st = check_indexer_common("index_full", idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq,
                                         H, D, block, P, k, idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool_out || !n_pool) return fail(FP4KV_ERR_NULL, "index_full: pool_out and n_pool must be non-NULL");
  st = check_max_ctx("index_full", max_ctx);
  if (st != FP4KV_OK) return st;
  if (n_q == 0) return ok();
  const size_t need = fp4kv_index_workspace_bytes(n_q, max_ctx, block);
  if (need == 0) return fail(FP4KV_ERR_SHAPE, "index_full: n_q x max_ctx scores do not fit size_t");
  if (!workspace || ws_bytes < need)
    return fail(FP4KV_ERR_WORKSPACE, "index_full: workspace of %zu bytes, %zu required", ws_bytes, need);
  return index_full_into(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block, P, k,
                         pool_out, n_pool, idx_out, n_idx, workspace, static_cast<hipStream_t>(stream));
}

fp4kv_status fp4kv_index_scores(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                int32_t H, int32_t D, int64_t max_ctx, int32_t block, float* scores,
                                float* blockmax, void* stream) {
  int32_t dummy = 0;
  fp4kv_status st = check_indexer_common("index_scores", idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q,
                                         q_per_seq, H, D, block, 1, 1, &dummy, &dummy);
  if (st != FP4KV_OK) return st;
  if (!scores || !blockmax) return fail(FP4KV_ERR_NULL, "index_scores: scores and blockmax must be non-NULL");
  st = check_max_ctx("index_scores", max_ctx);
  if (st != FP4KV_OK) return st;
  if (n_q == 0) return ok();
  return launch_scores(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block, scores,
                       blockmax, static_cast<hipStream_t>(stream));
}

fp4kv_status fp4kv_index_select(const float* scores, const float* blockmax, int64_t total_rows,
                                const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                int64_t max_ctx, int32_t block, int32_t P, int32_t k, int32_t* pool_out,
                                int32_t* n_pool, int32_t* idx_out, int32_t* n_idx, void* stream) {
  if (!scores || !blockmax || !seq_start || !q_pos || !pool_out || !n_pool || !idx_out || !n_idx)
    return fail(FP4KV_ERR_NULL, "index_select: a required pointer is NULL");
  if (n_q < 0 || q_per_seq < 1 || total_rows < 0)
    return fail(FP4KV_ERR_SHAPE, "index_select: n_q >= 0, q_per_seq >= 1 and total_rows >= 0 required");
  fp4kv_status st = check_max_ctx("index_select", max_ctx);
  if (st != FP4KV_OK) return st;
  if (block != 8) return fail(FP4KV_ERR_UNSUPPORTED, "index_select: block=%d (only 8 is implemented)", block);
  if (P < 1 || k < 1) return fail(FP4KV_ERR_SHAPE, "index_select: P=%d and k=%d must be >= 1", P, k);
  if ((int64_t)P * block > 16384) return fail(FP4KV_ERR_UNSUPPORTED, "index_select: P*block exceeds 16384");
  if (k > P * block) return fail(FP4KV_ERR_SHAPE, "index_select: k=%d exceeds P*block=%d", k, P * block);
  if (n_q == 0) return ok();
  return launch_select_full(scores, blockmax, total_rows, seq_start, q_pos, n_q, q_per_seq, max_ctx, block, P, k,
                            pool_out, n_pool, idx_out, n_idx, static_cast<hipStream_t>(stream));
}

fp4kv_status fp4kv_index_scores_append(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                       const int64_t* seq_start, const int32_t* q_pos, int32_t n_q,
                                       int32_t q_per_seq, int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                                       float* scores, float* blockmax, int32_t kv_fmt, const void* kv_src,
                                       int64_t n_rows, int32_t C, const int64_t* dst_rows, int64_t dst_start,
                                       uint8_t* codes, uint8_t* scales, int64_t cap_rows, void* stream) {
  const char* fn = "index_scores_append";
  int32_t dummy = 0;
  fp4kv_status st = check_indexer_common(fn, idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D,
                                         block, 1, 1, &dummy, &dummy);
  if (st != FP4KV_OK) return st;
  if (!scores || !blockmax) return fail(FP4KV_ERR_NULL, "%s: scores and blockmax must be non-NULL", fn);
  st = check_max_ctx(fn, max_ctx);
  if (st != FP4KV_OK) return st;
  st = check_append(fn, kv_fmt, kv_src, n_rows, C, dst_rows, dst_start, codes, scales, cap_rows);
  if (st != FP4KV_OK) return st;
  fp4kv::AppendDst dd{};
  dd.dst_rows = dst_rows;
  dd.dst_start = dst_start;
  const fp4kv::AppendJob job = fp4kv::make_append_job(kv_fmt, kv_src, n_rows, C, dd, codes, scales, cap_rows);
  if (n_q == 0) {
    if (n_rows == 0) return ok();
    return hip_status(fp4kv::launch_quantize_append(kv_fmt, kv_src, n_rows, C, dd, codes, scales, cap_rows,
                                                    static_cast<hipStream_t>(stream)), fn);
  }
  return launch_scores(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block, scores,
                       blockmax, static_cast<hipStream_t>(stream), nullptr, &job);
}

fp4kv_status fp4kv_index_full_append(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                     const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                     int32_t H, int32_t D, int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                                     int32_t* pool_out, int32_t* n_pool, int32_t* idx_out, int32_t* n_idx,
                                     int32_t kv_fmt, const void* kv_src, int64_t n_rows, int32_t C,
                                     const int64_t* dst_rows, int64_t dst_start, uint8_t* codes, uint8_t* scales,
                                     int64_t cap_rows, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "index_full_append";
  fp4kv_status st = check_indexer_common(fn, idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D,
                                         block, P, k, idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool_out || !n_pool) return fail(FP4KV_ERR_NULL, "%s: pool_out and n_pool must be non-NULL", fn);
  st = check_max_ctx(fn, max_ctx);
  if (st != FP4KV_OK) return st;
  st = check_append(fn, kv_fmt, kv_src, n_rows, C, dst_rows, dst_start, codes, scales, cap_rows);
  if (st != FP4KV_OK) return st;
  const size_t need = n_q > 0 ? fp4kv_index_workspace_bytes(n_q, max_ctx, block) : 0;
  if (n_q > 0 && need == 0) return fail(FP4KV_ERR_SHAPE, "%s: n_q x max_ctx scores do not fit size_t", fn);
  if (n_q > 0 && (!workspace || ws_bytes < need))
    return fail(FP4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu required", fn, ws_bytes, need);
  fp4kv::AppendDst dd{};
  dd.dst_rows = dst_rows;
  dd.dst_start = dst_start;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_q == 0) {
    if (n_rows == 0) return ok();
    return hip_status(fp4kv::launch_quantize_append(kv_fmt, kv_src, n_rows, C, dd, codes, scales, cap_rows, s), fn);
  }
  const fp4kv::AppendJob job = fp4kv::make_append_job(kv_fmt, kv_src, n_rows, C, dd, codes, scales, cap_rows);
  return index_full_into(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block, P, k,
                         pool_out, n_pool, idx_out, n_idx, workspace, s, &job);
}

fp4kv_status fp4kv_index_reindex(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                 const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                 int32_t H, int32_t D, const int32_t* pool, const int32_t* n_pool, int32_t block,
                                 int32_t P, int32_t k, int32_t* idx_out, int32_t* n_idx, void* workspace,
                                 size_t ws_bytes, void* stream) {
  fp4kv_status st = check_indexer_common("index_reindex", idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q,
                                         q_per_seq, H, D, block, P, k, idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool || !n_pool) return fail(FP4KV_ERR_NULL, "index_reindex: pool and n_pool must be non-NULL");
  if (n_q == 0) return ok();
  const size_t need = fp4kv_reindex_workspace_bytes(n_q, P, block);
  if (!workspace || ws_bytes < need)
    return fail(FP4KV_ERR_WORKSPACE, "index_reindex: workspace of %zu bytes, %zu required", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* pscores = static_cast<float*>(workspace);
  // Positions are bounded by the sequence (rows past total_rows are invisible),
  // so the clamp of q_pos uses the largest representable context.
  const int64_t max_ctx = total_rows > 0 ? total_rows : 1;

  fp4kv::ScanArgs sa{};
  sa.idx_q = static_cast<const uint16_t*>(idx_q);
  sa.w = w;
  sa.idx_k = static_cast<const uint16_t*>(idx_k);
  sa.total_rows = total_rows;
  sa.seq_start = seq_start;
  sa.q_pos = q_pos;
  sa.q_per_seq = q_per_seq;
  sa.max_ctx = max_ctx;
  sa.pool = pool;
  sa.n_pool = n_pool;
  sa.P = P;
  sa.pool_scores = pscores;
  hipError_t e = fp4kv::launch_scan(sa, H, D, n_q, (int64_t)P * block, true, s);
  if (e != hipSuccess) return hip_status(e, "index_reindex scan");

  fp4kv::SelectArgs se{};
  se.seq_start = seq_start;
  se.q_pos = q_pos;
  se.q_per_seq = q_per_seq;
  se.total_rows = total_rows;
  se.max_ctx = max_ctx;
  se.scores = pscores;
  se.P = P;
  se.k = k;
  se.pool = const_cast<int32_t*>(pool);
  se.n_pool = const_cast<int32_t*>(n_pool);
  se.idx_out = idx_out;
  se.n_idx = n_idx;
  return hip_status(fp4kv::launch_select(se, n_q, true, s), "index_reindex select");
}

static fp4kv_status check_attn(const char* fn, int32_t fmt, const void* q, const uint8_t* codes,
                               const uint8_t* scales, const int32_t* idx, const int32_t* n_idx, const void* swa_k,
                               const void* swa_v, int32_t nq, int32_t Hq, int32_t C, int32_t k, int32_t W, float scale,
                               const float* out, void* workspace, size_t ws_bytes) {
  if (!valid_fmt(fmt)) return fail(FP4KV_ERR_UNSUPPORTED, "%s: format %d (0, 1 or 2 implemented)", fn, fmt);
  if (fmt == FP4KV_KV_FP8) scales = nullptr;       // not read
  if (!q || !codes || (fmt != FP4KV_KV_FP8 && !scales) || !idx || !n_idx || !swa_k || !swa_v || !out)
    return fail(FP4KV_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (nq < 0 || Hq <= 0 || C <= 0 || k < 1 || W < 1 || k > 16384 || W > 16384)
    return fail(FP4KV_ERR_SHAPE, "%s: n_q=%d Hq=%d C=%d k=%d W=%d out of range", fn, nq, Hq, C, k, W);
  if (!(Hq == 16 || Hq == 32 || Hq == 64)) return fail(FP4KV_ERR_UNSUPPORTED, "%s: Hq=%d (16, 32 or 64 implemented)", fn, Hq);
  if (C != 512) return fail(FP4KV_ERR_UNSUPPORTED, "%s: C=%d (only 512 implemented)", fn, C);
  if (!std::isfinite(scale)) return fail(FP4KV_ERR_SHAPE, "%s: scale must be finite", fn);
  if (!aligned16(q) || !aligned16(swa_k) || !aligned16(swa_v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(codes) & 7u) || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(FP4KV_ERR_SHAPE, "%s: q, swa_k, swa_v, out must be 16-byte, codes 8-byte and scales 4-byte aligned",
                fn);
  const size_t need = fp4kv_attn_workspace_bytes(nq, Hq, C, k, W);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(FP4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu required", fn, ws_bytes, need);
  return FP4KV_OK;
}

fp4kv_status fp4kv_sparse_attn_decode_kv(int32_t fmt, const void* q, const uint8_t* codes, const uint8_t* scales,
                                         int64_t total_rows, const int64_t* seq_start, const int32_t* idx,
                                         const int32_t* n_idx, const void* swa_k, const void* swa_v,
                                         const int32_t* q_pos, int32_t B, int32_t Hq, int32_t C, int32_t k, int32_t W,
                                         float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                                         void* stream) {
  fp4kv_status st = check_attn("sparse_attn_decode", fmt, q, codes, scales, idx, n_idx, swa_k, swa_v, B, Hq, C, k, W,
                               scale, out, workspace, ws_bytes);
  if (st != FP4KV_OK) return st;
  if (!seq_start || !q_pos) return fail(FP4KV_ERR_NULL, "sparse_attn_decode: seq_start and q_pos must be non-NULL");
  if (B == 0) return ok();
  fp4kv::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.codes = codes;
  a.scales = scales;
  a.kv_fmt = fmt;
  a.total_rows = total_rows;
  a.seq_start = seq_start;
  a.idx = idx;
  a.n_idx = n_idx;
  a.k = k;
  a.swa_k = static_cast<const uint16_t*>(swa_k);
  a.swa_v = static_cast<const uint16_t*>(swa_v);
  a.q_pos = q_pos;
  a.win_stride = W;
  a.W = W;
  a.nq = B;
  a.Hq = Hq;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  return hip_status(fp4kv::launch_attn(a, workspace, static_cast<hipStream_t>(stream)), "sparse_attn_decode");
}

fp4kv_status fp4kv_sparse_attn_prefill_kv(int32_t fmt, const void* q, const uint8_t* codes, const uint8_t* scales,
                                          int64_t total_rows, int64_t seq_start, const int32_t* idx,
                                          const int32_t* n_idx, const void* swa_k, const void* swa_v, int32_t pos0,
                                          int32_t T, int32_t Hq, int32_t C, int32_t k, int32_t W, float scale,
                                          float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  fp4kv_status st = check_attn("sparse_attn_prefill", fmt, q, codes, scales, idx, n_idx, swa_k, swa_v, T, Hq, C, k, W,
                               scale, out, workspace, ws_bytes);
  if (st != FP4KV_OK) return st;
  if (pos0 < 0 || seq_start < 0) return fail(FP4KV_ERR_SHAPE, "sparse_attn_prefill: pos0 and seq_start must be >= 0");
  if (T == 0) return ok();
  fp4kv::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.codes = codes;
  a.scales = scales;
  a.kv_fmt = fmt;
  a.total_rows = total_rows;
  a.seq_start = nullptr;
  a.seq_start_scalar = seq_start;
  a.idx = idx;
  a.n_idx = n_idx;
  a.k = k;
  a.swa_k = static_cast<const uint16_t*>(swa_k);
  a.swa_v = static_cast<const uint16_t*>(swa_v);
  a.q_pos = nullptr;
  a.pos0 = pos0;
  a.win_stride = 1;
  a.W = W;
  a.nq = T;
  a.Hq = Hq;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  return hip_status(fp4kv::launch_attn(a, workspace, static_cast<hipStream_t>(stream)), "sparse_attn_prefill");
}

fp4kv_status fp4kv_sparse_attn_decode(const void* q, const uint8_t* codes, const uint8_t* scales, int64_t total_rows,
                                      const int64_t* seq_start, const int32_t* idx, const int32_t* n_idx,
                                      const void* swa_k, const void* swa_v, const int32_t* q_pos, int32_t B,
                                      int32_t Hq, int32_t C, int32_t k, int32_t W, float scale, float* out, float* lse,
                                      void* workspace, size_t ws_bytes, void* stream) {
  return fp4kv_sparse_attn_decode_kv(FP4KV_KV_FP4, q, codes, scales, total_rows, seq_start, idx, n_idx, swa_k, swa_v,
                                     q_pos, B, Hq, C, k, W, scale, out, lse, workspace, ws_bytes, stream);
}

fp4kv_status fp4kv_sparse_attn_prefill(const void* q, const uint8_t* codes, const uint8_t* scales, int64_t total_rows,
                                       int64_t seq_start, const int32_t* idx, const int32_t* n_idx, const void* swa_k,
                                       const void* swa_v, int32_t pos0, int32_t T, int32_t Hq, int32_t C, int32_t k,
                                       int32_t W, float scale, float* out, float* lse, void* workspace,
                                       size_t ws_bytes, void* stream) {
  return fp4kv_sparse_attn_prefill_kv(FP4KV_KV_FP4, q, codes, scales, total_rows, seq_start, idx, n_idx, swa_k,
                                      swa_v, pos0, T, Hq, C, k, W, scale, out, lse, workspace, ws_bytes, stream);
}

// ---- paged cache and window ring ------------------------------------------

static fp4kv_status check_pages(const char* fn, const int32_t* block_table, int32_t n_seq, int32_t max_pages,
                                int32_t page_rows, int64_t n_pages, fp4kv::PageMap& m) {
  if (!block_table) return fail(FP4KV_ERR_NULL, "%s: block_table must be non-NULL", fn);
  if (n_seq < 0 || max_pages < 1 || n_pages < 1)
    return fail(FP4KV_ERR_SHAPE, "%s: n_seq >= 0, max_pages >= 1 and n_pages >= 1 required", fn);
  if (page_rows < 64 || page_rows > (1 << 20) || (page_rows & (page_rows - 1)) != 0)
    return fail(FP4KV_ERR_SHAPE, "%s: page_rows=%d must be a power of two in [64, 2^20]", fn, page_rows);
  if (n_pages > (INT64_MAX >> 21)) return fail(FP4KV_ERR_SHAPE, "%s: n_pages too large", fn);
  m.block_table = block_table;
  m.n_seq = n_seq;
  m.max_pages = max_pages;
  m.log2_page = __builtin_ctz((unsigned)page_rows);
  m.n_pages = n_pages;
  return FP4KV_OK;
}

fp4kv_status fp4kv_paged_kv_append(int32_t fmt, const void* kv_src, const void* idxk_src, int64_t n_rows, int32_t C,
                                   int32_t D, const int32_t* row_seq, const int64_t* row_pos,
                                   const int32_t* block_table, int32_t n_seq, int32_t max_pages, int32_t page_rows,
                                   int64_t n_pages, uint8_t* codes, uint8_t* scales, void* idx_k, void* stream) {
  const char* fn = "paged_kv_append";
  if (!valid_fmt(fmt)) return fail(FP4KV_ERR_UNSUPPORTED, "%s: format %d (0, 1 or 2 implemented)", fn, fmt);
  fp4kv::AppendDst dd{};
  fp4kv_status st = check_pages(fn, block_table, n_seq, max_pages, page_rows, n_pages, dd.map);
  if (st != FP4KV_OK) return st;
  if (!row_seq || !row_pos || (!kv_src && !idxk_src))
    return fail(FP4KV_ERR_NULL, "%s: row_seq, row_pos and one of kv_src / idxk_src must be non-NULL", fn);
  if (kv_src && (!codes || (fmt != FP4KV_KV_FP8 && !scales)))
    return fail(FP4KV_ERR_NULL, "%s: codes and (except for FP8) scales must be non-NULL with kv_src", fn);
  if (idxk_src && !idx_k) return fail(FP4KV_ERR_NULL, "%s: idx_k must be non-NULL with idxk_src", fn);
  if (n_rows < 0) return fail(FP4KV_ERR_SHAPE, "%s: n_rows must be >= 0", fn);
  if (kv_src && (C <= 0 || C % 32 != 0)) return fail(FP4KV_ERR_SHAPE, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (idxk_src && (D <= 0 || D % 8 != 0)) return fail(FP4KV_ERR_SHAPE, "%s: D=%d must be a positive multiple of 8", fn, D);
  if ((kv_src && !aligned16(kv_src)) || (idxk_src && (!aligned16(idxk_src) || !aligned16(idx_k))) ||
      (codes && (reinterpret_cast<uintptr_t>(codes) & 7u)))
    return fail(FP4KV_ERR_SHAPE, "%s: kv_src, idxk_src, idx_k must be 16-byte and codes 8-byte aligned", fn);
  if (n_rows == 0) return ok();
  dd.row_seq = row_seq;
  dd.row_pos = row_pos;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t cap = n_pages << dd.map.log2_page;
  if (kv_src) {
    st = hip_status(fp4kv::launch_quantize_append(fmt, kv_src, n_rows, C, dd, codes, scales, cap, s), fn);
    if (st != FP4KV_OK) return st;
  }
  if (idxk_src) return hip_status(fp4kv::launch_copy_rows(idxk_src, n_rows, D, dd, idx_k, cap, s), fn);
  return ok();
}

fp4kv_status fp4kv_swa_ring_append(const void* k_src, const void* v_src, int64_t n_rows, int32_t C,
                                   const int32_t* row_seq, const int64_t* row_pos, int32_t n_seq, int32_t W,
                                   void* ring_k, void* ring_v, void* stream) {
  const char* fn = "swa_ring_append";
  if (!k_src || !v_src || !row_seq || !row_pos || !ring_k || !ring_v)
    return fail(FP4KV_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (n_rows < 0 || n_seq < 0 || W < 1 || C <= 0 || C % 8 != 0)
    return fail(FP4KV_ERR_SHAPE, "%s: n_rows=%lld n_seq=%d W=%d C=%d out of range", fn, (long long)n_rows, n_seq, W, C);
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(ring_k) || !aligned16(ring_v))
    return fail(FP4KV_ERR_SHAPE, "%s: all row buffers must be 16-byte aligned", fn);
  if (n_rows == 0) return ok();
  return hip_status(fp4kv::launch_ring_append(k_src, v_src, n_rows, C, row_seq, row_pos, n_seq, W, ring_k, ring_v,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

fp4kv_status fp4kv_index_full_paged(const void* idx_q, const float* w, const void* idx_k, const int32_t* block_table,
                                    int32_t n_seq, int32_t max_pages, int32_t page_rows, int64_t n_pages,
                                    const int32_t* q_pos, int32_t n_q, int32_t q_per_seq, int32_t H, int32_t D,
                                    int64_t max_ctx, int32_t block, int32_t P, int32_t k, int32_t* pool_out,
                                    int32_t* n_pool, int32_t* idx_out, int32_t* n_idx, void* workspace,
                                    size_t ws_bytes, void* stream) {
  const char* fn = "index_full_paged";
  fp4kv::PageMap m{};
  fp4kv_status st = check_pages(fn, block_table, n_seq, max_pages, page_rows, n_pages, m);
  if (st != FP4KV_OK) return st;
  const int64_t total_rows = n_pages * page_rows;
  const int64_t dummy_start = 0;     // not read: the block table places every row
  st = check_indexer_common(fn, idx_q, w, idx_k, total_rows, &dummy_start, q_pos, n_q, q_per_seq, H, D, block, P, k,
                            idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool_out || !n_pool) return fail(FP4KV_ERR_NULL, "%s: pool_out and n_pool must be non-NULL", fn);
  if (max_ctx < 1 || max_ctx > (int64_t)max_pages * page_rows)
    return fail(FP4KV_ERR_SHAPE, "%s: max_ctx=%lld must be in [1, max_pages*page_rows]", fn, (long long)max_ctx);
  if ((int64_t)n_q > (int64_t)n_seq * q_per_seq)
    return fail(FP4KV_ERR_SHAPE, "%s: n_q=%d exceeds n_seq*q_per_seq", fn, n_q);
  if (n_q == 0) return ok();
  const size_t need = fp4kv_index_workspace_bytes(n_q, max_ctx, block);
  if (need == 0) return fail(FP4KV_ERR_SHAPE, "%s: n_q x max_ctx scores do not fit size_t", fn);
  if (!workspace || ws_bytes < need)
    return fail(FP4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu required", fn, ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scores = static_cast<float*>(workspace);
  float* blockmax = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up((size_t)n_q * max_ctx * sizeof(float)));
  st = launch_scores(idx_q, w, idx_k, total_rows, nullptr, q_pos, n_q, q_per_seq, H, D, max_ctx, block, scores,
                     blockmax, s, &m);
  if (st != FP4KV_OK) return st;
  return launch_select_full(scores, blockmax, INT64_MAX, nullptr, q_pos, n_q, q_per_seq, max_ctx, block, P, k,
                            pool_out, n_pool, idx_out, n_idx, s);
}

fp4kv_status fp4kv_index_reindex_paged(const void* idx_q, const float* w, const void* idx_k,
                                       const int32_t* block_table, int32_t n_seq, int32_t max_pages,
                                       int32_t page_rows, int64_t n_pages, const int32_t* q_pos, int32_t n_q,
                                       int32_t q_per_seq, int32_t H, int32_t D, const int32_t* pool,
                                       const int32_t* n_pool, int32_t block, int32_t P, int32_t k, int32_t* idx_out,
                                       int32_t* n_idx, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "index_reindex_paged";
  fp4kv::PageMap m{};
  fp4kv_status st = check_pages(fn, block_table, n_seq, max_pages, page_rows, n_pages, m);
  if (st != FP4KV_OK) return st;
  const int64_t total_rows = n_pages * page_rows;
  const int64_t dummy_start = 0;
  st = check_indexer_common(fn, idx_q, w, idx_k, total_rows, &dummy_start, q_pos, n_q, q_per_seq, H, D, block, P, k,
                            idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool || !n_pool) return fail(FP4KV_ERR_NULL, "%s: pool and n_pool must be non-NULL", fn);
  if ((int64_t)n_q > (int64_t)n_seq * q_per_seq)
    return fail(FP4KV_ERR_SHAPE, "%s: n_q=%d exceeds n_seq*q_per_seq", fn, n_q);
  if (n_q == 0) return ok();
  const size_t need = fp4kv_reindex_workspace_bytes(n_q, P, block);
  if (!workspace || ws_bytes < need)
    return fail(FP4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu required", fn, ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  fp4kv::ScanArgs sa{};
  sa.idx_q = static_cast<const uint16_t*>(idx_q);
  sa.w = w;
  sa.idx_k = static_cast<const uint16_t*>(idx_k);
  sa.total_rows = total_rows;
  sa.seq_start = nullptr;
  sa.q_pos = q_pos;
  sa.q_per_seq = q_per_seq;
  sa.max_ctx = (int64_t)max_pages * page_rows;   // every position the table can map
  sa.pool = pool;
  sa.n_pool = n_pool;
  sa.P = P;
  sa.pool_scores = static_cast<float*>(workspace);
  sa.map = m;
  hipError_t e = fp4kv::launch_scan(sa, H, D, n_q, (int64_t)P * block, true, s);
  if (e != hipSuccess) return hip_status(e, "index_reindex_paged scan");
  fp4kv::SelectArgs se{};
  se.seq_start = nullptr;
  se.q_pos = q_pos;
  se.q_per_seq = q_per_seq;
  se.total_rows = INT64_MAX;
  se.max_ctx = (int64_t)max_pages * page_rows;
  se.scores = static_cast<float*>(workspace);
  se.P = P;
  se.k = k;
  se.pool = const_cast<int32_t*>(pool);
  se.n_pool = const_cast<int32_t*>(n_pool);
  se.idx_out = idx_out;
  se.n_idx = n_idx;
  return hip_status(fp4kv::launch_select(se, n_q, true, s), "index_reindex_paged select");
}

fp4kv_status fp4kv_sparse_attn_decode_paged(int32_t fmt, const void* q, const uint8_t* codes, const uint8_t* scales,
                                            const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                                            int64_t n_pages, const int32_t* idx, const int32_t* n_idx,
                                            const void* ring_k, const void* ring_v, const int32_t* q_pos, int32_t B,
                                            int32_t Hq, int32_t C, int32_t k, int32_t W, float scale, float* out,
                                            float* lse, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "sparse_attn_decode_paged";
  fp4kv::PageMap m{};
  fp4kv_status st = check_pages(fn, block_table, B, max_pages, page_rows, n_pages, m);
  if (st != FP4KV_OK) return st;
  st = check_attn(fn, fmt, q, codes, scales, idx, n_idx, ring_k, ring_v, B, Hq, C, k, W, scale, out, workspace,
                  ws_bytes);
  if (st != FP4KV_OK) return st;
  if (!q_pos) return fail(FP4KV_ERR_NULL, "%s: q_pos must be non-NULL", fn);
  if (B == 0) return ok();
  fp4kv::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.codes = codes;
  a.scales = fmt == FP4KV_KV_FP8 ? nullptr : scales;
  a.kv_fmt = fmt;
  a.total_rows = n_pages * page_rows;
  a.idx = idx;
  a.n_idx = n_idx;
  a.k = k;
  a.swa_k = static_cast<const uint16_t*>(ring_k);
  a.swa_v = static_cast<const uint16_t*>(ring_v);
  a.q_pos = q_pos;
  a.win_stride = W;
  a.W = W;
  a.nq = B;
  a.Hq = Hq;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.map = m;
  a.page_q_per_seq = 1;
  a.ring = 1;
  return hip_status(fp4kv::launch_attn(a, workspace, static_cast<hipStream_t>(stream)), fn);
}

fp4kv_status fp4kv_index_full_noalloc(const void* idx_q, const float* w, const void* idx_k, int64_t total_rows,
                                      const int64_t* seq_start, const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                      int32_t H, int32_t D, int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                                      int32_t* pool_out, int32_t* n_pool, int32_t* idx_out, int32_t* n_idx,
                                      void* stream) {
  const char* fn = "index_full_noalloc";
  fp4kv_status st = check_indexer_common(fn, idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D,
                                         block, P, k, idx_out, n_idx);
  if (st != FP4KV_OK) return st;
  if (!pool_out || !n_pool) return fail(FP4KV_ERR_NULL, "%s: pool_out and n_pool must be non-NULL", fn);
  st = check_max_ctx(fn, max_ctx);
  if (st != FP4KV_OK) return st;
  if (n_q == 0) return ok();
  const size_t need = fp4kv_index_workspace_bytes(n_q, max_ctx, block);
  if (need == 0 || need > kNoallocScratchBytes)
    return fail(FP4KV_ERR_WORKSPACE, "%s: n_q=%d x max_ctx=%lld needs %zu bytes of scores, beyond the fixed %zu",
                fn, n_q, (long long)max_ctx, need, kNoallocScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_address(fn, s, &ws);
  if (st != FP4KV_OK) return st;
  return index_full_into(idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D, max_ctx, block, P, k,
                         pool_out, n_pool, idx_out, n_idx, ws, s);
}

}  // extern "C"
