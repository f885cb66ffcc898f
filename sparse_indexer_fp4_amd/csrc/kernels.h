// Internal interface between the C ABI (api.hip) and the kernels: argument
// blocks and launchers. Not part of the public header.
#pragma once
#include "common.h"

namespace fp4kv {

// Main-KV storage formats (values of the ABI's format argument).
enum KvFmt : int32_t {
  kKvFp4 = 0,     // E2M1 codes + an E4M3 scale for each 16-channel group
  kKvMxfp4 = 1,   // E2M1 codes + one E8M0 scale per 32 channels
  kKvFp8 = 2,     // one E4M3FN code per channel, no scale
};

// Paged storage: a sequence's positions in pages of 2^log2_page rows;
// block_table[s * max_pages + i] is the physical page of sequence s's page i,
// rows page << log2_page .. of every per-token store. block_table == nullptr:
// contiguous storage (rows seq_start[s] + position).
struct PageMap {
  const int32_t* block_table;
  int32_t n_seq, max_pages, log2_page;
  int64_t n_pages;
};

// Physical row of position pos of sequence seq, or -1 where nothing is mapped
// (sequence, page or page id out of range).
__device__ __forceinline__ int64_t paged_row(const PageMap& m, int64_t seq, int64_t pos) {
  if (seq < 0 || seq >= m.n_seq || pos < 0) return -1;
  const int64_t page = pos >> m.log2_page;
  if (page >= m.max_pages) return -1;
  const int64_t g = m.block_table[seq * m.max_pages + page];
  if (g < 0 || g >= m.n_pages) return -1;
  return (g << m.log2_page) + (pos & ((int64_t(1) << m.log2_page) - 1));
}

// Destination rows of appended rows: dst_rows[i], dst_start + i, or (paged)
// the physical row of (row_seq[i], row_pos[i]); -1 = not written.
struct AppendDst {
  const int64_t* dst_rows;
  int64_t dst_start;
  const int32_t* row_seq;
  const int64_t* row_pos;
  PageMap map;
};

__device__ __forceinline__ int64_t append_dst(const AppendDst& d, int64_t i) {
  if (d.map.block_table) return paged_row(d.map, d.row_seq[i], d.row_pos[i]);
  return d.dst_rows ? d.dst_rows[i] : d.dst_start + i;
}

// A main-KV append: rows of src (bf16 [n_rows, C]) quantised in format fmt
// into (codes, scales) at their destinations.
struct AppendJob {
  int32_t fmt;
  const uint16_t* src;
  int64_t n_rows;
  int32_t C;
  AppendDst dd;
  uint8_t* codes;
  uint8_t* scales;
  int64_t cap_rows;
};

struct ScanArgs {
  const uint16_t* idx_q;     // [n_q, H, D] bf16
  const float* w;            // [n_q, H]
  const uint16_t* idx_k;     // [total_rows, D] bf16
  int64_t total_rows;
  const int64_t* seq_start;  // [n_seq]
  const int32_t* q_pos;      // [n_q]
  int32_t q_per_seq;
  int64_t max_ctx;
  // Full scan outputs
  float* scores;             // [n_q, max_ctx]
  float* blockmax;           // [n_q, nblk_max]
  int64_t nblk_max;
  // Reindex scan inputs/outputs
  const int32_t* pool;       // [n_q, P]
  const int32_t* n_pool;     // [n_q]
  int32_t P;
  float* pool_scores;        // [n_q, P*8]
  int32_t steps;             // 64-token steps per workgroup
  PageMap map;               // paged idx_k when map.block_table (seq_start unused)
  // An append carried by the same launch (contiguous Full scan only): grid
  // rows n_q .. n_q + app_rows - 1 quantise app's rows instead of scanning.
  AppendJob app;
  int32_t app_rows;
  int32_t n_q;
  // Work-list scan (Full, up to 512 queries): the first list_wgs workgroups of
  // a 1-D grid walk the (query, range) list; app_wgs more carry the append.
  int32_t list_wgs;
  int32_t app_wgs;
};

// Launch geometry of the matrix-core scan (host-computed).
struct MfmaScanGrid {
  int32_t qblocks_per_seq;   // 32-query blocks per sequence
  int32_t n_qblocks;         // over all sequences
  int32_t n_ranges;          // token ranges
  int64_t range_tokens;      // tokens per range, a multiple of 64
  int32_t per_xcd;           // work items per XCD
  int32_t H;                 // indexer heads (<= 16; missing heads are zero)
  int32_t n_q;
};

struct SelectArgs {
  const int64_t* seq_start;  // nullptr for paged storage (positions are bounded by max_ctx only)
  const int32_t* q_pos;
  int32_t q_per_seq;
  int64_t total_rows;
  int64_t max_ctx;
  const float* scores;       // Full: [n_q, max_ctx]; Reindex: [n_q, P*8]
  const float* blockmax;     // [n_q, nblk_max] (Full)
  int64_t nblk_max;
  int32_t P, k;
  int32_t* pool;             // Full: output [n_q, P]; Reindex: input
  int32_t* n_pool;           // Full: output; Reindex: input
  int32_t* idx_out;          // [n_q, k]
  int32_t* n_idx;            // [n_q]
};

struct AttnArgs {
  const uint16_t* q;              // [nq, Hq, C] bf16
  const uint8_t* codes;           // [total_rows, C/2] (FP8: [total_rows, C])
  const uint8_t* scales;          // [total_rows, C/16] (MXFP4: C/32; FP8: unused)
  int32_t kv_fmt;                 // KvFmt
  int64_t total_rows;
  const int64_t* seq_start;       // [nq] (decode) or nullptr (prefill: seq_start_scalar)
  int64_t seq_start_scalar;
  const int32_t* idx;             // [nq, k]
  const int32_t* n_idx;           // [nq]
  int32_t k;
  const uint16_t* swa_k;          // window keys, bf16
  const uint16_t* swa_v;          // window values, bf16
  const int32_t* q_pos;           // [nq] (decode) or nullptr (prefill: pos0 + i)
  int32_t pos0;
  int64_t win_stride;             // window-buffer rows between consecutive queries
  int32_t W;
  int32_t nq, Hq;
  float scale_log2;               // softmax scale * log2(e)
  int32_t n_split;
  float* out;                     // [nq, Hq, C]
  float* lse;                     // [nq, Hq] or nullptr
  float* part_o;                  // [nq, n_split, Hq, C]
  float* part_ml;                 // [nq, n_split, Hq, 2]
  PageMap map;                    // paged main KV when map.block_table
  int32_t page_q_per_seq;         // paged: query i belongs to sequence i / page_q_per_seq
  int32_t ring;                   // window rows in a ring [nq, W, C]: position t in slot t mod W
};

AppendJob make_append_job(int32_t fmt, const void* src, int64_t n_rows, int32_t C, const AppendDst& dst,
                          uint8_t* codes, uint8_t* scales, int64_t cap_rows);
hipError_t launch_quantize_append(int32_t fmt, const void* src, int64_t n_rows, int32_t C, const AppendDst& dst,
                                  uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream);
// Copy of bf16 rows [n_rows, width] to their destinations (indexer keys of a paged cache).
hipError_t launch_copy_rows(const void* src, int64_t n_rows, int32_t width, const AppendDst& dst, void* out,
                            int64_t cap_rows, hipStream_t stream);
// Window ring append: row i to slot row_pos[i] mod W of sequence row_seq[i].
hipError_t launch_ring_append(const void* k_src, const void* v_src, int64_t n_rows, int32_t C, const int32_t* row_seq,
                              const int64_t* row_pos, int32_t n_seq, int32_t W, void* ring_k, void* ring_v,
                              hipStream_t stream);
bool scan_supported(int H, int D);
// slots: max_ctx for a Full scan, P*8 for a Reindex scan. A Full scan over
// contiguous keys also runs the append `app` (if any rows) in its launch.
hipError_t launch_scan(ScanArgs a, int H, int D, int n_q, int64_t slots, bool reindex, hipStream_t stream,
                       const AppendJob* app = nullptr);
// Matrix-core Full scan for sequences with many queries (q_per_seq >= 16).
bool scan_mfma_supported(int H, int D, int q_per_seq, int64_t max_ctx);
hipError_t launch_scan_mfma(ScanArgs a, int H, int D, int n_q, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, int n_q, bool reindex, hipStream_t stream);
size_t attn_workspace_bytes(int nq, int Hq, int k, int W);
hipError_t launch_attn(AttnArgs a, void* ws, hipStream_t stream);

}  // namespace fp4kv
