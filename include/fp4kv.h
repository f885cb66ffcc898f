/*
 * fp4kv: the hot path of CSA2-style sparse attention over an FP4 main-KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on DeepSeek V4.1-Flash's KV cache):
 *   [G] "DeepSeek V4.1 Flash KV Cache: 890 Bytes per Token Explained"
 *       (paragraphs on CSA2 modes, the hierarchical sparse indexer, FP4 main KV,
 *       SWA Bounded Replay; the page has no section headings).
 *   [T] "890 bytes per token: how DeepSeek V4.1-Flash's KV cache works",
 *       sections "Mechanism 3: FP4 KV via quantization-aware training" and
 *       "Mechanism 4: the hierarchical sparse indexer".
 *   [N] "DeepSeek-V4.1-Flash: 890 Bytes Per Token, 437x Smaller KV Cache",
 *       sections "CSA2: Sharing Main KV, Indexer K, and Top-K Indices Across
 *       Layers", "FP4 KV Quantization and Cache Lifetime Management" and
 *       "Causal Encoder-Decoder and Prefill Halving".
 *
 * How a model calls this library, one layer at a time ([N] "CSA2: ..."):
 *   Full layer     -> fp4kv_index_full, then fp4kv_sparse_attn_{decode,prefill}
 *   Reindex layer  -> fp4kv_index_reindex on the Full layer's pool, then attention
 *   Reuse layer    -> no indexer call; attention with the indices it is handed
 * Every layer attends with its own main Q and its own sliding-window KV.
 * New main-KV rows enter the cache through fp4kv_quantize_append.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) point to GPU memory; all others are host values.
 *     The caller owns every buffer. The library never allocates or frees, and
 *     keeps no pointer after a call returns.
 *   - Inputs are read-only. Work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) and the call returns without waiting for it.
 *   - Grids are sized from host scalars only; device-resident counts and
 *     positions are read by the kernels, which clamp them to the sizes given
 *     here so that no access leaves the buffers described.
 *   - Arguments are checked before anything is launched. On error nothing is
 *     launched, a negative status is returned and fp4kv_last_error() describes
 *     it (a thread-local string, valid until the next call on that thread).
 *     FP4KV_ERR_HIP reports a launch failure; outputs are then undefined.
 *   - Results are deterministic: identical inputs give identical bits.
 *   - Positions are relative to the first row of their sequence. Index lists are
 *     ascending; entries past the count are -1.
 *   - bf16 is bfloat16 stored as 16-bit words.
 */
#ifndef FP4KV_H
#define FP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp4kv_status;

enum {
    FP4KV_OK = 0,
    FP4KV_ERR_NULL = -1,        /* a required pointer is NULL */
    FP4KV_ERR_SHAPE = -2,       /* a size or layout argument is out of range */
    FP4KV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    FP4KV_ERR_UNSUPPORTED = -4, /* valid, but not a shape these kernels implement */
    FP4KV_ERR_HIP = -5          /* the HIP runtime reported an error */
};

#define FP4KV_ABI_VERSION 1

/* Version of this interface (FP4KV_ABI_VERSION of the built library). */
int32_t fp4kv_abi_version(void);

/* Description of the last failed call on this thread ("" if none). */
const char* fp4kv_last_error(void);

/*
 * FP4 quantize-append of main-KV rows.
 * [G] FP4 main KV paragraph, [N] "FP4 KV Quantization and Cache Lifetime
 * Management": E2M1 values, an E4M3 factor for every 16-channel group, no global
 * scale.
 *
 * For each source row i and each group g of 16 channels:
 *   scale code  = E4M3 (FN: bias 7, max 448, no inf) value nearest amax/6,
 *                 ties to the even code, saturating at 448; subnormal scales
 *                 are kept, amax/6 <= 2^-10 gives 0;
 *   value code  = sign bit of x, then the E2M1 magnitude nearest |x|/scale
 *                 (ties to the even code, saturating at 6; 0 if the scale is 0).
 * Codes are exact (no floating-point rounding of the ratio is involved).
 *
 *   src       (device) bf16 [n_rows, C], row-major.
 *   n_rows    rows to append (0 is allowed: nothing is launched, and the
 *             pointers are then not checked or read).
 *   C         channels per row, a positive multiple of 32.
 *   dst_rows  (device) int64 [n_rows]: destination row of each source row, or
 *             NULL to write rows dst_start .. dst_start+n_rows-1. Destination
 *             rows outside [0, cap_rows) are skipped (not written).
 *   codes     (device) uint8 [cap_rows, C/2]: channel 2j in the low nibble of
 *             byte j, channel 2j+1 in the high nibble.
 *   scales    (device) uint8 [cap_rows, C/16]: E4M3 scale codes.
 *   Together 288 bytes per row at C = 512.
 * Errors: NULL src/codes/scales; C not a positive multiple of 32; n_rows < 0;
 * with dst_rows NULL, dst_start < 0 or dst_start + n_rows > cap_rows.
 */
fp4kv_status fp4kv_quantize_append(const void* src, int64_t n_rows, int32_t C,
                                   const int64_t* dst_rows, int64_t dst_start,
                                   uint8_t* codes, uint8_t* scales, int64_t cap_rows,
                                   void* stream);

/*
 * Main-KV storage formats. The FP4 cache above is format 0. Formats 1 and 2 are
 * the formats the pages compare it with, for measuring the storage, bandwidth
 * and accuracy trade: [T] "Mechanism 3" names the KV format MXFP4, and [G] FP4
 * main KV paragraph and [N] "FP4 KV Quantization and Cache Lifetime Management"
 * say FP4 takes about half the bytes of an FP8 cache.
 *   FP4KV_KV_FP4    E2M1 codes + an E4M3 scale for each 16-channel group (as above);
 *                   C/2 + C/16 bytes per row (288 at C = 512).
 *   FP4KV_KV_MXFP4  E2M1 codes + one E8M0 scale per 32 channels (OCP
 *                   microscaling): per block, e = floor(log2 amax) - 2 clamped
 *                   to [-127, 127] (-127 if amax = 0), scale byte e + 127, each
 *                   value the E2M1 code nearest x / 2^e (ties to the even code,
 *                   saturating at 6). Codes as for FP4; scales uint8
 *                   [rows, C/32]; 272 bytes per row at C = 512.
 *   FP4KV_KV_FP8    one E4M3FN code per channel (nearest finite value, ties to
 *                   the even code, saturating at 448, sign bit of x); codes
 *                   uint8 [rows, C], no scale plane; 512 bytes per row.
 */
enum {
    FP4KV_KV_FP4 = 0,
    FP4KV_KV_MXFP4 = 1,
    FP4KV_KV_FP8 = 2
};

/* Bytes per row of the code plane and of the scale plane of format fmt (-1 for
 * an unknown format or a C that is not a positive multiple of 32). */
int64_t fp4kv_kv_code_bytes(int32_t fmt, int32_t C);
int64_t fp4kv_kv_scale_bytes(int32_t fmt, int32_t C);

/*
 * Quantize-append of main-KV rows in format fmt; arguments as for
 * fp4kv_quantize_append (which is this call with FP4KV_KV_FP4), with codes
 * [cap_rows, fp4kv_kv_code_bytes(fmt, C)] and scales
 * [cap_rows, fp4kv_kv_scale_bytes(fmt, C)]. scales may be NULL for
 * FP4KV_KV_FP8. Codes are exact, as for FP4.
 * Errors: as for fp4kv_quantize_append; an unknown fmt (FP4KV_ERR_UNSUPPORTED).
 */
fp4kv_status fp4kv_kv_append(int32_t fmt, const void* src, int64_t n_rows, int32_t C,
                             const int64_t* dst_rows, int64_t dst_start, uint8_t* codes,
                             uint8_t* scales, int64_t cap_rows, void* stream);

/*
 * Workspace bytes fp4kv_index_full needs for n_q queries whose positions are
 * below max_ctx (token scores and block maxima, fp32). 0 when n_q, max_ctx or
 * block is not positive, max_ctx exceeds 2^40, or the size does not fit size_t;
 * the indexer entry points refuse such a request (FP4KV_ERR_SHAPE).
 */
size_t fp4kv_index_workspace_bytes(int32_t n_q, int64_t max_ctx, int32_t block);

/*
 * Full-mode indexer: score every visible token, keep the best blocks as the
 * candidate pool, then the best tokens inside the pool.
 * [G] hierarchical sparse indexer paragraph (a query first narrows the context to
 * 2,048 eight-token blocks, then to 512 tokens); [T] "Mechanism 4"; [N] "CSA2: ...", Full
 * bullet.
 *
 * The pages leave the scoring rule open. This library computes, for query i at
 * position p and each token t <= p of its sequence,
 *     score(t) = sum_h w[i,h] * max(0, sum_d q[i,h,d] * k[t,d])   (fp32)
 * (one indexer key per token, shared by the heads), the score of block b as
 * the max over its visible tokens 8b..min(8b+7, p), the pool as the
 * min(P, p/8+1) best blocks, and the selection as the min(k, #visible pool
 * positions) best positions inside the pool. Ranking is by score descending,
 * ties to the lower block id / position. With integer-valued bf16 inputs whose
 * partial sums stay below 2^24 the scores are exact.
 *
 *   idx_q       (device) bf16 [n_q, H, D]
 *   w           (device) fp32 [n_q, H]
 *   idx_k       (device) bf16 [total_rows, D]: indexer keys of all sequences.
 *   seq_start   (device) int64 [ceil(n_q / q_per_seq)]: first row of each
 *               sequence; query i belongs to sequence i / q_per_seq. A start
 *               outside [0, total_rows] makes the sequence empty (no token).
 *   q_pos       (device) int32 [n_q]: position of each query (its causal
 *               limit; decode: context length - 1). Clamped to max_ctx-1; a
 *               negative position sees no token (empty pool and selection);
 *               rows at or past total_rows are treated as not visible.
 *   H, D        H in {4, 8, 16}; D in {64, 128}.
 *   max_ctx     host bound: every q_pos < max_ctx (sizes the grid); in
 *               [1, 2^40] for every indexer entry point.
 *   block       tokens per block; must be 8.
 *   P, k        pool blocks and kept tokens; 1 <= P, 1 <= k <= P*block,
 *               P*block <= 16384.
 *   pool_out    (device) int32 [n_q, P]; n_pool (device) int32 [n_q].
 *   idx_out     (device) int32 [n_q, k]; n_idx  (device) int32 [n_q].
 *   workspace   (device) at least fp4kv_index_workspace_bytes(n_q, max_ctx, block).
 * The prefill case is a single sequence with q_per_seq = n_q queries at
 * consecutive positions; it runs the same computation.
 */
fp4kv_status fp4kv_index_full(const void* idx_q, const float* w, const void* idx_k,
                              int64_t total_rows, const int64_t* seq_start,
                              const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                              int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                              int32_t P, int32_t k, int32_t* pool_out, int32_t* n_pool,
                              int32_t* idx_out, int32_t* n_idx, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * The two halves of fp4kv_index_full, for callers that keep the scores:
 *
 * fp4kv_index_scores: token scores and block maxima of every visible token
 * (the scan). Same arguments and scoring rule as fp4kv_index_full; writes
 *   scores    (device) fp32 [n_q, max_ctx]: score of position t of query i at
 *             scores[i*max_ctx + t] for t <= the clamped q_pos[i] (rows past
 *             total_rows excluded); other entries are left untouched;
 *   blockmax  (device) fp32 [n_q, ceil(max_ctx/block)]: max over the visible
 *             tokens of each block with at least one visible token.
 *
 * fp4kv_index_select: the candidate pool and the top-k positions from those
 * buffers (same ranking and outputs as fp4kv_index_full). seq_start, q_pos,
 * total_rows, q_per_seq, max_ctx and block must be the values the scores were
 * computed with.
 */
fp4kv_status fp4kv_index_scores(const void* idx_q, const float* w, const void* idx_k,
                                int64_t total_rows, const int64_t* seq_start,
                                const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                                float* scores, float* blockmax, void* stream);

fp4kv_status fp4kv_index_select(const float* scores, const float* blockmax, int64_t total_rows,
                                const int64_t* seq_start, const int32_t* q_pos, int32_t n_q,
                                int32_t q_per_seq, int64_t max_ctx, int32_t block, int32_t P,
                                int32_t k, int32_t* pool_out, int32_t* n_pool, int32_t* idx_out,
                                int32_t* n_idx, void* stream);

/*
 * A layer's indexer and its main-KV append in one go: fp4kv_index_full (or
 * fp4kv_index_scores) together with fp4kv_kv_append of the layer's new rows.
 * [N] "FP4 KV Quantization and Cache Lifetime Management" (new tokens enter
 * the FP4 cache); [G] hierarchical sparse indexer paragraph.
 *
 * The indexer scan reads only indexer keys, never the main KV, so the append's
 * work items ride in the scan's own launch as extra workgroups (one launch
 * fewer per layer; where the scan cannot carry them, e.g. the matrix-core
 * scan of many queries per sequence, the append is launched first). Results
 * are exactly those of the two separate calls. The new rows are in the cache
 * when the call's work completes, so a following attention call on the same
 * stream can select them.
 *   idx_q .. n_idx (or .. blockmax), workspace, ws_bytes: as for
 *               fp4kv_index_full (fp4kv_index_scores).
 *   kv_fmt, kv_src, n_rows, C, dst_rows, dst_start, codes, scales, cap_rows:
 *               as fmt, src, n_rows, C, ... of fp4kv_kv_append (n_rows may
 *               be 0).
 * Errors: those of either call; nothing is launched on error.
 */
fp4kv_status fp4kv_index_full_append(const void* idx_q, const float* w, const void* idx_k,
                                     int64_t total_rows, const int64_t* seq_start,
                                     const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                     int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                                     int32_t P, int32_t k, int32_t* pool_out, int32_t* n_pool,
                                     int32_t* idx_out, int32_t* n_idx, int32_t kv_fmt,
                                     const void* kv_src, int64_t n_rows, int32_t C,
                                     const int64_t* dst_rows, int64_t dst_start, uint8_t* codes,
                                     uint8_t* scales, int64_t cap_rows, void* workspace,
                                     size_t ws_bytes, void* stream);
fp4kv_status fp4kv_index_scores_append(const void* idx_q, const float* w, const void* idx_k,
                                       int64_t total_rows, const int64_t* seq_start,
                                       const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                       int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                                       float* scores, float* blockmax, int32_t kv_fmt,
                                       const void* kv_src, int64_t n_rows, int32_t C,
                                       const int64_t* dst_rows, int64_t dst_start, uint8_t* codes,
                                       uint8_t* scales, int64_t cap_rows, void* stream);

/* Workspace bytes fp4kv_index_reindex needs (pool token scores, fp32). */
size_t fp4kv_reindex_workspace_bytes(int32_t n_q, int32_t P, int32_t block);

/*
 * Reindex-mode indexer: rescore an inherited pool with this layer's own
 * indexer Q and weights, then keep the best tokens.
 * [N] "CSA2: ...", Reindex bullet: reuses the preceding Full layer's main KV
 * and indexer keys, scoring that layer's pool again with a fresh indexer query;
 * [G] hierarchical sparse indexer paragraph: deeper layers search the pool.
 *
 * Same scoring and ranking rule as fp4kv_index_full, over the visible
 * positions (<= q_pos) of pool blocks pool[i, 0 .. n_pool[i]-1] only (n_pool
 * clamped to [0, P]; block ids outside the sequence are ignored). Selects
 * min(k, #visible pool positions) positions, ascending.
 *   idx_q, w, idx_k, total_rows, seq_start, q_pos, n_q, q_per_seq, H, D:
 *               as for fp4kv_index_full (this layer's own idx_q and w).
 *   pool        (device) int32 [n_q, P] ascending block ids; n_pool (device) [n_q].
 *   idx_out     (device) int32 [n_q, k]; n_idx (device) int32 [n_q].
 *   workspace   (device) at least fp4kv_reindex_workspace_bytes(n_q, P, block).
 */
fp4kv_status fp4kv_index_reindex(const void* idx_q, const float* w, const void* idx_k,
                                 int64_t total_rows, const int64_t* seq_start,
                                 const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                 int32_t H, int32_t D, const int32_t* pool,
                                 const int32_t* n_pool, int32_t block, int32_t P, int32_t k,
                                 int32_t* idx_out, int32_t* n_idx, void* workspace,
                                 size_t ws_bytes, void* stream);

/*
 * Workspace bytes the attention entry points need for n_q queries (partial
 * softmax states when a query's rows are split over several workgroups; may
 * be 0).
 */
size_t fp4kv_attn_workspace_bytes(int32_t n_q, int32_t Hq, int32_t C, int32_t k, int32_t W);

/*
 * Sparse attention over selected FP4 main-KV rows plus a sliding-window branch,
 * merged by log-sum-exp; one query per sequence (decode).
 * [T] "Mechanism 4" (attention runs over the selected candidates); [N] "CSA2:
 * ..." (each layer brings a main query and window keys/values of its own) and "Causal
 * Encoder-Decoder and Prefill Halving" (a 128-token sliding window).
 *
 * For query b at position p = q_pos[b] and every head h:
 *   sparse branch: rows j = idx[b, 0 .. n_idx[b]-1] (n_idx clamped to [0, k];
 *     positions outside [0, p] or past total_rows are skipped), dequantised
 *     from (codes, scales); logits scale * q[b,h,:] . row; keys = values = the
 *     dequantised row. Softmax over the rows gives (o_s, lse_s).
 *   window branch: the last n_w = min(W, p+1) rows of swa_k[b] / swa_v[b]
 *     (row W-1 is position p), softmax -> (o_w, lse_w).
 *   out = (e^lse_s o_s + e^lse_w o_w) / (e^lse_s + e^lse_w); lse = log of the
 *     denominator (natural log). An empty sparse branch contributes nothing;
 *     a query with p < 0 has no rows at all and gets out = 0, lse = -inf.
 *
 *   q          (device) bf16 [B, Hq, C]
 *   codes      (device) uint8 [total_rows, C/2]; scales (device) uint8 [total_rows, C/16]
 *   seq_start  (device) int64 [B]: first main-KV row of each query's sequence
 *              (a start outside [0, total_rows] leaves the sparse branch empty).
 *   Alignment: q, swa_k, swa_v and out 16 bytes, codes 8 bytes, scales 4 bytes
 *     (FP4KV_ERR_SHAPE otherwise).
 *   idx        (device) int32 [B, k]; n_idx (device) int32 [B]
 *   swa_k, swa_v (device) bf16 [B, W, C]
 *   q_pos      (device) int32 [B]
 *   Hq in {16, 32, 64}; C = 512; 1 <= k <= 16384; 1 <= W <= 16384.
 *   scale      softmax scale (finite).
 *   out        (device) fp32 [B, Hq, C]; lse (device) fp32 [B, Hq], or NULL.
 *   workspace  (device) at least fp4kv_attn_workspace_bytes(B, Hq, C, k, W).
 * Numerics: logits and outputs accumulate in fp32; dequantised rows are exact
 * in bf16 and P enters the P.V product as a bf16 hi + lo pair.
 */
fp4kv_status fp4kv_sparse_attn_decode(const void* q, const uint8_t* codes,
                                      const uint8_t* scales, int64_t total_rows,
                                      const int64_t* seq_start, const int32_t* idx,
                                      const int32_t* n_idx, const void* swa_k,
                                      const void* swa_v, const int32_t* q_pos, int32_t B,
                                      int32_t Hq, int32_t C, int32_t k, int32_t W,
                                      float scale, float* out, float* lse, void* workspace,
                                      size_t ws_bytes, void* stream);

/*
 * The same attention for a prefill chunk: T queries of one sequence at
 * positions pos0 .. pos0+T-1 (first main-KV row seq_start, a host value).
 * The window buffer is shared: swa_k / swa_v (device) bf16 [T+W-1, C], row r
 * holding position pos0-W+1+r; query i uses rows i+W-n_w .. i+W-1 with
 * n_w = min(W, pos0+i+1). Rows for negative positions are never read.
 * Other arguments as for fp4kv_sparse_attn_decode, with B replaced by T
 * (workspace: fp4kv_attn_workspace_bytes(T, Hq, C, k, W)); pos0 >= 0.
 */
fp4kv_status fp4kv_sparse_attn_prefill(const void* q, const uint8_t* codes,
                                       const uint8_t* scales, int64_t total_rows,
                                       int64_t seq_start, const int32_t* idx,
                                       const int32_t* n_idx, const void* swa_k,
                                       const void* swa_v, int32_t pos0, int32_t T,
                                       int32_t Hq, int32_t C, int32_t k, int32_t W,
                                       float scale, float* out, float* lse, void* workspace,
                                       size_t ws_bytes, void* stream);

/*
 * The two attention calls for a cache in format fmt (see FP4KV_KV_*); every
 * other argument as for fp4kv_sparse_attn_decode / fp4kv_sparse_attn_prefill,
 * which are these calls with FP4KV_KV_FP4. codes and scales are laid out as
 * fp4kv_kv_append writes them; scales is not read (and may be NULL) for
 * FP4KV_KV_FP8. Rows are dequantised exactly to bf16 for every format. The
 * append writes MXFP4 scale bytes up to 252 only; bytes 253 and 254 decode
 * to values beyond bf16, and 255 (NaN) and the FP8 NaN codes 0x7F and 0xFF
 * are not supported.
 * Errors: as for the FP4 calls; an unknown fmt (FP4KV_ERR_UNSUPPORTED).
 */
fp4kv_status fp4kv_sparse_attn_decode_kv(int32_t fmt, const void* q, const uint8_t* codes,
                                         const uint8_t* scales, int64_t total_rows,
                                         const int64_t* seq_start, const int32_t* idx,
                                         const int32_t* n_idx, const void* swa_k,
                                         const void* swa_v, const int32_t* q_pos, int32_t B,
                                         int32_t Hq, int32_t C, int32_t k, int32_t W,
                                         float scale, float* out, float* lse, void* workspace,
                                         size_t ws_bytes, void* stream);
fp4kv_status fp4kv_sparse_attn_prefill_kv(int32_t fmt, const void* q, const uint8_t* codes,
                                          const uint8_t* scales, int64_t total_rows,
                                          int64_t seq_start, const int32_t* idx,
                                          const int32_t* n_idx, const void* swa_k,
                                          const void* swa_v, int32_t pos0, int32_t T,
                                          int32_t Hq, int32_t C, int32_t k, int32_t W,
                                          float scale, float* out, float* lse, void* workspace,
                                          size_t ws_bytes, void* stream);

/*
 * Paged cache and window ring: the serving-side storage around the path.
 * [N] "FP4 KV Quantization and Cache Lifetime Management" (a long-lived global
 * KV cache, with the window state kept apart from it); [G] SWA Bounded Replay
 * paragraph and [N] "Causal Encoder-Decoder and Prefill Halving" (each layer's
 * window is the last 128 tokens). The pages give no layout; this one:
 *
 *   Pages. A sequence's positions are cut into pages of page_rows consecutive
 *   positions (a power of two in [64, 2^20]); page i holds positions
 *   i*page_rows .. (i+1)*page_rows - 1. block_table (device) int32
 *   [n_seq, max_pages]: block_table[s*max_pages + i] is the physical page of
 *   sequence s's page i, and physical page g is rows g*page_rows ..
 *   (g+1)*page_rows - 1 of every per-token store: main-KV codes and scales (in
 *   a format of FP4KV_KV_*) and indexer keys, each with n_pages*page_rows rows.
 *   An entry outside [0, n_pages) maps nowhere.
 *   Window ring. Per layer, ring_k and ring_v (device) bf16 [n_seq, W, C]:
 *   position t of sequence s is row s*W + (t mod W). After positions
 *   0..p have been appended in order it holds the last min(W, p+1) of them.
 *
 * The method's results are unchanged by paging: a paged call returns exactly
 * what the contiguous call returns for the same logical sequences (same bits).
 * The block table must map every position a call reads (0..q_pos); a page that
 * maps nowhere is read as row 0 by the indexer and is skipped by attention,
 * so no access leaves the stores.
 */

/*
 * Append new tokens' rows to a paged cache (variable counts per sequence): row
 * i goes to position row_pos[i] of sequence row_seq[i], i.e. to its physical
 * row through the block table; rows that map nowhere are not written.
 *   kv_src    (device) bf16 [n_rows, C] main-KV rows, quantised into (codes,
 *             scales) in format fmt as fp4kv_kv_append does; or NULL.
 *   idxk_src  (device) bf16 [n_rows, D] indexer keys, copied into idx_k
 *             [n_pages*page_rows, D]; or NULL. At least one of the two.
 *   row_seq   (device) int32 [n_rows]; row_pos (device) int64 [n_rows].
 * Errors: NULL pointers as required; C (multiple of 32) or D (multiple of 8)
 * out of range; the page arguments (see above); alignment as for
 * fp4kv_kv_append (idxk_src and idx_k 16-byte).
 */
fp4kv_status fp4kv_paged_kv_append(int32_t fmt, const void* kv_src, const void* idxk_src,
                                   int64_t n_rows, int32_t C, int32_t D, const int32_t* row_seq,
                                   const int64_t* row_pos, const int32_t* block_table,
                                   int32_t n_seq, int32_t max_pages, int32_t page_rows,
                                   int64_t n_pages, uint8_t* codes, uint8_t* scales, void* idx_k,
                                   void* stream);

/*
 * Append window rows to a layer's ring: row i (k_src, v_src (device) bf16
 * [n_rows, C]) to slot row_pos[i] mod W of sequence row_seq[i]. Rows with a
 * sequence outside [0, n_seq) or a negative position are not written. Within
 * one call a sequence's positions must be distinct modulo W (for example at
 * most W consecutive positions: a prefill chunk appends only its last W rows);
 * where two rows of a call share a slot, which one the slot keeps is not
 * specified. C a positive multiple of 8; every buffer 16-byte aligned.
 */
fp4kv_status fp4kv_swa_ring_append(const void* k_src, const void* v_src, int64_t n_rows, int32_t C,
                                   const int32_t* row_seq, const int64_t* row_pos, int32_t n_seq,
                                   int32_t W, void* ring_k, void* ring_v, void* stream);

/*
 * fp4kv_index_full over a paged indexer-key store idx_k [n_pages*page_rows, D]:
 * query i belongs to sequence i / q_per_seq (n_q <= n_seq * q_per_seq); every
 * other argument and every output as for fp4kv_index_full, with
 * max_ctx <= max_pages*page_rows. Queries are scanned one by one (the
 * matrix-core scan for many queries per sequence needs contiguous keys).
 */
fp4kv_status fp4kv_index_full_paged(const void* idx_q, const float* w, const void* idx_k,
                                    const int32_t* block_table, int32_t n_seq, int32_t max_pages,
                                    int32_t page_rows, int64_t n_pages, const int32_t* q_pos,
                                    int32_t n_q, int32_t q_per_seq, int32_t H, int32_t D,
                                    int64_t max_ctx, int32_t block, int32_t P, int32_t k,
                                    int32_t* pool_out, int32_t* n_pool, int32_t* idx_out,
                                    int32_t* n_idx, void* workspace, size_t ws_bytes, void* stream);

/* fp4kv_index_reindex over a paged indexer-key store (arguments as above). */
fp4kv_status fp4kv_index_reindex_paged(const void* idx_q, const float* w, const void* idx_k,
                                       const int32_t* block_table, int32_t n_seq, int32_t max_pages,
                                       int32_t page_rows, int64_t n_pages, const int32_t* q_pos,
                                       int32_t n_q, int32_t q_per_seq, int32_t H, int32_t D,
                                       const int32_t* pool, const int32_t* n_pool, int32_t block,
                                       int32_t P, int32_t k, int32_t* idx_out, int32_t* n_idx,
                                       void* workspace, size_t ws_bytes, void* stream);

/*
 * fp4kv_sparse_attn_decode_kv over a paged main-KV store (codes, scales with
 * n_pages*page_rows rows, one sequence per query: B = n_seq, block_table
 * [B, max_pages]) and the layer's window ring (ring_k, ring_v [B, W, C]): the
 * window of query b at position p is positions max(0, p-W+1)..p, read from
 * slots t mod W. Every other argument as for fp4kv_sparse_attn_decode_kv.
 */
fp4kv_status fp4kv_sparse_attn_decode_paged(int32_t fmt, const void* q, const uint8_t* codes,
                                            const uint8_t* scales, const int32_t* block_table,
                                            int32_t max_pages, int32_t page_rows, int64_t n_pages,
                                            const int32_t* idx, const int32_t* n_idx,
                                            const void* ring_k, const void* ring_v,
                                            const int32_t* q_pos, int32_t B, int32_t Hq, int32_t C,
                                            int32_t k, int32_t W, float scale, float* out, float* lse,
                                            void* workspace, size_t ws_bytes, void* stream);

/*
 * fp4kv_index_full for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, and hosts that forbid
 * hipMalloc. Same arguments, outputs and errors as fp4kv_index_full, without
 * the workspace: the token scores and block maxima go to a fixed 64 MiB
 * device array inside the library (one per GPU, held until the process
 * ends). The call itself allocates nothing.
 *   Limit: fp4kv_index_workspace_bytes(n_q, max_ctx, block) <= 64 MiB, e.g.
 *   32 queries at max_ctx 131,072 (18.9 MB) or 8 at 2^20 (37.7 MB); larger
 *   calls fail with FP4KV_ERR_WORKSPACE before anything is launched.
 *   The stream must belong to the current device (FP4KV_ERR_SHAPE otherwise).
 *   The array is shared by every call on the same GPU and keeps the last
 *   call's contents; nothing in it needs to start at zero. Calls that overlap
 *   on one GPU (other streams, other threads) race on it and must be ordered
 *   by the caller.
 */
fp4kv_status fp4kv_index_full_noalloc(const void* idx_q, const float* w, const void* idx_k,
                                      int64_t total_rows, const int64_t* seq_start,
                                      const int32_t* q_pos, int32_t n_q, int32_t q_per_seq,
                                      int32_t H, int32_t D, int64_t max_ctx, int32_t block,
                                      int32_t P, int32_t k, int32_t* pool_out, int32_t* n_pool,
                                      int32_t* idx_out, int32_t* n_idx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4KV_H */
