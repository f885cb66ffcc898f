// Host-only driver for the C ABI's argument checks, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_cpu_sanitize.py). Every call below
// must be refused before anything is launched, or have nothing to launch, so
// no GPU is needed; a sanitizer report or a wrong status fails the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fp4kv.h"

static int failures = 0;

static void expect(const char* what, fp4kv_status got, fp4kv_status want) {
  const char* msg = fp4kv_last_error();
  const bool msg_ok = (want == FP4KV_OK) ? msg[0] == '\0' : msg[0] != '\0';
  if (got != want || !msg_ok) {
    std::printf("FAIL %s: status %d (want %d), message \"%s\"\n", what, got, want, msg);
    ++failures;
  }
}

int main() {
  // A pointer that is never dereferenced: each call fails validation first.
  alignas(256) static unsigned char arena[4096];
  void* p = arena;
  auto* i32 = reinterpret_cast<int32_t*>(arena);
  auto* i64 = reinterpret_cast<int64_t*>(arena);
  auto* f32 = reinterpret_cast<float*>(arena);
  auto* u8 = reinterpret_cast<uint8_t*>(arena);
  void* misaligned = arena + 2;

  // ---- appends
  expect("append NULL src", fp4kv_quantize_append(nullptr, 4, 512, nullptr, 0, u8, u8, 4, nullptr), FP4KV_ERR_NULL);
  expect("append C not /32", fp4kv_quantize_append(p, 4, 500, nullptr, 0, u8, u8, 4, nullptr), FP4KV_ERR_SHAPE);
  expect("append negative rows", fp4kv_quantize_append(p, -1, 512, nullptr, 0, u8, u8, 4, nullptr), FP4KV_ERR_SHAPE);
  expect("append past the cache", fp4kv_quantize_append(p, 4, 512, nullptr, 1, u8, u8, 4, nullptr), FP4KV_ERR_SHAPE);
  expect("append start near INT64_MAX",
         fp4kv_quantize_append(p, 4, 512, nullptr, INT64_MAX - 1, u8, u8, 4, nullptr), FP4KV_ERR_SHAPE);
  expect("append misaligned src", fp4kv_quantize_append(misaligned, 4, 512, nullptr, 0, u8, u8, 4, nullptr),
         FP4KV_ERR_SHAPE);
  expect("append nothing", fp4kv_quantize_append(nullptr, 0, 512, nullptr, 0, nullptr, nullptr, 0, nullptr), FP4KV_OK);
  expect("kv_append unknown format", fp4kv_kv_append(7, p, 4, 512, nullptr, 0, u8, u8, 4, nullptr),
         FP4KV_ERR_UNSUPPORTED);
  expect("kv_append MXFP4 needs scales", fp4kv_kv_append(1, p, 4, 512, nullptr, 0, u8, nullptr, 4, nullptr),
         FP4KV_ERR_NULL);
  expect("kv_append FP8 without scales, nothing", fp4kv_kv_append(2, p, 0, 512, nullptr, 0, u8, nullptr, 4, nullptr),
         FP4KV_OK);
  if (fp4kv_kv_code_bytes(0, 512) != 256 || fp4kv_kv_scale_bytes(1, 512) != 16 || fp4kv_kv_code_bytes(3, 512) != -1 ||
      fp4kv_kv_scale_bytes(0, 48) != -1 || fp4kv_kv_code_bytes(2, INT32_MIN) != -1) {
    std::printf("FAIL kv row sizes\n");
    ++failures;
  }

  // ---- workspace sizes: zero for invalid or empty requests, no overflow
  if (fp4kv_index_workspace_bytes(0, 100, 8) != 0 || fp4kv_index_workspace_bytes(4, -5, 8) != 0 ||
      fp4kv_index_workspace_bytes(4, 100, 0) != 0 || fp4kv_reindex_workspace_bytes(-1, 2048, 8) != 0 ||
      fp4kv_attn_workspace_bytes(0, 64, 512, 512, 128) != 0 || fp4kv_attn_workspace_bytes(4, 64, 256, 512, 128) != 0) {
    std::printf("FAIL workspace sizes of empty or invalid requests\n");
    ++failures;
  }
  // beyond 2^40 positions, or scores that do not fit size_t: refused with 0
  if (fp4kv_index_workspace_bytes(INT32_MAX, INT64_MAX, 8) != 0 ||
      fp4kv_index_workspace_bytes(1, (int64_t(1) << 40) + 1, 8) != 0 ||
      fp4kv_index_workspace_bytes(INT32_MAX, int64_t(1) << 40, 8) != 0 ||
      fp4kv_index_workspace_bytes(1, int64_t(1) << 40, 8) != (size_t(1) << 42) + (size_t(1) << 39)) {
    std::printf("FAIL workspace sizes at the max_ctx limit\n");
    ++failures;
  }
  (void)fp4kv_reindex_workspace_bytes(INT32_MAX, INT32_MAX, INT32_MAX);
  (void)fp4kv_attn_workspace_bytes(INT32_MAX, 64, 512, 16384, 16384);

  // ---- indexer
  int32_t* o = i32;
  expect("index_full NULL", fp4kv_index_full(nullptr, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 2, o, o, o, o, p,
                                             1 << 20, nullptr), FP4KV_ERR_NULL);
  expect("index_full block 16", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 16, 4, 2, o, o, o, o, p,
                                                 1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("index_full H 3", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 3, 128, 100, 8, 4, 2, o, o, o, o, p,
                                            1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("index_full k > P*8", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 33, o, o, o, o, p,
                                                1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full P*8 > 16384", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4096, 2, o, o, o,
                                                    o, p, 1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("index_full P huge", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, INT32_MAX, 2, o, o, o,
                                               o, p, 1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("index_full small workspace", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 2, o, o, o,
                                                        o, p, 10, nullptr), FP4KV_ERR_WORKSPACE);
  expect("index_full max_ctx 0", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 0, 8, 4, 2, o, o, o, o, p,
                                                  1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full max_ctx INT64_MAX", fp4kv_index_full(p, f32, p, 100, i64, i32, 1, 1, 16, 128, INT64_MAX, 8, 4, 2,
                                                          o, o, o, o, p, 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full misaligned keys", fp4kv_index_full(p, f32, misaligned, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 2,
                                                        o, o, o, o, p, 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full scores beyond size_t", fp4kv_index_full(p, f32, p, 100, i64, i32, INT32_MAX, 1, 16, 128,
                                                             int64_t(1) << 40, 8, 4, 2, o, o, o, o, p, SIZE_MAX,
                                                             nullptr), FP4KV_ERR_SHAPE);
  expect("index_full_noalloc scores beyond size_t",
         fp4kv_index_full_noalloc(p, f32, p, 100, i64, i32, INT32_MAX, 1, 16, 128, int64_t(1) << 40, 8, 4, 2, o, o, o,
                                  o, nullptr), FP4KV_ERR_WORKSPACE);
  expect("index_select max_ctx beyond 2^40", fp4kv_index_select(f32, f32, 100, i64, i32, 1, 1, INT64_MAX, 8, 4, 2, o,
                                                                o, o, o, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full_append rows past INT64_MAX",
         fp4kv_index_full_append(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 2, o, o, o, o, 0, p, 8, 512,
                                 nullptr, INT64_MAX - 2, u8, u8, INT64_MAX, p, 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_full no queries", fp4kv_index_full(p, f32, p, 100, i64, i32, 0, 1, 16, 128, 100, 8, 4, 2, o, o, o, o,
                                                   nullptr, 0, nullptr), FP4KV_OK);
  expect("index_scores NULL outputs", fp4kv_index_scores(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, nullptr,
                                                         nullptr, nullptr), FP4KV_ERR_NULL);
  expect("index_select q_per_seq 0", fp4kv_index_select(f32, f32, 100, i64, i32, 1, 0, 100, 8, 4, 2, o, o, o, o,
                                                        nullptr), FP4KV_ERR_SHAPE);
  expect("index_reindex small workspace", fp4kv_index_reindex(p, f32, p, 100, i64, i32, 1, 1, 16, 128, o, o, 8, 4, 2,
                                                              o, o, p, 4, nullptr), FP4KV_ERR_WORKSPACE);
  expect("index_full_append bad append", fp4kv_index_full_append(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, 4, 2,
                                                                 o, o, o, o, 0, p, 4, 500, nullptr, 0, u8, u8, 4, p,
                                                                 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("index_scores_append bad format",
         fp4kv_index_scores_append(p, f32, p, 100, i64, i32, 1, 1, 16, 128, 100, 8, f32, f32, 9, p, 4, 512, nullptr, 0,
                                   u8, u8, 4, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("index_full_noalloc beyond its array",
         fp4kv_index_full_noalloc(p, f32, p, 1 << 26, i64, i32, 64, 1, 16, 128, 1 << 20, 8, 2048, 512, o, o, o, o,
                                  nullptr), FP4KV_ERR_WORKSPACE);
  expect("index_full_noalloc no queries",
         fp4kv_index_full_noalloc(p, f32, p, 100, i64, i32, 0, 1, 16, 128, 100, 8, 4, 2, o, o, o, o, nullptr), FP4KV_OK);

  // ---- attention
  const float sc = 0.044f;
  expect("decode C 256", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64, 256, 8, 128, sc, f32,
                                                  nullptr, p, 1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("decode Hq 48", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 48, 512, 8, 128, sc, f32,
                                                  nullptr, p, 1 << 20, nullptr), FP4KV_ERR_UNSUPPORTED);
  expect("decode k 0", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64, 512, 0, 128, sc, f32,
                                                nullptr, p, 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("decode W too large", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64, 512, 8, 1 << 20,
                                                        sc, f32, nullptr, p, 1 << 20, nullptr), FP4KV_ERR_SHAPE);
  expect("decode infinite scale", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64, 512, 8, 128,
                                                           1.0f / 0.0f, f32, nullptr, p, 1 << 20, nullptr),
         FP4KV_ERR_SHAPE);
  expect("decode misaligned scales", fp4kv_sparse_attn_decode(p, u8, u8 + 1, 100, i64, i32, i32, p, p, i32, 1, 64, 512,
                                                              8, 128, sc, f32, nullptr, p, 1 << 20, nullptr),
         FP4KV_ERR_SHAPE);
  expect("decode small workspace", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64, 512, 8,
                                                            128, sc, f32, nullptr, p, 8, nullptr), FP4KV_ERR_WORKSPACE);
  expect("decode no queries", fp4kv_sparse_attn_decode(p, u8, u8, 100, i64, i32, i32, p, p, i32, 0, 64, 512, 8, 128, sc,
                                                       f32, nullptr, nullptr, 0, nullptr), FP4KV_OK);
  expect("prefill negative pos0", fp4kv_sparse_attn_prefill(p, u8, u8, 100, 0, i32, i32, p, p, -1, 4, 64, 512, 8, 128,
                                                             sc, f32, nullptr, p, SIZE_MAX, nullptr), FP4KV_ERR_SHAPE);
  expect("decode_kv unknown format", fp4kv_sparse_attn_decode_kv(5, p, u8, u8, 100, i64, i32, i32, p, p, i32, 1, 64,
                                                                 512, 8, 128, sc, f32, nullptr, p, 1 << 20, nullptr),
         FP4KV_ERR_UNSUPPORTED);

  // ---- paged cache and window ring
  expect("paged page_rows 96", fp4kv_paged_kv_append(0, p, nullptr, 4, 512, 0, i32, i64, i32, 2, 8, 96, 16, u8, u8,
                                                     nullptr, nullptr), FP4KV_ERR_SHAPE);
  expect("paged page_rows 2^30", fp4kv_paged_kv_append(0, p, nullptr, 4, 512, 0, i32, i64, i32, 2, 8, 1 << 30, 16, u8,
                                                       u8, nullptr, nullptr), FP4KV_ERR_SHAPE);
  expect("paged n_pages huge", fp4kv_paged_kv_append(0, p, nullptr, 4, 512, 0, i32, i64, i32, 2, 8, 64, INT64_MAX, u8,
                                                     u8, nullptr, nullptr), FP4KV_ERR_SHAPE);
  expect("paged no table", fp4kv_paged_kv_append(0, p, nullptr, 4, 512, 0, i32, i64, nullptr, 2, 8, 64, 16, u8, u8,
                                                 nullptr, nullptr), FP4KV_ERR_NULL);
  expect("ring W 0", fp4kv_swa_ring_append(p, p, 4, 512, i32, i64, 2, 0, p, p, nullptr), FP4KV_ERR_SHAPE);
  expect("ring nothing", fp4kv_swa_ring_append(p, p, 0, 512, i32, i64, 2, 128, p, p, nullptr), FP4KV_OK);
  expect("index_full_paged max_ctx beyond the table",
         fp4kv_index_full_paged(p, f32, p, i32, 2, 8, 64, 16, i32, 2, 1, 16, 128, 513, 8, 64, 32, o, o, o, o, p, 1 << 30,
                                nullptr), FP4KV_ERR_SHAPE);
  expect("decode_paged NULL q_pos",
         fp4kv_sparse_attn_decode_paged(0, p, u8, u8, i32, 8, 64, 16, i32, i32, p, p, nullptr, 1, 64, 512, 8, 128, sc,
                                        f32, nullptr, p, 1 << 20, nullptr), FP4KV_ERR_NULL);

  if (failures) {
    std::printf("%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("all ABI checks passed\n");
  return 0;
}
