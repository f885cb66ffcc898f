// Main-KV quantize-append kernels (the work items are in quant_dev.h), the
// paged indexer-key copy and the window-ring append.
#include "quant_dev.h"

namespace fp4kv {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendJob j) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < append_items(j)) append_item(j, gid);
}

// ---- indexer-key rows of a paged cache: a plain copy, 16 bytes per thread.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ src, int64_t n_rows, int32_t units,
                                                        AppendDst dd, uint4* __restrict__ out, int64_t cap_rows) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_rows * units) return;
  const int64_t row = gid / units;
  const int32_t u = (int32_t)(gid - row * units);
  const int64_t dst = append_dst(dd, row);
  if (dst < 0 || dst >= cap_rows) return;
  out[dst * units + u] = src[gid];
}

// ---- window ring: position t of sequence s goes to slot t mod W (keys and values).
__global__ __launch_bounds__(256) void ring_append_kernel(const uint4* __restrict__ k_src,
                                                          const uint4* __restrict__ v_src, int64_t n_rows,
                                                          int32_t units, const int32_t* __restrict__ row_seq,
                                                          const int64_t* __restrict__ row_pos, int32_t n_seq,
                                                          int32_t W, uint4* __restrict__ ring_k,
                                                          uint4* __restrict__ ring_v) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_rows * units) return;
  const int64_t row = gid / units;
  const int32_t u = (int32_t)(gid - row * units);
  const int64_t s = row_seq[row], t = row_pos[row];
  if (s < 0 || s >= n_seq || t < 0) return;
  const int64_t dst = (s * W + t % W) * units + u;
  ring_k[dst] = k_src[gid];
  ring_v[dst] = v_src[gid];
}

AppendJob make_append_job(int32_t fmt, const void* src, int64_t n_rows, int32_t C, const AppendDst& dst,
                          uint8_t* codes, uint8_t* scales, int64_t cap_rows) {
  AppendJob j;
  j.fmt = fmt;
  j.src = static_cast<const uint16_t*>(src);
  j.n_rows = n_rows;
  j.C = C;
  j.dd = dst;
  j.codes = codes;
  j.scales = scales;
  j.cap_rows = cap_rows;
  return j;
}

hipError_t launch_quantize_append(int32_t fmt, const void* src, int64_t n_rows, int32_t C, const AppendDst& dst,
                                  uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream) {
  const AppendJob j = make_append_job(fmt, src, n_rows, C, dst, codes, scales, cap_rows);
  const int64_t n = n_rows * (C >> (fmt == kKvMxfp4 ? 5 : 4));
  if (n == 0) return hipSuccess;
  kv_append_kernel<<<dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream>>>(j);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t n_rows, int32_t width, const AppendDst& dst, void* out,
                            int64_t cap_rows, hipStream_t stream) {
  const int32_t units = width / 8;          // 16-byte units of a bf16 row
  const int64_t n = n_rows * units;
  copy_rows_kernel<<<dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(src), n_rows, units, dst, static_cast<uint4*>(out), cap_rows);
  return hipGetLastError();
}

hipError_t launch_ring_append(const void* k_src, const void* v_src, int64_t n_rows, int32_t C, const int32_t* row_seq,
                              const int64_t* row_pos, int32_t n_seq, int32_t W, void* ring_k, void* ring_v,
                              hipStream_t stream) {
  const int32_t units = C / 8;
  const int64_t n = n_rows * units;
  ring_append_kernel<<<dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src), n_rows, units, row_seq, row_pos, n_seq, W,
      static_cast<uint4*>(ring_k), static_cast<uint4*>(ring_v));
  return hipGetLastError();
}

}  // namespace fp4kv
