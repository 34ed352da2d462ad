// write.hip -- slot-mapping scatter of new K/V rows into the page pools.
//
// Page "Add paged / block-table KV cache export (--features paged-cache)"
// (onnxruntime/mobius #395), PR summary and table "ONNX I/O contract": each new
// token's row goes to pool row slot = page_id * page_size + offset of a
// [num_pages, page_size, kv_hidden] pool (ScatterND).  A pool row is
// Hkv * D contiguous elements, so slot * row_bytes is the byte offset of
// (page, offset) in the pool.  The copy moves 16-byte integer vectors, so any
// bit pattern (NaN payloads included) is stored unchanged; a negative slot
// writes nothing.
#include "common.h"
#include "kernels.h"

namespace pkv {

// One thread moves one 16-byte chunk of one K or V row.  Consecutive threads
// take consecutive chunks of the same row, so reads of k/v and stores into the
// pool row are both fully coalesced.
__global__ __launch_bounds__(256) void slot_scatter_kernel(const uint4* __restrict__ k,
                                                           const uint4* __restrict__ v,
                                                           const int64_t* __restrict__ slots,
                                                           uint4* __restrict__ key_pool,
                                                           uint4* __restrict__ value_pool,
                                                           int64_t n_tokens, int64_t row_vecs) {
  const int64_t per_tensor = n_tokens * row_vecs;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= 2 * per_tensor) return;
  const bool is_v = gid >= per_tensor;
  const int64_t idx = is_v ? gid - per_tensor : gid;
  const int64_t t = idx / row_vecs;
  const int64_t c = idx - t * row_vecs;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const uint4* src = is_v ? v : k;
  uint4* dst = is_v ? value_pool : key_pool;
  dst[slot * row_vecs + c] = src[t * row_vecs + c];
}

hipError_t launch_write(const WriteParams& p, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t row_vecs = p.row_bytes / 16;
  const int64_t work = 2 * p.n_tokens * row_vecs;
  const int64_t blocks = (work + 255) / 256;
  hipLaunchKernelGGL(slot_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4*)p.k, (const uint4*)p.v, p.slots, (uint4*)p.key_pool,
                     (uint4*)p.value_pool, p.n_tokens, row_vecs);
  return hipGetLastError();
}

}  // namespace pkv
