// csr.hip -- block_table and seq_lens from the packed (CSR) page-list form
// of the metadata (page "Refactor KV Cache Manager with a new torch
// exportable KVCache backend", NVIDIA/recsys-examples #400, KVCacheMetadata:
// kv_indices, kv_indptr, kv_last_page_len).  Sequence b's pages are
// kv_indices[kv_indptr[b] .. kv_indptr[b+1]) and its last page holds
// kv_last_page_len[b] rows.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pkv {

// One thread per block_table entry (consecutive threads fill one row, so the
// stores are coalesced; the row's page ids are read contiguously too; with
// more entries than the grid's threads, a thread takes every grid-size-th
// entry).  The
// row's first thread also writes the length.  Rows are cut at max_blocks and
// lengths clamped to the pages the row lists, so the attention kernels'
// reads stay inside block_table, and page ids are read only inside
// kv_indices [0, nnz), whatever the index values.
__global__ __launch_bounds__(256) void csr_to_block_table_kernel(const int64_t* __restrict__ indptr,
                                                                 const int64_t* __restrict__ indices,
                                                                 const int64_t* __restrict__ last_len, int64_t nnz,
                                                                 int64_t B, int64_t max_blocks, int64_t page_size,
                                                                 int64_t pad_page, int64_t* __restrict__ block_table,
                                                                 int64_t* __restrict__ seq_lens) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < B * max_blocks; gid += stride) {
    const int64_t b = gid / max_blocks, j = gid - b * max_blocks;
    const int64_t a = indptr[b];
    const int64_t n = indptr[b + 1] - a;  // pages of sequence b
    const int64_t e = a + j;
    block_table[gid] = j < n && e >= 0 && e < nnz ? indices[e] : pad_page;
    if (j == 0) {
      const int64_t held = n < max_blocks ? n : max_blocks;
      int64_t len = n > 0 ? (n - 1) * page_size + last_len[b] : 0;
      len = len < 0 ? 0 : (len > held * page_size ? held * page_size : len);
      seq_lens[b] = len;
    }
  }
}

// workgroups of the launch (entries are looped over beyond that): the
// launch's work-items stay below 2^32
constexpr int64_t kCsrMaxGroups = 1 << 20;

hipError_t launch_csr_to_block_table(const int64_t* indptr, const int64_t* indices, const int64_t* last_len,
                                     int64_t nnz, int64_t B, int64_t max_blocks, int64_t page_size,
                                     int64_t pad_page, int64_t* block_table, int64_t* seq_lens,
                                     hipStream_t stream) {
  const int64_t work = B * max_blocks;
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(csr_to_block_table_kernel, dim3((unsigned)std::min((work + 255) / 256, kCsrMaxGroups)), dim3(256),
                     0, stream,
                     indptr, indices, last_len, nnz, B, max_blocks, page_size, pad_page, block_table, seq_lens);
  return hipGetLastError();
}

}  // namespace pkv
