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

// ---------------------------------------------------------------------------
// Quantising form for fp8 pools: bf16 rows in, OCP E4M3FN codes out.  Element
// x of KV head h is stored as the code of y = x / scale[h] (one IEEE binary32
// division; scale[h] is the factor the attention multiplies codes by),
// rounded to nearest even, with |y| beyond 448 saturated to +-448 (the format
// has no infinity) and a NaN x stored as the NaN code with x's sign.  The rounding is
// gfx950's own fp32 -> fp8 conversion, fed values already clamped to +-448 so
// that it never overflows.

// Codes of the quotients ya = xa / s and yb = xb / s (ya in bits 0..7, yb
// in bits 8..15).  fmax/fmin return the other operand for a NaN, so NaNs
// (which arise exactly from NaN inputs, the scale being positive and finite)
// are patched afterwards from the input's sign bit.
__device__ __forceinline__ uint32_t e4m3fn_pair(float ya, float yb, uint32_t xa_bits, uint32_t xb_bits) {
  const float ca = __builtin_fminf(__builtin_fmaxf(ya, -448.0f), 448.0f);
  const float cb = __builtin_fminf(__builtin_fmaxf(yb, -448.0f), 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if (ya != ya) r = (r & 0xFF00u) | ((xa_bits >> 31) ? 0xFFu : 0x7Fu);
  if (yb != yb) r = (r & 0x00FFu) | ((xb_bits >> 31) ? 0xFF00u : 0x7F00u);
  return r;
}

// One thread converts 8 consecutive elements of one K or V row (16 bytes in,
// 8 bytes out); consecutive threads take consecutive groups, so loads and
// stores are coalesced.  D is a multiple of 8, so a group lies in one head.
__global__ __launch_bounds__(256) void slot_scatter_fp8_kernel(const uint4* __restrict__ k,
                                                               const uint4* __restrict__ v,
                                                               const int64_t* __restrict__ slots,
                                                               uint2* __restrict__ key_pool,
                                                               uint2* __restrict__ value_pool,
                                                               const float* __restrict__ k_scale,
                                                               const float* __restrict__ v_scale,
                                                               int64_t n_tokens, int64_t row_groups,
                                                               int64_t head_groups) {
  const int64_t per_tensor = n_tokens * row_groups;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= 2 * per_tensor) return;
  const bool is_v = gid >= per_tensor;
  const int64_t idx = is_v ? gid - per_tensor : gid;
  const int64_t t = idx / row_groups;
  const int64_t c = idx - t * row_groups;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const float s = (is_v ? v_scale : k_scale)[c / head_groups];
  const uint4 x = (is_v ? v : k)[t * row_groups + c];
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t code[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t xl = w[i] << 16, xh = w[i] & 0xFFFF0000u;
    code[i] = e4m3fn_pair(__builtin_bit_cast(float, xl) / s, __builtin_bit_cast(float, xh) / s, xl, xh);
  }
  uint2 out;
  out.x = code[0] | (code[1] << 16);
  out.y = code[2] | (code[3] << 16);
  (is_v ? value_pool : key_pool)[slot * row_groups + c] = out;
}

hipError_t launch_write_fp8(const WriteFp8Params& p, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t row_groups = p.Hkv * p.D / 8;
  const int64_t work = 2 * p.n_tokens * row_groups;
  const int64_t blocks = (work + 255) / 256;
  hipLaunchKernelGGL(slot_scatter_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4*)p.k, (const uint4*)p.v, p.slots, (uint2*)p.key_pool,
                     (uint2*)p.value_pool, p.k_scale, p.v_scale, p.n_tokens, row_groups, p.D / 8);
  return hipGetLastError();
}

}  // namespace pkv
