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
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pkv {

// A workgroup per new token (tokens t = blockIdx.x, + gridDim.x, ... when
// there are more tokens than workgroups): the token's slot is read once (a
// negative slot skips it), and the threads move the row's 16-byte chunks, the
// K row's and the V row's, consecutive threads taking consecutive chunks, so
// the reads of k/v and the stores into the pool rows are both fully coalesced.
__global__ __launch_bounds__(256) void slot_scatter_kernel(const uint4* __restrict__ k,
                                                           const uint4* __restrict__ v,
                                                           const int64_t* __restrict__ slots,
                                                           uint4* __restrict__ key_pool,
                                                           uint4* __restrict__ value_pool,
                                                           int64_t row_vecs, int64_t n_tokens) {
  for (int64_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
    const int64_t slot = slots[t];
    if (slot < 0) continue;
    const uint4* ks = k + t * row_vecs;
    const uint4* vs = v + t * row_vecs;
    uint4* kd = key_pool + slot * row_vecs;
    uint4* vd = value_pool + slot * row_vecs;
    for (int64_t c = threadIdx.x; c < row_vecs; c += blockDim.x) {
      const uint4 a = ks[c], b = vs[c];
      kd[c] = a;
      vd[c] = b;
    }
  }
}

// threads per write workgroup: the row's chunks rounded up to whole waves, at most 256
static unsigned write_threads(int64_t row_chunks) {
  return (unsigned)std::min<int64_t>(256, (row_chunks + 63) / 64 * 64);
}

// workgroups of a write launch: one per token, at most kWriteMaxGroups (the
// workgroups then loop over the tokens), which keeps the launch's work-items
// (workgroups x threads) below 2^32
constexpr int64_t kWriteMaxGroups = 1 << 20;
static unsigned write_groups(int64_t n_tokens) { return (unsigned)std::min(n_tokens, kWriteMaxGroups); }

hipError_t launch_write(const WriteParams& p, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t row_vecs = p.row_bytes / 16;
  hipLaunchKernelGGL(slot_scatter_kernel, dim3(write_groups(p.n_tokens)), dim3(write_threads(row_vecs)), 0, stream,
                     (const uint4*)p.k, (const uint4*)p.v, p.slots, (uint4*)p.key_pool, (uint4*)p.value_pool,
                     row_vecs, p.n_tokens);
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

// A workgroup per new token, as in the plain write (its slot read once; a
// negative slot skips it); a thread converts 8 consecutive elements of the K
// row and the same 8 of the V row (16 bytes in, 8 bytes out each),
// consecutive threads taking consecutive groups, so loads and stores are
// coalesced.  D is a multiple of 8, so a group lies in one head.
__global__ __launch_bounds__(256) void slot_scatter_fp8_kernel(const uint4* __restrict__ k,
                                                               const uint4* __restrict__ v,
                                                               const int64_t* __restrict__ slots,
                                                               uint2* __restrict__ key_pool,
                                                               uint2* __restrict__ value_pool,
                                                               const float* __restrict__ k_scale,
                                                               const float* __restrict__ v_scale,
                                                               int64_t row_groups, int32_t head_groups,
                                                               int64_t n_tokens) {
  auto convert = [](const uint4 x, float s) {
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
    return out;
  };
  for (int64_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
    const int64_t slot = slots[t];
    if (slot < 0) continue;
    for (int64_t c = threadIdx.x; c < row_groups; c += blockDim.x) {
      const uint32_t h = (uint32_t)c / (uint32_t)head_groups;
      const uint4 xk = k[t * row_groups + c], xv = v[t * row_groups + c];
      const float sk = k_scale[h], sv = v_scale[h];
      key_pool[slot * row_groups + c] = convert(xk, sk);
      value_pool[slot * row_groups + c] = convert(xv, sv);
    }
  }
}

hipError_t launch_write_fp8(const WriteFp8Params& p, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t row_groups = p.Hkv * p.D / 8;
  hipLaunchKernelGGL(slot_scatter_fp8_kernel, dim3(write_groups(p.n_tokens)), dim3(write_threads(row_groups)), 0,
                     stream, (const uint4*)p.k, (const uint4*)p.v, p.slots, (uint2*)p.key_pool,
                     (uint2*)p.value_pool, p.k_scale, p.v_scale, row_groups, (int32_t)(p.D / 8), p.n_tokens);
  return hipGetLastError();
}

}  // namespace pkv
