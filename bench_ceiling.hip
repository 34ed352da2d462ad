// bench_ceiling.hip -- measurement kernel for bench.py (not part of
// libpagedkv.so): a plain read-only stream over a list of KV pages, as the
// practical HBM ceiling of a paged decode.  It reads every byte of the listed
// pages of two pools (the K and the V pool) once, in list order, with the
// decode kernel's access shape (16-byte non-temporal buffer loads, a page base
// in a scalar descriptor, one workgroup of 8 waves per CU streaming a
// contiguous range of the list), and does no other work: each lane folds what
// it loaded into one word by XOR so the loads stay live, and each wave stores
// one word to `sink`.
//
//   stream_read_pages(key_pool, value_pool, pages [n_pages] int64, n_pages,
//                     page_bytes (a multiple of 8192), workgroups, sink
//                     [workgroups * 8] uint32, stream)
// Page ids must be in range; returns 0, or -1 for bad arguments, or the HIP
// error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kChunk = kThreads * 16;  // bytes one load instruction of the workgroup covers
constexpr int kWord3 = 0x00020000;     // raw buffer descriptor, 32-bit data format
constexpr int kNonTemporal = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, kWord3);
}

// PER = page_bytes / kChunk loads per page and pool.  A ring of DEPTH list
// entries is in flight: entry i + DEPTH is issued as soon as entry i has been
// folded.  Entries past the range get a zero-length descriptor, so their loads
// return zeros without touching memory and every issue is unconditional (the
// waits then count exactly the older entries).
constexpr int kDepth = 4;

template <int PER>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* kp, const char* vp, const int64_t* pages,
                                                               int64_t n_pages, uint32_t* sink) {
  const int tid = threadIdx.x;
  const int64_t W = gridDim.x, w = blockIdx.x;
  const int64_t lo = n_pages * w / W, hi = n_pages * (w + 1) / W;
  const uint32_t page_bytes = (uint32_t)PER * kChunk;
  uint32_t acc = 0;
  u32x4 r[kDepth][2 * PER];
  auto issue = [&](u32x4 (&d)[2 * PER], int64_t i) {
    const bool live = i < hi;
    const int64_t pg = live ? pages[i] : 0;
    const uint32_t bytes = live ? page_bytes : 0u;
    const auto rk = page_rsrc(kp + pg * page_bytes, bytes);
    const auto rv = page_rsrc(vp + pg * page_bytes, bytes);
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      d[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, tid * 16 + c * kChunk, 0, kNonTemporal);
      d[PER + c] = __builtin_amdgcn_raw_buffer_load_b128(rv, tid * 16 + c * kChunk, 0, kNonTemporal);
    }
  };
#pragma unroll
  for (int s = 0; s < kDepth; ++s) issue(r[s], lo + s);
  for (int64_t i = lo; i < hi; i += kDepth) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
#pragma unroll
      for (int c = 0; c < 2 * PER; ++c) acc ^= r[s][c].x ^ r[s][c].y ^ r[s][c].z ^ r[s][c].w;
      issue(r[s], i + s + kDepth);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) sink[w * (kThreads / 64) + tid / 64] = acc;
}

}  // namespace

extern "C" int stream_read_pages(const void* key_pool, const void* value_pool, const int64_t* pages, int64_t n_pages,
                                 int64_t page_bytes, int workgroups, uint32_t* sink, void* stream) {
  if (!key_pool || !value_pool || !pages || !sink || n_pages < 0 || workgroups <= 0) return -1;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)workgroups), block(kThreads);
  switch (page_bytes) {
    case 1 * kChunk: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, s, (const char*)key_pool,
                                        (const char*)value_pool, pages, n_pages, sink); break;
    case 2 * kChunk: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, s, (const char*)key_pool,
                                        (const char*)value_pool, pages, n_pages, sink); break;
    case 4 * kChunk: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, s, (const char*)key_pool,
                                        (const char*)value_pool, pages, n_pages, sink); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}
