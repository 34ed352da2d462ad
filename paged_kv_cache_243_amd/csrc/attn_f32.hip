// attn_f32.hip -- paged attention for fp32 pools and fp32 queries.
//
// Same step as the bf16/fp8 kernels (page "Add paged / block-table KV cache
// export (--features paged-cache)", onnxruntime/mobius #395, "How it works"
// step 3: causal Attention over the pages named by block_table, cut to
// nonpad_kv_seqlen), for the case where the model dtype is fp32.  fp32 has no
// throughput target here and must match an fp64 reference to 1e-5, so this is
// a plain VALU kernel in fp32 arithmetic rather than a bf16 MFMA tiling.
//
// One wave per (packed query row t, KV head h) (with more rows than the grid's
// kF32MaxRowGroups, a wave takes rows t, t + gridDim.x, ...).  Lanes take 64 key positions at
// a time and compute the G dot products of their key; an online softmax
// (natural exponent, fp32) keeps a running max and sum per head; the lanes then
// switch to value dimensions and accumulate the weighted value rows.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pkv {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// rows of the grid: the launch's work-items (rows x 64) stay below 2^32
constexpr int64_t kF32MaxRowGroups = 1 << 20;

template <int D>
__device__ __forceinline__ void attention_f32_row(const AttnParams& p, const int64_t t) {
  constexpr int PER = D / 64;
  constexpr int GMAX = 16;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int G = p.G;

  // sequence owning row t: the largest b with qsl[b] <= t
  int64_t lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (p.qsl[mid] <= t) lo = mid; else hi = mid;
  }
  const int64_t b = lo;
  const int64_t L = p.seq_lens[b];
  const int64_t n_b = p.qsl[b + 1] - p.qsl[b];
  const int64_t pos = L - n_b + (t - p.qsl[b]);  // this row's position; sees keys 0..pos

  __shared__ float qs[GMAX][D];
  __shared__ float ps[GMAX][64];
  const float* q = (const float*)p.q;
  for (int idx = lane; idx < G * D; idx += 64)
    qs[idx / D][idx % D] = q[(t * p.Hq + (int64_t)h * G + idx / D) * D + idx % D];
  __syncthreads();

  const float* kpool = (const float*)p.key_pool;
  const float* vpool = (const float*)p.value_pool;
  const int64_t* bt = p.block_table + b * p.max_blocks;
  const int64_t row = (int64_t)p.Hkv * D;

  float m[GMAX], l[GMAX], o[GMAX][PER];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[g][i] = 0.f;
  }

  for (int64_t c = 0; c <= pos; c += 64) {
    const int64_t key = c + lane;
    const bool valid = key <= pos;
    float dots[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) dots[g] = 0.f;
    if (valid) {
      const float* krow = kpool + (bt[key >> 4] * kPageSize + (key & 15)) * row + (int64_t)h * D;
      for (int d = 0; d < D; ++d) {
        const float kd = krow[d];
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
          if (g < G) dots[g] = fmaf(qs[g][d], kd, dots[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      const float x = valid ? dots[g] * p.scale : -INFINITY;
      const float m_new = fmaxf(m[g], wave_max(x));
      const float alpha = expf(m[g] - m_new);
      const float w = valid ? expf(x - m_new) : 0.f;
      l[g] = l[g] * alpha + wave_sum(w);
      m[g] = m_new;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[g][i] *= alpha;
      ps[g][lane] = w;
    }
    __syncthreads();
    const int n_valid = (int)min((int64_t)64, pos - c + 1);
    for (int u = 0; u < n_valid; ++u) {
      const int64_t k2 = c + u;
      const float* vrow = vpool + (bt[k2 >> 4] * kPageSize + (k2 & 15)) * row + (int64_t)h * D;
      float v[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) v[i] = vrow[lane + 64 * i];
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= G) break;
        const float w = ps[g][u];
#pragma unroll
        for (int i = 0; i < PER; ++i) o[g][i] = fmaf(w, v[i], o[g][i]);
      }
    }
    __syncthreads();
  }

  float* out = (float*)p.out;
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
    const float inv = 1.0f / l[g];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      out[(t * p.Hq + (int64_t)h * G + g) * D + lane + 64 * i] = o[g][i] * inv;
  }
}

template <int D>
__global__ __launch_bounds__(64) void attention_f32_kernel(AttnParams p) {
  for (int64_t t = blockIdx.x; t < p.T; t += gridDim.x) {
    attention_f32_row<D>(p, t);
    __syncthreads();  // the next row rewrites the query and weight tiles
  }
}

hipError_t launch_attention_f32(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((unsigned)std::min<int64_t>(p.T, kF32MaxRowGroups), (unsigned)p.Hkv);
  if (ev.begin) (void)hipEventRecord(ev.begin, stream);
  if (p.D == 128)
    hipLaunchKernelGGL(attention_f32_kernel<128>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(64), 0, stream, p);
  if (ev.end) (void)hipEventRecord(ev.end, stream);
  return hipGetLastError();
}

}  // namespace pkv
