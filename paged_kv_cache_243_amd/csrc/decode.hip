// decode.hip -- split-K paged decode attention (one query token per sequence)
// and the log-sum-exp merge of the partitions.
//
// What is computed: for sequence b, KV head h and every query head hq of h's
// GQA group (hq in [h*G, (h+1)*G)), softmax(scale * <q_hq, k_p>) . v_p over the
// positions p < seq_lens[b], each found at row p % 16 of page
// block_table[b][p / 16] (page "Add paged / block-table KV cache export
// (--features paged-cache)", onnxruntime/mobius #395, "How it works" step 3:
// causal Attention cut to nonpad_kv_seqlen; a decode row is the last position,
// so every valid key is visible).
//
// Mapping onto gfx950:
//  * One workgroup = 4 waves = one (partition s, KV head h, sequence b).  The
//    partition covers positions [s*S, min((s+1)*S, L)); its page ids are read
//    from block_table once into LDS.  Wave w takes the partition's 32-position
//    blocks w, w+4, ... .  Every K/V byte of (b, h) is read from HBM once and
//    serves all G query heads.
//  * Scores use v_mfma_f32_16x16x32_bf16 as S^T = K . Q^T: A = 16 keys (one
//    page) x 32 dims read straight from the pool into registers, B = the G query
//    heads (zero-padded to 16 columns).  Lane l then holds 4 keys of one head,
//    so the softmax max needs two cross-lane steps and the sum none until the end.
//  * P.V uses the same MFMA as O^T = V^T . P^T.  Lane (r, g) loads an 8-key x
//    D/16-dim block of V (coalesced full rows per 16 lanes) and transposes it in
//    registers with v_perm_b32, so no LDS round trip is needed.
//  * fp8 E4M3FN codes are widened to bf16 (exact) with v_cvt_scalef32_pk_bf16_fp8;
//    the per-head k scale is folded into the logit scale and the v scale into
//    the output.
//  * Masking selects -inf for positions >= the partition end (never multiplies
//    by zero), and V rows of masked positions are zeroed before the MFMA, so
//    stale or NaN bytes in unused slots cannot reach the output.
//  * The four waves' (m, l, O) states merge through LDS.  A sequence with a
//    single partition writes its normalised output directly; otherwise the
//    partition's unnormalised O with (m, l) goes to the workspace and
//    merge_kernel combines the partitions:
//        M = max_s m_s,  out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kDecodeWaves = 4;
constexpr int kMaxSplitPages = 256;  // split_tokens <= 4096

template <int ESZ, int D>
struct DecodeTraits {
  static constexpr int NKK = D / 32;  // score MFMAs per page
  static constexpr int NJ = D / 16;   // value dims per lane = output MFMAs
};

// K operand of one page for score MFMA kk: row (lane & 15) of the page, dims
// [32*kk + 8*grp, +8).
template <int ESZ, int D>
__device__ __forceinline__ void load_k_page(const char* __restrict__ page_row, int grp,
                                            bf16x8 (&ka)[D / 32]) {
  constexpr int NKK = D / 32;
  if constexpr (ESZ == 2) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      ka[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(page_row + (32 * kk + 8 * grp) * 2));
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x2 c = *(const u32x2*)(page_row + 32 * kk + 8 * grp);
      const u32x2 a = fp8x4_to_bf16x4(c.x), b = fp8x4_to_bf16x4(c.y);
      const u32x4 w = {a.x, a.y, b.x, b.y};
      ka[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// Raw V rows a lane needs: 8 keys (4*grp + e of page 0 for e < 4, 4*grp + e - 4
// of page 1 otherwise), dims [r*NJ, (r+1)*NJ) with r = lane & 15.
template <int ESZ, int D>
struct VRows {
  static constexpr int NJ = D / 16;
  static constexpr int DW = (NJ * ESZ) / 4;  // dwords per row chunk (bf16: NJ/2, fp8: NJ/4)
  uint32_t w[8][DW];
};

template <int ESZ, int D>
__device__ __forceinline__ void load_v_rows(const char* __restrict__ p0, const char* __restrict__ p1,
                                            int64_t row_stride, int grp, int r,
                                            VRows<ESZ, D>& vr) {
  constexpr int NJ = D / 16;
  constexpr int DW = VRows<ESZ, D>::DW;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const char* base = (e < 4 ? p0 : p1) + (int64_t)(4 * grp + (e & 3)) * row_stride + r * NJ * ESZ;
    if constexpr (DW == 4) {
      u32x4 x = *(const u32x4*)base;
      vr.w[e][0] = x.x; vr.w[e][1] = x.y; vr.w[e][2] = x.z; vr.w[e][3] = x.w;
    } else if constexpr (DW == 2) {
      u32x2 x = *(const u32x2*)base;
      vr.w[e][0] = x.x; vr.w[e][1] = x.y;
    } else {
      vr.w[e][0] = *(const uint32_t*)base;
    }
  }
}

// Zero the V rows of masked keys (key e of this lane invalid).
template <int ESZ, int D>
__device__ __forceinline__ void mask_v_rows(VRows<ESZ, D>& vr, const bool (&valid)[8]) {
  constexpr int DW = VRows<ESZ, D>::DW;
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < DW; ++i) vr.w[e][i] = valid[e] ? vr.w[e][i] : 0u;
}

// Transpose the 8 x NJ block into NJ MFMA A operands: va[j] holds dim r*NJ + j of
// the 8 keys, as bf16.
template <int ESZ, int D>
__device__ __forceinline__ void transpose_v(const VRows<ESZ, D>& vr, bf16x8 (&va)[D / 16]) {
  constexpr int NJ = D / 16;
  if constexpr (ESZ == 2) {
    // dword q of operand j = (key 2q, key 2q+1) elements j
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 o;
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = vr.w[2 * q][j >> 1], y = vr.w[2 * q + 1][j >> 1];
        o[q] = __builtin_amdgcn_perm(y, x, sel);
      }
      va[j] = __builtin_bit_cast(bf16x8, o);
    }
  } else {
    // interleave bytes of keys (2q, 2q+1), then widen pairs to bf16
    u32x4 o[NJ];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int wd = 0; wd < NJ / 4; ++wd) {
        const uint32_t x = vr.w[2 * q][wd], y = vr.w[2 * q + 1][wd];
        const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05010400u);  // (x0, y0, x1, y1)
        const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07030602u);  // (x2, y2, x3, y3)
        const u32x2 ab = fp8x4_to_bf16x4(lo), cd = fp8x4_to_bf16x4(hi);
        o[4 * wd + 0][q] = ab.x;
        o[4 * wd + 1][q] = ab.y;
        o[4 * wd + 2][q] = cd.x;
        o[4 * wd + 3][q] = cd.y;
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) va[j] = __builtin_bit_cast(bf16x8, o[j]);
  }
}

template <int ESZ, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(AttnParams p) {
  constexpr int NKK = D / 32;
  constexpr int NJ = D / 16;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  const int64_t L = p.seq_lens[b];
  const int64_t q_row = p.qsl[b];
  if (p.qsl[b + 1] == q_row) return;  // no query row for this sequence
  const int64_t start = (int64_t)s * p.split_tokens;
  if (start >= L) return;
  const int64_t end = min(start + (int64_t)p.split_tokens, L);
  const int n_blocks = (int)((end - start + 31) >> 5);
  const int n_parts = (int)((L + p.split_tokens - 1) / p.split_tokens);

  __shared__ int32_t s_pages[kMaxSplitPages];
  __shared__ float s_m[kDecodeWaves][16];
  __shared__ float s_l[kDecodeWaves][16];
  __shared__ float s_o[kDecodeWaves][D][17];

  // page ids of this partition; entries past the sequence's last page are never
  // read from block_table (their positions are masked), the last valid page
  // stands in for them.
  {
    const int64_t first = start >> 4;
    const int64_t last_valid = ((L + 15) >> 4) - 1;
    const int64_t* row = p.block_table + (int64_t)b * p.max_blocks;
    for (int i = tid; i < 2 * n_blocks; i += 256) {
      int64_t lp = first + i;
      lp = lp > last_valid ? last_valid : lp;
      s_pages[i] = (int32_t)row[lp];
    }
  }

  // query operand: head col of the group (zero for padding columns)
  bf16x8 qb[NKK];
  {
    const int hq = h * p.G + col;
    const __bf16* qrow = (const __bf16*)p.q + ((int64_t)q_row * p.Hq + hq) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (col < p.G) x = *(const u32x4*)(qrow + 32 * kk + 8 * grp);
      qb[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  float logit_scale = p.scale * kLog2e;
  if constexpr (ESZ == 1) logit_scale *= p.k_scale[h];
  __syncthreads();

  const int64_t row_stride = (int64_t)p.Hkv * D * ESZ;
  const int64_t page_stride = row_stride * kPageSize;
  const char* kbase = (const char*)p.key_pool + (int64_t)h * D * ESZ;
  const char* vbase = (const char*)p.value_pool + (int64_t)h * D * ESZ;

  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int blk = wave; blk < n_blocks; blk += kDecodeWaves) {
    const int64_t pos0 = start + 32 * (int64_t)blk;
    const char* kp0 = kbase + (int64_t)s_pages[2 * blk] * page_stride;
    const char* kp1 = kbase + (int64_t)s_pages[2 * blk + 1] * page_stride;
    const char* vp0 = vbase + (int64_t)s_pages[2 * blk] * page_stride;
    const char* vp1 = vbase + (int64_t)s_pages[2 * blk + 1] * page_stride;

    bf16x8 k0[NKK], k1[NKK];
    load_k_page<ESZ, D>(kp0 + col * row_stride, grp, k0);
    load_k_page<ESZ, D>(kp1 + col * row_stride, grp, k1);
    VRows<ESZ, D> vr;
    load_v_rows<ESZ, D>(vp0, vp1, row_stride, grp, col, vr);

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s0 = mfma16(k0[kk], qb[kk], s0);
      s1 = mfma16(k1[kk], qb[kk], s1);
    }
    // lane holds keys pos0 + 4*grp + i (s0) and pos0 + 16 + 4*grp + i (s1)
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = s0[i] * logit_scale;
      x[4 + i] = s1[i] * logit_scale;
    }
    if (pos0 + 32 > end) {  // only the partition's last block can be partial
      bool valid[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t pos = pos0 + (e < 4 ? 0 : 16) + 4 * grp + (e & 3);
        valid[e] = pos < end;
        x[e] = valid[e] ? x[e] : -INFINITY;
      }
      mask_v_rows<ESZ, D>(vr, valid);
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, xor_shuffle(mx, 16));
    mx = fmaxf(mx, xor_shuffle(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
      psum += pr[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] *= alpha;
    }
    u32x4 pw;
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[q] = pack_bf16x2(pr[2 * q], pr[2 * q + 1]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);

    bf16x8 va[NJ];
    transpose_v<ESZ, D>(vr, va);
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = mfma16(va[j], pb, acc[j]);
  }

  // combine the lane groups' partial sums (same head, same running max)
  l_run += xor_shuffle(l_run, 16);
  l_run += xor_shuffle(l_run, 32);
  if (grp == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  // acc[j][i] = O^T[dim (4*grp + i)*NJ + j][head col]
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][(4 * grp + i) * NJ + j][col] = acc[j][i];
  __syncthreads();

  float out_scale = 1.0f;
  if constexpr (ESZ == 1) out_scale = p.v_scale[h];
  for (int idx = tid; idx < p.G * D; idx += 256) {
    const int c = idx / D, d = idx - c * D;
    float M = s_m[0][c];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][c]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][c] - M);  // 0 for a wave that saw no block
      o += f * s_o[w][d][c];
      l += f * s_l[w][c];
    }
    const int hq = h * p.G + c;
    if (n_parts == 1) {
      ((__bf16*)p.out)[((int64_t)q_row * p.Hq + hq) * D + d] = (__bf16)(o * out_scale / l);
    } else {
      const int64_t slot = ((int64_t)b * p.n_splits + s) * p.Hq + hq;
      p.ws_o[slot * D + d] = o * out_scale;
      if (d == 0) {
        p.ws_ml[2 * slot] = M;
        p.ws_ml[2 * slot + 1] = l;
      }
    }
  }
}

// One wave per (query head, sequence): log-sum-exp merge of the partitions.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(AttnParams p) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t q_row = p.qsl[b];
  if (p.qsl[b + 1] == q_row) return;
  const int64_t L = p.seq_lens[b];
  const int n_parts = (int)((L + p.split_tokens - 1) / p.split_tokens);
  if (n_parts <= 1) return;  // written directly by the split kernel
  const int64_t base = (int64_t)b * p.n_splits * p.Hq + hq;
  float M = -INFINITY;
  for (int s = 0; s < n_parts; ++s) M = fmaxf(M, p.ws_ml[2 * (base + (int64_t)s * p.Hq)]);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float l = 0.f;
  for (int s = 0; s < n_parts; ++s) {
    const int64_t slot = base + (int64_t)s * p.Hq;
    const float f = __builtin_amdgcn_exp2f(p.ws_ml[2 * slot] - M);
    l += f * p.ws_ml[2 * slot + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += f * p.ws_o[slot * D + lane + 64 * i];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    ((__bf16*)p.out)[((int64_t)q_row * p.Hq + hq) * D + lane + 64 * i] = (__bf16)(o[i] * inv);
}

size_t decode_workspace_bytes(int64_t B, int Hq, int D, int n_splits) {
  if (n_splits <= 1) return 0;
  const size_t slots = (size_t)B * n_splits * Hq;
  return slots * D * sizeof(float) + slots * 2 * sizeof(float);
}

template <int ESZ, int D>
static void launch_decode_t(const AttnParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.n_splits, (unsigned)p.Hkv, (unsigned)p.B);
  hipLaunchKernelGGL((decode_split_kernel<ESZ, D>), grid, dim3(256), 0, stream, p);
  if (p.n_splits > 1)
    hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)p.Hq, (unsigned)p.B), dim3(64), 0, stream, p);
}

hipError_t launch_decode(const AttnParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  const bool fp8 = p.kv_type == KV_FP8;
  if (p.D == 128) {
    if (fp8) launch_decode_t<1, 128>(p, stream); else launch_decode_t<2, 128>(p, stream);
  } else {
    if (fp8) launch_decode_t<1, 64>(p, stream); else launch_decode_t<2, 64>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
