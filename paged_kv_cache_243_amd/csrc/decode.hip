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
//  * Stream-K work split.  The work is the list of (sequence, unit) pairs, a
//    unit being 32 consecutive positions (two pages) of one sequence for all KV
//    heads.  The grid has one 8-wave workgroup per CU (or a multiple of the CU
//    count when the caller asks for smaller partitions); workgroup w takes the
//    w-th of gridDim.x equal contiguous ranges, so every CU streams the same
//    number of bytes whatever the length mix.  Wave k of a workgroup handles KV
//    head k (or heads k, k + 8, ...): the waves of a workgroup read the same
//    pages together, so HBM sees whole 2 KiB rows.  Every K/V byte of (b, h) is
//    read from HBM once and serves all G query heads.
//  * Page ids come from block_table through a 64-entry window held one per
//    lane and broadcast with v_readlane; the next unit's loads are issued
//    before the current unit is computed (register double buffering).
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
//  * Masking selects -inf for positions >= seq_lens (never multiplies by zero),
//    and V rows of masked positions are zeroed before the MFMA, so stale or NaN
//    bytes in unused slots cannot reach the output.
//  * A segment (the part of one sequence inside a workgroup's range) that is a
//    whole sequence writes its normalised output directly; otherwise it writes
//    its unnormalised O with (m, l) to a partial slot and merge_kernel combines
//    a sequence's partials:
//        M = max_w m_w,  out = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kUnit = 32;      // key positions per unit of work (two pages)
// dword 3 of a raw (unformatted, stride 0) buffer descriptor: 32-bit data format
constexpr int kBufferWord3 = 0x00020000;
// cache policy of the KV stream: non-temporal (each byte is read once)
constexpr int kStreamAux = 2;
constexpr int kMaxWaves = 8;   // waves per workgroup

__host__ __device__ inline int decode_heads_per_wave(int Hkv) { return (Hkv + kMaxWaves - 1) / kMaxWaves; }
__host__ __device__ inline int decode_waves(int Hkv) {
  const int hpw = decode_heads_per_wave(Hkv);
  return (Hkv + hpw - 1) / hpw;
}

// Units of sequence b: its 32-position blocks, or none when it has no query row.
__device__ __forceinline__ int32_t seq_units(const AttnParams& p, int b) {
  if (p.qsl[b + 1] == p.qsl[b]) return 0;
  return (int32_t)((p.seq_lens[b] + kUnit - 1) / kUnit);
}

// Raw K and V bytes of one unit for one KV head, as one lane holds them.
template <int ESZ, int D>
struct UnitRegs {
  static constexpr int KDW = 2 * ESZ;                 // dwords per K chunk of 8 elements
  static constexpr int VDW = (D / 16) * ESZ / 4;      // dwords per V row chunk
  uint32_t k[2][D / 32][KDW];
  uint32_t v[8][VDW];
};

// Buffer resource for one page: wave-uniform base (forced into scalar
// registers), `bytes` addressable bytes; loads past them read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, kBufferWord3);
}

// Per-lane address parts of a unit (32-bit offsets from a page base).
struct LaneOffsets {
  uint32_t k;     // K row (lane & 15), dims [8*grp, +8) of each 32-dim chunk
  uint32_t v[4];  // V rows 4*grp + e (e < 4), dims [col*NJ, +NJ)
};

// Loads of one unit: page bases live in buffer descriptors (scalar
// registers), the per-lane part of every address is a 32-bit offset.
template <int ESZ, int D>
__device__ __forceinline__ void issue_k(UnitRegs<ESZ, D>& u, __amdgpu_buffer_rsrc_t kp0, __amdgpu_buffer_rsrc_t kp1,
                                        const LaneOffsets& off) {
  constexpr int NKK = D / 32;
  using U = UnitRegs<ESZ, D>;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int o = (int)off.k + 32 * kk * ESZ;
      if constexpr (U::KDW == 4) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(pp ? kp1 : kp0, o, 0, kStreamAux);
        u.k[pp][kk][0] = x.x; u.k[pp][kk][1] = x.y; u.k[pp][kk][2] = x.z; u.k[pp][kk][3] = x.w;
      } else {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(pp ? kp1 : kp0, o, 0, kStreamAux);
        u.k[pp][kk][0] = x.x; u.k[pp][kk][1] = x.y;
      }
    }
  }
}

template <int ESZ, int D>
__device__ __forceinline__ void issue_v(UnitRegs<ESZ, D>& u, __amdgpu_buffer_rsrc_t vp0, __amdgpu_buffer_rsrc_t vp1,
                                        const LaneOffsets& off) {
  using U = UnitRegs<ESZ, D>;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __amdgpu_buffer_rsrc_t r = e < 4 ? vp0 : vp1;
    const int o = (int)off.v[e & 3];
    if constexpr (U::VDW == 4) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, kStreamAux);
      u.v[e][0] = x.x; u.v[e][1] = x.y; u.v[e][2] = x.z; u.v[e][3] = x.w;
    } else if constexpr (U::VDW == 2) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, kStreamAux);
      u.v[e][0] = x.x; u.v[e][1] = x.y;
    } else {
      u.v[e][0] = __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, kStreamAux);
    }
  }
}

// Page ids of unit j of a sequence (its logical pages 2j and 2j+1), read with
// wave-uniform scalar loads; positions past the sequence's last page reuse
// that page (they are masked).
struct UnitPages {
  int64_t p0, p1;
};
__device__ __forceinline__ UnitPages unit_pages(const __attribute__((address_space(4))) int64_t* bt_row,
                                                int64_t j, int64_t last_page) {
  const int64_t a = min(2 * j, last_page), b = min(2 * j + 1, last_page);
  return UnitPages{bt_row[a], bt_row[b]};
}

// K chunk (page pp, MFMA kk) as a bf16 operand.
template <int ESZ, int D>
__device__ __forceinline__ bf16x8 k_operand(const UnitRegs<ESZ, D>& u, int pp, int kk) {
  if constexpr (ESZ == 2) {
    const u32x4 w = {u.k[pp][kk][0], u.k[pp][kk][1], u.k[pp][kk][2], u.k[pp][kk][3]};
    return __builtin_bit_cast(bf16x8, w);
  } else {
    const u32x2 a = fp8x4_to_bf16x4(u.k[pp][kk][0]), b = fp8x4_to_bf16x4(u.k[pp][kk][1]);
    const u32x4 w = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, w);
  }
}

// One unit of the online softmax for one KV head: scores for 32 keys, running
// max/sum update, P.V accumulation.  pos0 = position of the unit's first key;
// keys at positions >= len are masked.
// next_k() runs once the K registers have been consumed (it issues the next
// unit's K loads into them); next_v() runs once the V registers have been
// consumed.
template <int ESZ, int D, class NextK, class NextV>
__device__ __forceinline__ void consume_unit(UnitRegs<ESZ, D>& u, const bf16x8 (&qb)[D / 32], f32x4 (&acc)[D / 16],
                                             float& m_run, float& l_run, float logit_scale, int64_t pos0,
                                             int64_t len, int grp, NextK next_k, NextV next_v) {
  constexpr int NKK = D / 32, NJ = D / 16;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    s0 = mfma16(k_operand<ESZ, D>(u, 0, kk), qb[kk], s0);
    s1 = mfma16(k_operand<ESZ, D>(u, 1, kk), qb[kk], s1);
  }
  next_k();
  // lane holds keys pos0 + 4*grp + i (s0) and pos0 + 16 + 4*grp + i (s1)
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i] * logit_scale;
    x[4 + i] = s1[i] * logit_scale;
  }
  if (pos0 + kUnit > len) {  // only a sequence's last unit can be partial
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool valid = pos0 + (e < 4 ? 0 : 16) + 4 * grp + (e & 3) < len;
      x[e] = valid ? x[e] : -INFINITY;
#pragma unroll
      for (int i = 0; i < UnitRegs<ESZ, D>::VDW; ++i) u.v[e][i] = valid ? u.v[e][i] : 0u;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
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
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] *= alpha;
  u32x4 pw;
#pragma unroll
  for (int q = 0; q < 4; ++q) pw[q] = pack_bf16x2(pr[2 * q], pr[2 * q + 1]);
  const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);

  // P.V: operand j holds dim r*NJ + j of the lane's 8 keys; built right before
  // its MFMA so the raw rows die progressively
  if constexpr (ESZ == 2) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(u.v[2 * q + 1][j >> 1], u.v[2 * q][j >> 1], sel);
      acc[j] = mfma16(__builtin_bit_cast(bf16x8, o), pb, acc[j]);
    }
  } else {
#pragma unroll
    for (int wd = 0; wd < NJ / 4; ++wd) {
      u32x4 o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = u.v[2 * q][wd], y = u.v[2 * q + 1][wd];
        const u32x2 ab = fp8x4_to_bf16x4(__builtin_amdgcn_perm(y, x, 0x05010400u));  // keys 2q, 2q+1 dims 0, 1
        const u32x2 cd = fp8x4_to_bf16x4(__builtin_amdgcn_perm(y, x, 0x07030602u));  // dims 2, 3
        o[0][q] = ab.x;
        o[1][q] = ab.y;
        o[2][q] = cd.x;
        o[3][q] = cd.y;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[4 * wd + t] = mfma16(__builtin_bit_cast(bf16x8, o[t]), pb, acc[4 * wd + t]);
    }
  }
  next_v();
}

// Stream-K decode.  The flattened list of (sequence, unit) pairs is cut into
// gridDim.x equal contiguous ranges, one per workgroup; a workgroup walks the
// sequences its range overlaps (segments).  Wave w handles KV heads w, w +
// waves, ... of every segment.  A segment that covers a whole sequence writes
// the normalised output; otherwise it writes an unnormalised partial to slot
// (b + workgroup), which merge_kernel combines.  Slots are unique because the
// ranges are ordered: a later sequence only meets later workgroups.
template <int ESZ, int D>
__global__ __launch_bounds__(512) void decode_kernel(AttnParams p) {
  constexpr int NKK = D / 32;
  constexpr int NJ = D / 16;
  __shared__ int32_t s_cum[kDecodeMaxSeqs + 1];
  __shared__ int32_t s_scan[512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int col = lane & 15, grp = lane >> 4;
  const int B = (int)p.B;

  // ---- units before each sequence (block-wide exclusive scan)
  {
    const int per = (B + nthreads - 1) / nthreads;
    const int b_lo = tid * per;
    int32_t run = 0;
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b < B) run += seq_units(p, b);
    }
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < nthreads; off <<= 1) {
      const int32_t v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int32_t acc_units = tid ? s_scan[tid - 1] : 0;
    if (tid == 0) s_cum[0] = 0;
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b < B) {
        acc_units += seq_units(p, b);
        s_cum[b + 1] = acc_units;
      }
    }
    __syncthreads();
  }
  const int W = gridDim.x, wg = blockIdx.x;
  if (wg == 0)
    for (int b = tid; b <= B; b += nthreads) p.ws_cum[b] = s_cum[b];
  const int64_t U = s_cum[B];
  const int32_t u0 = (int32_t)(((int64_t)wg * U) / W);
  const int32_t u1 = (int32_t)(((int64_t)(wg + 1) * U) / W);
  if (u0 >= u1) return;

  // sequence holding unit u0: the largest b with s_cum[b] <= u0
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= u0) lo = mid; else hi = mid - 1;
  }

  const int hpw = decode_heads_per_wave(p.Hkv);
  const int waves = nthreads >> 6;
  const uint32_t row_stride = (uint32_t)p.Hkv * D * ESZ;
  const int64_t page_stride = (int64_t)row_stride * kPageSize;
  LaneOffsets off;
  off.k = (uint32_t)col * row_stride + 8 * grp * ESZ;
#pragma unroll
  for (int e = 0; e < 4; ++e) off.v[e] = (uint32_t)(4 * grp + e) * row_stride + col * NJ * ESZ;

  for (int b = __builtin_amdgcn_readfirstlane(lo); b < B; ++b) {
    const int32_t cb = s_cum[b], ce = s_cum[b + 1];
    if (cb >= u1) break;
    const int32_t seg_lo = __builtin_amdgcn_readfirstlane(max(u0, cb));
    const int32_t seg_hi = __builtin_amdgcn_readfirstlane(min(u1, ce));
    if (seg_lo >= seg_hi) continue;
    const bool whole = seg_lo == cb && seg_hi == ce;
    const int j0 = seg_lo - cb, j1 = seg_hi - cb;  // units of b in this segment
    const int64_t L = p.seq_lens[b];
    const int64_t q_row = p.qsl[b];
    const int64_t last_page = ((L + 15) >> 4) - 1;
    const __attribute__((address_space(4))) int64_t* bt_row =
        (const __attribute__((address_space(4))) int64_t*)(p.block_table + (int64_t)b * p.max_blocks);

    for (int hk = 0; hk < hpw; ++hk) {
      const int h = wave + hk * waves;
      if (h >= p.Hkv) break;
      // query operand: head col of the group (zero for padding columns)
      bf16x8 qb[NKK];
      {
        const __bf16* qrow = (const __bf16*)p.q + (q_row * p.Hq + h * p.G + col) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (col < p.G) x = *(const u32x4*)(qrow + 32 * kk + 8 * grp);
          qb[kk] = __builtin_bit_cast(bf16x8, x);
        }
      }
      float logit_scale = p.scale * kLog2e;
      if constexpr (ESZ == 1) logit_scale *= p.k_scale[h];
      const char* kbase = (const char*)p.key_pool + (int64_t)h * D * ESZ;
      const char* vbase = (const char*)p.value_pool + (int64_t)h * D * ESZ;
      const uint32_t page_bytes = (uint32_t)page_stride;
      auto krsrc = [&](int64_t pg) { return page_rsrc(kbase + pg * page_stride, page_bytes); };
      auto vrsrc = [&](int64_t pg) { return page_rsrc(vbase + pg * page_stride, page_bytes); };

      f32x4 acc[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m_run = -INFINITY, l_run = 0.f;

      // One unit of registers: unit j+1's K loads are issued into them as soon
      // as unit j's scores are computed, its V loads as soon as unit j's P.V is
      // done, so each load has a whole unit of compute to land.  Page ids are
      // fetched one unit further ahead.
      UnitRegs<ESZ, D> u;
      const UnitPages first = unit_pages(bt_row, j0, last_page);
      UnitPages nxt = unit_pages(bt_row, j0 + 1, last_page);
      issue_k<ESZ, D>(u, krsrc(first.p0), krsrc(first.p1), off);
      issue_v<ESZ, D>(u, vrsrc(first.p0), vrsrc(first.p1), off);
      // the loop issues unconditionally (straight-line load order, so each wait
      // covers exactly the loads it needs); the last unit is peeled
      for (int j = j0; j < j1 - 1; ++j) {
        consume_unit<ESZ, D>(
            u, qb, acc, m_run, l_run, logit_scale, (int64_t)j * kUnit, L, grp,
            [&] { issue_k<ESZ, D>(u, krsrc(nxt.p0), krsrc(nxt.p1), off); },
            [&] { issue_v<ESZ, D>(u, vrsrc(nxt.p0), vrsrc(nxt.p1), off); });
        nxt = unit_pages(bt_row, j + 2, last_page);
      }
      consume_unit<ESZ, D>(u, qb, acc, m_run, l_run, logit_scale, (int64_t)(j1 - 1) * kUnit, L, grp, [] {}, [] {});

      // the four lane groups hold partial sums of the same head (same max)
      l_run += xor_shuffle(l_run, 16);
      l_run += xor_shuffle(l_run, 32);
      float out_scale = 1.0f;
      if constexpr (ESZ == 1) out_scale = p.v_scale[h];
      if (col < p.G) {
        const int hq = h * p.G + col;
        // acc[j][i] = O^T[dim (4*grp + i)*NJ + j][head col]
        if (whole) {
          const float inv = out_scale / l_run;
          __bf16* orow = (__bf16*)p.out + (q_row * p.Hq + hq) * D;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t w[NJ / 2];
#pragma unroll
            for (int j = 0; j < NJ / 2; ++j) w[j] = pack_bf16x2(acc[2 * j][i] * inv, acc[2 * j + 1][i] * inv);
            __bf16* dst = orow + (4 * grp + i) * NJ;
            if constexpr (NJ == 8) *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
            else *(u32x2*)dst = u32x2{w[0], w[1]};
          }
        } else {
          const int64_t slot = ((int64_t)b + wg) * p.Hq + hq;
          float* orow = p.ws_o + slot * D;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; j += 4)
              *(f32x4*)(orow + (4 * grp + i) * NJ + j) =
                  f32x4{acc[j][i] * out_scale, acc[j + 1][i] * out_scale, acc[j + 2][i] * out_scale,
                        acc[j + 3][i] * out_scale};
          if (grp == 0) {
            p.ws_ml[2 * slot] = m_run;
            p.ws_ml[2 * slot + 1] = l_run;
          }
        }
      }
    }
  }
}

// Partition range start of workgroup w and the workgroup owning unit u, for
// U units cut into W ranges (start(w) = floor(w * U / W)).
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t U, int64_t W) { return (w * U) / W; }
__device__ __forceinline__ int64_t range_owner(int64_t u, int64_t U, int64_t W) { return ((u + 1) * W - 1) / U; }

// One wave per (query head, sequence): log-sum-exp merge of the partials of a
// sequence whose units span several workgroups:
//   M = max_w m_w,  out = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(AttnParams p) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t q_row = p.qsl[b];
  if (p.qsl[b + 1] == q_row) return;
  const int64_t cb = p.ws_cum[b], ce = p.ws_cum[b + 1], U = p.ws_cum[p.B];
  const int64_t W = p.grid_parts;
  if (ce <= cb) return;
  const int64_t wa = range_owner(cb, U, W), wz = range_owner(ce - 1, U, W);
  if (wa == wz) return;  // written directly by decode_kernel
  float M = -INFINITY;
  for (int64_t w0 = wa; w0 <= wz; w0 += 64) {
    const int64_t w = w0 + lane;
    if (w <= wz && range_start(w, U, W) < range_start(w + 1, U, W))
      M = fmaxf(M, p.ws_ml[2 * ((b + w) * p.Hq + hq)]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float l = 0.f;
  for (int64_t w = wa; w <= wz; ++w) {
    if (range_start(w, U, W) >= range_start(w + 1, U, W)) continue;  // empty range wrote nothing
    const int64_t slot = (b + w) * p.Hq + hq;
    const float f = __builtin_amdgcn_exp2f(p.ws_ml[2 * slot] - M);
    l += f * p.ws_ml[2 * slot + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += f * p.ws_o[slot * D + lane + 64 * i];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    ((__bf16*)p.out)[(q_row * p.Hq + hq) * D + lane + 64 * i] = (__bf16)(o[i] * inv);
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t decode_workspace_bytes(int64_t B, int Hq, int D) {
  const size_t slots = (size_t)(B + kDecodeMaxParts) * Hq;
  return align256((size_t)(B + 1) * sizeof(int32_t)) + align256(slots * 2 * sizeof(float)) +
         slots * D * sizeof(float);
}

void decode_workspace_carve(AttnParams& p, void* workspace) {
  char* w = (char*)workspace;
  const size_t slots = (size_t)(p.B + kDecodeMaxParts) * p.Hq;
  p.ws_cum = (int32_t*)w;
  w += align256((size_t)(p.B + 1) * sizeof(int32_t));
  p.ws_ml = (float*)w;
  w += align256(slots * 2 * sizeof(float));
  p.ws_o = (float*)w;
}

// Workgroups of the decode grid: one per CU (one 8-wave workgroup fits a CU),
// or, when the caller asks for partitions of split_tokens positions, about
// B * max_len / 2 / split_tokens of them rounded to a multiple of the CU count.
int decode_grid_parts(int64_t B, int64_t max_len, int split_tokens, int n_cu) {
  int64_t parts = n_cu;
  if (split_tokens > 0) {
    const int64_t want = (B * max_len / 2 + split_tokens - 1) / split_tokens;
    const int64_t rounds = std::max<int64_t>(1, (want + n_cu / 2) / n_cu);
    parts = rounds * n_cu;
  }
  return (int)std::min<int64_t>(parts, kDecodeMaxParts);
}

template <int ESZ, int D>
static void launch_decode_t(const AttnParams& p, hipStream_t stream) {
  const int threads = 64 * decode_waves(p.Hkv);
  hipLaunchKernelGGL((decode_kernel<ESZ, D>), dim3((unsigned)p.grid_parts), dim3(threads), 0, stream, p);
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
