// prefill.hip -- chunked causal prefill over paged KV, bf16 MFMA.
//
// What is computed: for sequence b with n_b query rows and L_b keys, query row i
// sits at position P_b + i (P_b = L_b - n_b) and attends to positions
// 0 .. P_b + i, each found at row p % 16 of page block_table[b][p / 16]
// (page "Add paged / block-table KV cache export (--features paged-cache)",
// onnxruntime/mobius #395, "How it works" step 3: opset-24 Attention with
// is_causal=1 and nonpad_kv_seqlen, the new tokens being the last ones).
// Query head hq reads KV head hq / G.
//
// Mapping onto gfx950 (FlashAttention-style online softmax):
//  * One workgroup = 4 waves = one (query tile, KV head h, sequence b).  A query
//    tile packs (token, head-of-group) pairs row = token * G + g, 256 / G tokens,
//    so the G heads sharing a KV head share every K/V tile.  Each wave owns 64
//    rows (two 32-row column blocks).
//  * Keys stream in tiles of 32 positions (2 pages).  The tile's page ids come
//    from block_table; K and V rows are copied (fp8 codes widened to bf16) into
//    LDS, double buffered, with the next tile's global loads in flight while the
//    current tile is computed.  Tiles past the last query's position are never
//    visited; masking is applied only on tiles that cross the diagonal.
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from
//    LDS, B = 16 dims x 32 query rows held in registers), so each lane owns 16
//    keys of one query row per block: the row max needs one cross-lane step.
//  * O^T = V^T . P^T with the same MFMA; the V^T operand is read from LDS with
//    ds_read_b64_tr_b16 (gfx950 transposing LDS read), P is rounded to bf16.
//  * Masking selects -inf for keys after the row's position; V rows past the
//    keys any row may see are zeroed in LDS, so stale or NaN bytes never reach
//    the output.  The fp8 k scale is folded into the logit scale, the v scale
//    into the output.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kPrefillRows = 256;  // query rows per workgroup (4 waves x 64)
constexpr int kKeyTile = 32;       // key positions per LDS tile (2 pages)

int prefill_tokens_per_tile(int G) { return kPrefillRows / G; }

size_t prefill_workspace_bytes(const AttnParams&) { return 0; }

template <int D>
struct PrefillLds {
  static constexpr int KS = D + 8;   // K row stride (elements): 272 B for D = 128
  static constexpr int VS = D + 16;  // V row stride (elements): 288 B for D = 128
  __bf16 k[2][kKeyTile * KS];
  __bf16 v[2][kKeyTile * VS];
};

// Global -> register staging of one K or V tile.  Thread t copies 16-byte
// chunks: CPR chunks per key row, 256 / CPR rows per pass.
template <int ESZ, int D>
struct Stage {
  static constexpr int CPR = D * ESZ / 16;
  static constexpr int RPP = 256 / CPR;
  static constexpr int PASSES = RPP >= kKeyTile ? 1 : kKeyTile / RPP;
  u32x4 x[PASSES];
};

template <int ESZ, int D>
__device__ __forceinline__ void stage_load(Stage<ESZ, D>& st, const char* __restrict__ base,
                                           const int64_t* __restrict__ bt_row, int64_t key0,
                                           int64_t last_page, int64_t page_stride, int64_t row_stride,
                                           int tid) {
  using S = Stage<ESZ, D>;
  const int chunk = tid % S::CPR;
  const int r0 = tid / S::CPR;
#pragma unroll
  for (int i = 0; i < S::PASSES; ++i) {
    const int r = r0 + S::RPP * i;
    if (r < kKeyTile) {
      const int64_t key = key0 + r;
      int64_t lp = key >> 4;
      lp = lp > last_page ? last_page : lp;
      const int64_t page = bt_row[lp];
      st.x[i] = *(const u32x4*)(base + page * page_stride + (key & 15) * row_stride + chunk * 16);
    }
  }
}

// Register -> LDS row (row stride RS elements); fp8 codes are widened to bf16.
// Rows of keys >= zero_from are stored as zeros (used for V: masked keys must
// not meet P = 0 with a NaN).
template <int ESZ, int D, int RS>
__device__ __forceinline__ void stage_store(const Stage<ESZ, D>& st, __bf16* __restrict__ lds,
                                            int64_t key0, int64_t zero_from, int tid) {
  using S = Stage<ESZ, D>;
  const int chunk = tid % S::CPR;
  const int r0 = tid / S::CPR;
#pragma unroll
  for (int i = 0; i < S::PASSES; ++i) {
    const int r = r0 + S::RPP * i;
    if (r < kKeyTile) {
      const bool live = key0 + r < zero_from;
      if constexpr (ESZ == 2) {
        u32x4 v = st.x[i];
        if (!live) v = u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)(lds + r * RS + chunk * 8) = v;
      } else {
        const u32x2 c0 = fp8x4_to_bf16x4(st.x[i].x), c1 = fp8x4_to_bf16x4(st.x[i].y);
        const u32x2 c2 = fp8x4_to_bf16x4(st.x[i].z), c3 = fp8x4_to_bf16x4(st.x[i].w);
        u32x4 a = {c0.x, c0.y, c1.x, c1.y};
        u32x4 b = {c2.x, c2.y, c3.x, c3.y};
        if (!live) {
          a = u32x4{0u, 0u, 0u, 0u};
          b = a;
        }
        *(u32x4*)(lds + r * RS + chunk * 16) = a;
        *(u32x4*)(lds + r * RS + chunk * 16 + 8) = b;
      }
    }
  }
}

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<__bf16*>(p)));
}

template <int ESZ, int D>
__global__ __launch_bounds__(256, 1) void prefill_kernel(AttnParams p) {
  constexpr int NKS = D / 16;  // score MFMA k-steps
  constexpr int NDB = D / 32;  // output dim blocks
  using Lds = PrefillLds<D>;
  __shared__ Lds lds;

  const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;  // later (longer) tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int tpt = kPrefillRows / G;  // tokens per tile

  const int64_t q0 = p.qsl[b];
  const int64_t n = p.qsl[b + 1] - q0;
  const int64_t L = p.seq_lens[b];
  const int64_t P = L - n;
  const int64_t tok0 = (int64_t)tile * tpt;
  if (tok0 >= n) return;
  const int64_t tok_end = min(tok0 + (int64_t)tpt, n);
  const int64_t kv_len = P + tok_end;  // keys any row of this tile can see
  const int n_tiles = (int)((kv_len + kKeyTile - 1) / kKeyTile);
  const int64_t last_page = ((L + 15) >> 4) - 1;

  // ---- query operand (B of S^T = K Q^T): lane l holds row (l & 31) of block nb,
  // dims [16*ks + 8*(l >> 5), +8)
  const int qcol = lane & 31, qgrp = lane >> 5;
  bf16x8 qb[2][NKS];
  int64_t qpos[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = wave * 64 + nb * 32 + qcol;
    const int64_t tok = tok0 + r / G;
    const bool live = r < tpt * G && tok < tok_end;
    qpos[nb] = live ? P + tok : P + tok_end - 1;
    const __bf16* qrow = (const __bf16*)p.q + ((q0 + (live ? tok : 0)) * p.Hq + h * G + r % G) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (live) x = *(const u32x4*)(qrow + 16 * ks + 8 * qgrp);
      qb[nb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  float logit_scale = p.scale * kLog2e;
  if constexpr (ESZ == 1) logit_scale *= p.k_scale[h];
  const int64_t min_qpos = P + tok0;

  const int64_t row_stride = (int64_t)p.Hkv * D * ESZ;
  const int64_t page_stride = row_stride * kPageSize;
  const char* kbase = (const char*)p.key_pool + (int64_t)h * D * ESZ;
  const char* vbase = (const char*)p.value_pool + (int64_t)h * D * ESZ;
  const int64_t* bt_row = p.block_table + (int64_t)b * p.max_blocks;

  f32x16 acc[NDB][2];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][nb][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  {
    Stage<ESZ, D> sk0, sv0;
    stage_load<ESZ, D>(sk0, kbase, bt_row, 0, last_page, page_stride, row_stride, tid);
    stage_load<ESZ, D>(sv0, vbase, bt_row, 0, last_page, page_stride, row_stride, tid);
    stage_store<ESZ, D, Lds::KS>(sk0, lds.k[0], 0, INT64_MAX, tid);
    stage_store<ESZ, D, Lds::VS>(sv0, lds.v[0], 0, kv_len, tid);
  }
  __syncthreads();

  const int blk16 = lane >> 4, li = lane & 15;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t key0 = (int64_t)t * kKeyTile;
    const bool more = t + 1 < n_tiles;
    Stage<ESZ, D> stg;
    if (more) stage_load<ESZ, D>(stg, kbase, bt_row, key0 + kKeyTile, last_page, page_stride, row_stride, tid);

    const __bf16* sk = lds.k[buf];
    const __bf16* sv = lds.v[buf];

    // ---- scores: s[nb] = S^T[key 8*(i/4) + 4*qgrp + i%4][row nb*32 + qcol]
    f32x16 s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 ka = *(const bf16x8*)(sk + qcol * Lds::KS + 16 * ks + 8 * qgrp);
      s[0] = mfma32(ka, qb[0][ks], s[0]);
      s[1] = mfma32(ka, qb[1][ks], s[1]);
    }
    if (more) {
      stage_store<ESZ, D, Lds::KS>(stg, lds.k[buf ^ 1], key0 + kKeyTile, INT64_MAX, tid);
      stage_load<ESZ, D>(stg, vbase, bt_row, key0 + kKeyTile, last_page, page_stride, row_stride, tid);
    }

    // ---- online softmax per query row: the lane owns row qcol of each nb and
    // keys 8*(i/4) + 4*qgrp + i%4; the other 16 keys are in lane ^ 32
    const bool diag = key0 + kKeyTile - 1 > min_qpos;
    bf16x8 pb[2][2];  // [half][nb]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = s[nb][i] * logit_scale;
      if (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t kp = key0 + 8 * (i >> 2) + 4 * qgrp + (i & 3);
          x[i] = kp <= qpos[nb] ? x[i] : -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, xor_shuffle(mx, 32));
      const float m_new = fmaxf(m_run[nb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_new);
      m_run[nb] = m_new;
      float sum = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = __builtin_amdgcn_exp2f(x[8 * hh + 2 * q] - m_new);
          const float c = __builtin_amdgcn_exp2f(x[8 * hh + 2 * q + 1] - m_new);
          sum += a + c;
          w[q] = pack_bf16x2(a, c);
        }
        pb[hh][nb] = __builtin_bit_cast(bf16x8, w);
      }
      l_run[nb] = l_run[nb] * alpha + sum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int d = 0; d < NDB; ++d) acc[d][nb] *= alpha;
      }
    }

    // ---- O^T += V^T P^T; V^T fragments come from transposing LDS reads
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int dim = d * 32 + 16 * (blk16 & 1) + 4 * (li & 3);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int krow = 16 * hh + 4 * qgrp + (li >> 2);
        const s16x4 lo = lds_read_tr16(sv + krow * Lds::VS + dim);
        const s16x4 hi = lds_read_tr16(sv + (krow + 8) * Lds::VS + dim);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[d][0] = mfma32(va, pb[hh][0], acc[d][0]);
        acc[d][1] = mfma32(va, pb[hh][1], acc[d][1]);
      }
    }

    if (more) stage_store<ESZ, D, Lds::VS>(stg, lds.v[buf ^ 1], key0 + kKeyTile, kv_len, tid);
    __syncthreads();
  }

  // ---- normalise and write: acc[d][nb][i] = O^T[dim d*32 + 8*(i/4) + 4*qgrp + i%4][row]
  float out_scale = 1.0f;
  if constexpr (ESZ == 1) out_scale = p.v_scale[h];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l = l_run[nb] + xor_shuffle(l_run[nb], 32);
    const int r = wave * 64 + nb * 32 + qcol;
    const int64_t tok = tok0 + r / G;
    if (r >= tpt * G || tok >= tok_end) continue;
    const float inv = out_scale / l;
    __bf16* orow = (__bf16*)p.out + ((q0 + tok) * p.Hq + h * G + r % G) * D;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 w;
        w.x = pack_bf16x2(acc[d][nb][4 * i4 + 0] * inv, acc[d][nb][4 * i4 + 1] * inv);
        w.y = pack_bf16x2(acc[d][nb][4 * i4 + 2] * inv, acc[d][nb][4 * i4 + 3] * inv);
        *(u32x2*)(orow + d * 32 + 8 * i4 + 4 * qgrp) = w;
      }
  }
}

hipError_t launch_prefill(const AttnParams& p, hipStream_t stream) {
  if (p.T == 0 || p.B == 0) return hipSuccess;
  const int tpt = prefill_tokens_per_tile(p.G);
  const int n_tiles = (p.max_query_len + tpt - 1) / tpt;
  dim3 grid((unsigned)n_tiles, (unsigned)p.Hkv, (unsigned)p.B);
  const bool fp8 = p.kv_type == KV_FP8;
  if (p.D == 128) {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<1, 128>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((prefill_kernel<2, 128>), grid, dim3(256), 0, stream, p);
  } else {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<1, 64>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((prefill_kernel<2, 64>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
