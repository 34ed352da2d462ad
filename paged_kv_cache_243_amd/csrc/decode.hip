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
//    heads.  It is cut into equal contiguous ranges (parts), so every CU
//    streams the same number of bytes whatever the length mix.  A part is run
//    by a group of waves, wave k of the group handling KV head k (or heads k,
//    k + 8, ...): the waves of a group read the same pages together, so HBM
//    sees whole rows of all heads.  A workgroup holds up to 8 waves: one group
//    when there are 8 or more KV heads, else several groups side by side (8 of
//    one wave each for a single KV head, as on a tensor-parallel shard), so
//    every CU keeps 8 waves' loads in flight.  The grid has one workgroup per
//    CU, or a multiple of the CU count when the caller asks for smaller
//    partitions.  Every K/V byte of (b, h) is read from HBM once and serves
//    all G query heads.
//  * Page ids come from block_table through wave-uniform scalar loads, two
//    units ahead.  K and V are read with buffer loads (page base in a scalar
//    descriptor, 32-bit lane offsets), non-temporal, in whole-row runs: each
//    load instruction covers complete 2*D-byte (bf16) rows of the head, the
//    access shape HBM streams fastest.  Each unit is then staged into per-wave
//    LDS tiles (chunk-swizzled against bank conflicts; fp8 widened to bf16 on
//    the way) and the next unit's loads are issued at once into the freed
//    registers, so every load has a whole unit of compute to land.
//  * Scores use v_mfma_f32_16x16x32_bf16 as S^T = K . Q^T: A = 16 keys (one
//    page) x 32 dims from the K tile, B = the G query heads (zero-padded to 16
//    columns).  Lane l then holds 4 keys of one head, so the softmax max needs
//    two cross-lane steps and the sum none until the end.
//  * P.V uses the same MFMA as O^T = V^T . P^T; the V^T operand comes straight
//    out of the V tile with ds_read_b64_tr_b16 (gfx950's transposing LDS read).
//  * fp8 E4M3FN codes are widened to bf16 (exact) with v_cvt_scalef32_pk_bf16_fp8;
//    the per-head k scale is folded into the logit scale and the v scale into
//    the output.
//  * Masking selects -inf for positions >= seq_lens (never multiplies by zero),
//    and V rows of masked positions are stored as zeros in the tile, so stale
//    or NaN bytes in unused slots cannot reach the output.
//  * A segment (the part of one sequence inside a workgroup's range) that is a
//    whole sequence writes its normalised output directly; otherwise it writes
//    its unnormalised O with (m, l) to a partial slot and merge_kernel combines
//    a sequence's partials:
//        M = max_w m_w,  out = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "decode_device.h"
#include "kernels.h"
namespace pkv {

using namespace dk;

template <int ESZ, int D>
__global__ __launch_bounds__(512) void decode_kernel(AttnParams p) {
  __shared__ DecodeLds<D> lds;
  decode_body<ESZ, D>(p, lds, blockIdx.x, gridDim.x);
}

// Log-sum-exp merge of the partials of a sequence whose units span several
// parts (and, with a shared prefix, of the prefix chunks' partials):
//   M = max_w m_w,  out = sum_w 2^(m_w - M) u_w R_w / sum_w 2^(m_w - M) l_w,
// where partial w's unnormalised row O_w is stored as R_w = O_w / u_w in fp16.
// A workgroup serves nh query heads of one sequence (threadIdx.y), with nw
// waves per head (1 .. kMergeWaves, by the partials a sequence has; nw * nh
// <= kMergeWaves).  Wave k of a head takes the chunks k, k + nw, ... of
// CHUNK consecutive partials; wave 0 also the prefix chunks', whose loads go out
// before the metadata's, as their slots do not depend on it.  Every (m, l)
// and O load of a chunk is issued before any of them is used, so the merge
// of a head costs two memory round trips (metadata, then partials) when its
// partials fit one chunk.  With several waves per head their (m, l, O) are
// then combined through LDS in wave order.  Several heads per workgroup (up to
// kMergeGroupWaves waves in all) keep the CUs' wave slots full when there are
// many rows of few partials.
constexpr int kMergeWaves = 16;
constexpr int kMergeGroupWaves = 4;

// merge waves per head for a grid of `parts` parts over B sequences: one per
// 8 partials a sequence holds on average, at most 4 up to 8 such chunks and at
// most kMergeWaves beyond (the 8-way head shard of the long fp8 decode, 129
// partials per row: 16 waves took its step from 81 to 78 us against 4; the
// long fp8 decode itself, 33 per row, measured no better with 5 than with 4)
static int merge_waves(int parts, int64_t B) {
  const int64_t per_seq = parts / std::max<int64_t>(B, 1) + 1;
  const int64_t chunks = (per_seq + 7) / 8;
  return (int)std::min<int64_t>(chunks > 8 ? kMergeWaves : kMergeGroupWaves, chunks);
}

// partials a merge wave loads together: as many as a sequence holds on
// average, rounded up to 2, 4 or 8 (fewer registers and loads when most rows
// have one or two decode partials, as with a shared prefix)
static int merge_chunk(int parts, int64_t B) {
  const int64_t per_seq = parts / std::max<int64_t>(B, 1) + 1;
  return per_seq <= 2 ? 2 : per_seq <= 4 ? 4 : 8;
}

// heads per merge workgroup: the most that divides Hq within kMergeGroupWaves waves
static int merge_heads(int Hq, int nw) {
  for (int nh = kMergeGroupWaves / nw; nh > 1; nh /= 2)
    if (Hq % nh == 0) return nh;
  return 1;
}

// rows (query heads of one sequence) a merge wave takes: 2 when the rows
// outnumber one round of the chip's wave slots and every head has one wave,
// so the waves fit one round; else 1
constexpr int64_t kMergeOneRoundRows = 8192;
static int merge_rows_per_wave(int64_t B, int Hq, int nw) {
  return nw == 1 && B * Hq > kMergeOneRoundRows && Hq % 2 == 0 ? 2 : 1;
}

// RPW rows per wave (consecutive query heads; only with one wave per head),
// CHUNK decode partials per load round, and the prefix chunks' partials held
// for at most PMAX chunks (1 when there is at most one).  Each row's
// arithmetic is the same whatever RPW and PMAX are.  A lane owns elements
// lane * PER .. + PER - 1 of each row.  A partial (decode or prefix) is its
// unnormalised row in fp16 times a power of two, with (max, sum, the power's
// inverse) in fp32.
template <int D, int CHUNK, int RPW, int PMAX>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(AttnParams p) {
  constexpr int PER = D / 64;
  __shared__ float s_ml[kMergeWaves][2];
  __shared__ float s_o[kMergeWaves][D];
  const int nw = blockDim.x >> 6;
  const int hq0 = (blockIdx.x * blockDim.y + threadIdx.y) * RPW, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_slot = threadIdx.y * nw;  // this head's LDS slots: row_slot .. row_slot + nw - 1
  const bool prefix = p.prefix_len > 0;
  // the prefix chunks' partials, loaded first
  f32x4 mlc[RPW][PMAX];
  float oc[RPW][PMAX][PER];
  if (prefix && wave == 0) {
    const f32x4* pml = (const f32x4*)p.ws_pre_ml;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < PMAX; ++c) {
        if (c < p.prefix_chunks) {
          const int64_t slot = ((int64_t)c * p.B + b) * p.Hq + hq0 + r;
          mlc[r][c] = pml[slot];
          load_f16_elems<PER>(p.ws_pre_o + slot * D, lane, oc[r][c]);
        }
      }
  }
  // every index this workgroup needs, loaded together
  const int64_t q_row = p.qsl[b], q_end = p.qsl[b + 1];
  const int32_t cb = p.ws_cum[b], ce = p.ws_cum[b + 1], units = p.ws_cum[p.B];
  const bool has_units = ce > cb && units > 0;
  if (q_end == q_row || (!prefix && !has_units)) return;
  const Partition part(units, p.grid_parts);
  int32_t wa = 0, wz = -1;  // parts holding the sequence's units (none: wz < wa)
  if (has_units) {
    wa = part.owner(cb);
    wz = part.owner(ce - 1);
  }
  if (!prefix && wa == wz) return;  // written directly by decode_kernel
  const f32x4* ml = (const f32x4*)p.ws_ml;
  float M[RPW], l[RPW], o[RPW][PER];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    M[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[r][i] = 0.f;
  }
  if (prefix && wave == 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int c = 0; c < PMAX; ++c)
        if (c < p.prefix_chunks) M[r] = fmaxf(M[r], mlc[r][c][0]);
#pragma unroll
      for (int c = 0; c < PMAX; ++c) {
        if (c < p.prefix_chunks) {
          const float f = __builtin_amdgcn_exp2f(mlc[r][c][0] - M[r]);
          l[r] += f * mlc[r][c][1];
          const float g = f * mlc[r][c][2];
#pragma unroll
          for (int i = 0; i < PER; ++i) o[r][i] += g * oc[r][c][i];
        }
      }
    }
  }
  for (int32_t w0 = wa + wave * CHUNK; w0 <= wz; w0 += nw * CHUNK) {
    f32x4 mlw[RPW][CHUNK];
    float ow[RPW][CHUNK][PER];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        const int32_t w = min(w0 + c, wz);
        const int64_t slot = ((int64_t)b + w) * p.Hq + hq0 + r;
        mlw[r][c] = ml[slot];
        load_f16_elems<PER>(p.ws_o + slot * D, lane, ow[r][c]);
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float Mc = M[r];
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        // slots past wz repeat wz, and empty ranges wrote nothing: weight 0
        const bool live = w0 + c <= wz && !part.empty(w0 + c);
        mlw[r][c][0] = live ? mlw[r][c][0] : -INFINITY;
        Mc = fmaxf(Mc, mlw[r][c][0]);
      }
      // rescale what earlier chunks summed (nothing yet: M = Mc = -inf would give NaN)
      const float alpha = M[r] == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M[r] - Mc);
      l[r] *= alpha;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[r][i] *= alpha;
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        const float f = __builtin_amdgcn_exp2f(mlw[r][c][0] - Mc);
        l[r] += f * mlw[r][c][1];
        const float g = f * mlw[r][c][2];
#pragma unroll
        for (int i = 0; i < PER; ++i) o[r][i] += g * ow[r][c][i];
      }
      M[r] = Mc;
    }
  }
  if constexpr (RPW == 1) {
    if (nw > 1) {
      // combine the head's waves' (M, l, O); a wave that took no partial has
      // M = -inf, l = 0, O = 0 and weight 0 (wave 0 holds at least one live
      // partial)
      if (lane == 0) {
        s_ml[row_slot + wave][0] = M[0];
        s_ml[row_slot + wave][1] = l[0];
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) s_o[row_slot + wave][lane * PER + i] = o[0][i];
      __syncthreads();
      if (wave != 0) return;
      float Mt = -INFINITY;
      for (int k = 0; k < nw; ++k) Mt = fmaxf(Mt, s_ml[row_slot + k][0]);
      float lt = 0.f, ot[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) ot[i] = 0.f;
      for (int k = 0; k < nw; ++k) {
        const float m_k = s_ml[row_slot + k][0];
        const float f = m_k == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_k - Mt);
        lt += f * s_ml[row_slot + k][1];
#pragma unroll
        for (int i = 0; i < PER; ++i) ot[i] += f * s_o[row_slot + k][lane * PER + i];
      }
      l[0] = lt;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[0][i] = ot[i];
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float inv = 1.0f / l[r];
    __bf16* orow = (__bf16*)p.out + (q_row * p.Hq + hq0 + r) * D;
    if constexpr (PER == 2)
      ((uint32_t*)orow)[lane] = pack_bf16x2(o[r][0] * inv, o[r][1] * inv);
    else
      orow[lane] = (__bf16)(o[r][0] * inv);
  }
}

template <int D, int CHUNK>
static void launch_merge_c(const AttnParams& p, int rpw, int pmax, dim3 grid, dim3 block, hipStream_t stream) {
  if (rpw == 2) {
    if (pmax == 1) hipLaunchKernelGGL((merge_kernel<D, CHUNK, 2, 1>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<D, CHUNK, 2, kMaxPrefixChunks>), grid, block, 0, stream, p);
  } else {
    if (pmax == 1) hipLaunchKernelGGL((merge_kernel<D, CHUNK, 1, 1>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<D, CHUNK, 1, kMaxPrefixChunks>), grid, block, 0, stream, p);
  }
}

template <int D>
static void launch_merge(const AttnParams& p, hipStream_t stream) {
  const int nw = merge_waves(p.grid_parts, p.B);
  const int rpw = merge_rows_per_wave(p.B, p.Hq, nw);
  const int nh = merge_heads(p.Hq / rpw, nw);
  const int pmax = p.prefix_len > 0 && p.prefix_chunks > 1 ? kMaxPrefixChunks : 1;
  const dim3 grid((unsigned)(p.Hq / (rpw * nh)), (unsigned)p.B), block(64 * nw, nh);
  switch (merge_chunk(p.grid_parts, p.B)) {
    case 2: launch_merge_c<D, 2>(p, rpw, pmax, grid, block, stream); break;
    case 4: launch_merge_c<D, 4>(p, rpw, pmax, grid, block, stream); break;
    default: launch_merge_c<D, 8>(p, rpw, pmax, grid, block, stream); break;
  }
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// partial slots: one per (sequence + part, query head); a segment of sequence
// b in part w writes slot b + w < B + parts
size_t decode_workspace_bytes(int64_t B, int Hq, int D, int parts) {
  const size_t slots = (size_t)(B + parts) * Hq;
  return align256((size_t)(B + 1) * sizeof(int32_t)) + align256(slots * 4 * sizeof(float)) +
         align256(slots * D * sizeof(_Float16));
}

void decode_workspace_carve(AttnParams& p, void* workspace, int parts) {
  char* w = (char*)workspace;
  const size_t slots = (size_t)(p.B + parts) * p.Hq;
  p.ws_cum = (int32_t*)w;
  w += align256((size_t)(p.B + 1) * sizeof(int32_t));
  p.ws_ml = (float*)w;
  w += align256(slots * 4 * sizeof(float));
  p.ws_o = (_Float16*)w;
}

// Workgroups of the decode grid: one per CU (one 8-wave workgroup fits a CU),
// or, when the caller asks for partitions of split_tokens positions, about
// B * max_len / 2 / split_tokens of them rounded to a multiple of the CU count.
int decode_grid_parts(int64_t B, int64_t max_len, int split_tokens, int n_cu, int Hkv) {
  int64_t parts = n_cu;
  if (split_tokens > 0) {
    const int64_t want = (B * max_len / 2 + split_tokens - 1) / split_tokens;
    const int64_t rounds = std::max<int64_t>(1, (want + n_cu / 2) / n_cu);
    parts = rounds * n_cu;
  }
  const int R = decode_groups(Hkv);
  return (int)(std::min<int64_t>(parts * R, kDecodeMaxParts) / R * R);
}

// More parts than one round of workgroups (a caller's small split_tokens) run
// as consecutive parts of one stream per group rather than as further rounds
// of workgroups, so that a group can hold a part's partial in registers until
// its stream ends (fp8 pools): with rounds of workgroups, the first round's
// partials were stored while the second round streamed.  The long fp8 decode
// at 2048-position parts (two parts per group) takes 7 % less time.
int decode_rounds(int grid_parts, int n_cu, int Hkv) {
  const int per_round = decode_groups(Hkv) * n_cu;
  return n_cu > 0 && grid_parts > per_round && grid_parts % per_round == 0 ? grid_parts / per_round : 1;
}

// Whether the decode launch for p can carry the write of n_new rows of
// row_bytes each: a workgroup holds kCopyRegs chunks of 16 bytes per thread
// and pool, and takes every gridDim.x-th row.
bool decode_can_fuse_write(const AttnParams& p, int64_t n_new, int64_t row_bytes) {
  if (row_bytes <= 0 || row_bytes % 16 != 0) return false;
  const int R = decode_groups(p.Hkv);
  const int64_t wgs = decode_workgroups(p), threads = 64 * decode_waves(p.Hkv) * R;
  if (wgs <= 0) return false;
  const int64_t rows_per_wg = (n_new + wgs - 1) / wgs;
  return rows_per_wg * (row_bytes / 16) <= kCopyRegs * threads;
}

template <int ESZ, int D>
static void launch_decode_t(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev) {
  const int R = decode_groups(p.Hkv);
  const int threads = 64 * decode_waves(p.Hkv) * R;
  if (ev.begin) (void)hipEventRecord(ev.begin, stream);
  if (p.prefix_len > 0)
    (void)launch_shared_prefix_decode(p, stream);
  else
    hipLaunchKernelGGL((decode_kernel<ESZ, D>), dim3((unsigned)decode_workgroups(p)), dim3(threads), 0, stream, p);
  if (ev.end) (void)hipEventRecord(ev.end, stream);
  launch_merge<D>(p, stream);
}

hipError_t launch_decode(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev) {
  if (p.B == 0) return hipSuccess;
  const bool fp8 = p.kv_type == KV_FP8;
  if (p.D == 128) {
    if (fp8) launch_decode_t<1, 128>(p, stream, ev); else launch_decode_t<2, 128>(p, stream, ev);
  } else {
    if (fp8) launch_decode_t<1, 64>(p, stream, ev); else launch_decode_t<2, 64>(p, stream, ev);
  }
  return hipGetLastError();
}

}  // namespace pkv
