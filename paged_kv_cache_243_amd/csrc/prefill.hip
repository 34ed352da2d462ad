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
//  * Work item = (query tile, KV head).  A query tile packs (token,
//    head-of-group) pairs, row = token * G + g, 256 / G tokens, so the G heads
//    that share a KV head share every K/V tile.  One workgroup of 4 waves per
//    item, each wave owning 64 rows (two 32-row column blocks).  A
//    one-workgroup plan kernel lists the tiles longest first (their KV length
//    sets their cost), so in-order dispatch fills the CUs greedily.
//  * Keys stream in tiles of 32 positions (2 pages).  bf16 tiles go from
//    global memory straight into LDS (buffer_load ... lds); every page gets a
//    buffer descriptor whose range ends at the sequence's last valid row, so
//    rows at positions >= seq_lens read as zeros whatever the pool holds.  fp8
//    tiles go through registers and are widened to bf16 (rows past seq_lens
//    stored as zeros).  Tiles are double buffered with one barrier per tile.
//    LDS rows keep their 16-byte chunks XOR-swizzled so the operand reads
//    below are spread over the banks.
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from
//    LDS, B = 16 dims x 32 query rows held in registers): each lane owns 16 keys
//    of one query row, so a row max needs one cross-lane step.
//  * O^T = V^T . P^T with the same MFMA; V^T comes out of LDS through
//    ds_read_b64_tr_b16 (gfx950's transposing LDS read); P is rounded to bf16
//    and the softmax denominator sums the same rounded values.
//  * Software pipeline: the scores of tile t+1 are computed in the same
//    iteration as the softmax and PV of tile t, so MFMA and VALU work of
//    different tiles can overlap within a wave.
//  * Online softmax in the exp2 domain with a lazy reference max: the
//    accumulator is rescaled only when a row's max grows by more than 2^8 over
//    the reference, so the common step is one FMA and one exp2 per score.  The
//    scale's sign is moved into q (an exact sign flip), so the running max can
//    be taken over raw scores.
//  * Masking selects -inf for keys after the row's position, only on tiles
//    that cross the diagonal.  The fp8 k scale joins the logit scale, the v
//    scale the output normalisation.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kPrefillRows = 256;      // query rows per workgroup (4 waves x 64)
constexpr int kKeyTile = 32;           // key positions per LDS tile (2 pages)
constexpr int kPlanSortMax = 2048;     // items the plan kernel orders by length
constexpr float kLazyRescale = 8.0f;   // log2 growth of a row max tolerated before rescaling
constexpr int kRawBufferWord3 = 0x00020000;

int prefill_tokens_per_tile(int G) { return kPrefillRows / G; }

int64_t prefill_max_items(int64_t T, int64_t B, int G) {
  const int tpt = prefill_tokens_per_tile(G);
  return (T + tpt - 1) / tpt + B;
}

size_t prefill_workspace_bytes(const AttnParams& p) {
  return (size_t)(prefill_max_items(p.T, p.B, p.G) + 1) * sizeof(uint32_t);
}

// ---------------------------------------------------------------------------
// Plan: enumerate the (sequence, query tile) items, longest KV range first.
// ws_plan[0] = item count, ws_plan[1 + rank] = b << 16 | tile.  Above
// kPlanSortMax items the natural order is kept.

__global__ __launch_bounds__(1024) void prefill_plan_kernel(AttnParams p) {
  __shared__ uint32_t s_item[kPlanSortMax];
  __shared__ int32_t s_work[kPlanSortMax];
  __shared__ int32_t s_scan[1024];
  const int tid = threadIdx.x;
  const int B = (int)p.B;
  const int tpt = kPrefillRows / p.G;
  const int per = (B + 1023) / 1024;  // sequences per thread
  int32_t mine = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < B) mine += (int32_t)((p.qsl[b + 1] - p.qsl[b] + tpt - 1) / tpt);
  }
  s_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int32_t v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int32_t total = s_scan[1023];
  const bool sort = total <= kPlanSortMax;
  int32_t at = tid ? s_scan[tid - 1] : 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b >= B) continue;
    const int64_t n = p.qsl[b + 1] - p.qsl[b];
    const int64_t P = p.seq_lens[b] - n;
    const int nt = (int)((n + tpt - 1) / tpt);
    for (int t = 0; t < nt; ++t, ++at) {
      const uint32_t item = ((uint32_t)b << 16) | (uint32_t)t;
      if (sort) {
        const int64_t w = P + min((int64_t)(t + 1) * tpt, n);
        s_item[at] = item;
        s_work[at] = (int32_t)min(w, (int64_t)INT32_MAX);
      } else {
        p.ws_plan[1 + at] = (int32_t)item;
      }
    }
  }
  if (tid == 0) p.ws_plan[0] = total;
  if (!sort) return;
  __syncthreads();
  // rank = items that go first: longer, or as long and listed earlier
  for (int i = tid; i < total; i += 1024) {
    const int32_t w = s_work[i];
    int32_t rank = 0;
    for (int j = 0; j < total; ++j) rank += (s_work[j] > w) | ((s_work[j] == w) & (j < i));
    p.ws_plan[1 + rank] = (int32_t)s_item[i];
  }
}

// ---------------------------------------------------------------------------

template <int D>
struct TileLayout {
  static constexpr int NC = D / 8;  // 16-byte chunks per bf16 row
  // K: the rows one 32-lane operand read touches land on distinct chunk slots
  __device__ static int swz_k(int row) { return (row / (16 / NC)) % NC; }
  // V: the 4 rows x 2 chunks one transposing read touches land on distinct slots
  __device__ static int swz_v(int row) { return (2 * ((row / (16 / NC)) % 4)) % NC; }
};

typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const char* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  // the range is uniform too, but may be computed on the VALU (e.g. a clamp):
  // without the readfirstlane the descriptor would not be known to be scalar
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kRawBufferWord3);
}

struct TileSrc {
  const char* kbase;   // pool + h * D * ESZ
  const char* vbase;
  const_i64_ptr bt;    // block_table row of the sequence
  int L;               // positions the sequence holds (< 2^31)
  int last_page;       // logical index of its last page
  int64_t page_stride;
  uint32_t row_stride;
};

// bf16: one 32-row tile (K or V) straight into LDS.  One load moves 1 KiB per
// wave (lane l -> LDS bytes 16 l after the wave's base), i.e. 1024 / (2 D)
// whole rows of one page, so the swizzle is applied by choosing which global
// chunk each lane fetches.  Tiles before position 0 or past seq_lens read as
// zeros and touch no memory.
template <int D>
struct Dma {
  static constexpr int ROWS = 1024 / (2 * D);        // rows per load: 4 (D = 128) or 8 (D = 64)
  static constexpr int LOADS = kKeyTile / ROWS / 4;  // loads per wave and tile
};

template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(const TileSrc& c, __bf16* tile, int t, int wave, int lane) {
  using TL = TileLayout<D>;
  using M = Dma<D>;
  const char* base = IS_V ? c.vbase : c.kbase;
#pragma unroll
  for (int i = 0; i < M::LOADS; ++i) {
    const int first_row = (wave * M::LOADS + i) * M::ROWS;
    const int lp = (t * kKeyTile + first_row) >> 4;  // logical page (negative before position 0)
    const int lpc = lp < 0 ? 0 : (lp < c.last_page ? lp : c.last_page);
    const int64_t page = c.bt[lpc];
    int valid = c.L - (lp << 4);  // rows of this page the sequence holds
    valid = lp < 0 || valid < 0 ? 0 : (valid > kPageSize ? kPageSize : valid);
    const __amdgpu_buffer_rsrc_t r = uniform_rsrc(base + page * c.page_stride, (uint32_t)valid * c.row_stride);
    const int row = first_row + lane / TL::NC;
    const int logical = (lane % TL::NC) ^ (IS_V ? TL::swz_v(row) : TL::swz_k(row));
    const uint32_t voff = (uint32_t)(row & 15) * c.row_stride + 16u * logical;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(tile + first_row * D), 16, (int)voff, 0, 0, 0);
  }
}

// fp8: a tile's codes through registers (one 16-byte chunk per thread and pass)
template <int D>
struct Fp8Tile {
  static constexpr int CPR = D / 16;     // 16-byte code chunks per row
  static constexpr int RPP = 256 / CPR;  // rows per pass
  static constexpr int PASSES = RPP >= kKeyTile ? 1 : kKeyTile / RPP;
  u32x4 x[PASSES];
};

template <int D>
__device__ __forceinline__ void fp8_fetch(Fp8Tile<D>& st, const TileSrc& c, const char* base, int t, int tid) {
  using S = Fp8Tile<D>;
  const int chunk = tid % S::CPR, r0 = tid / S::CPR;
#pragma unroll
  for (int i = 0; i < S::PASSES; ++i) {
    const int r = r0 + S::RPP * i;
    if (r < kKeyTile) {
      const int key = t * kKeyTile + r;
      const int lp = key >> 4;
      const int64_t page = c.bt[lp < c.last_page ? lp : c.last_page];
      st.x[i] = *(const u32x4*)(base + page * c.page_stride + (key & 15) * c.row_stride + 16 * chunk);
    }
  }
}

template <int D, bool IS_V>
__device__ __forceinline__ void fp8_store(const Fp8Tile<D>& st, __bf16* tile, int t, int64_t L, int tid) {
  using S = Fp8Tile<D>;
  using TL = TileLayout<D>;
  const int chunk = tid % S::CPR, r0 = tid / S::CPR;
#pragma unroll
  for (int i = 0; i < S::PASSES; ++i) {
    const int r = r0 + S::RPP * i;
    if (r < kKeyTile) {
      const bool live = (int64_t)t * kKeyTile + r < L;
      const u32x2 c0 = fp8x4_to_bf16x4(st.x[i].x), c1 = fp8x4_to_bf16x4(st.x[i].y);
      const u32x2 c2 = fp8x4_to_bf16x4(st.x[i].z), c3 = fp8x4_to_bf16x4(st.x[i].w);
      const u32x4 z = {0u, 0u, 0u, 0u};
      const int sw = IS_V ? TL::swz_v(r) : TL::swz_k(r);
      *(u32x4*)(tile + r * D + 8 * ((2 * chunk) ^ sw)) = live ? u32x4{c0.x, c0.y, c1.x, c1.y} : z;
      *(u32x4*)(tile + r * D + 8 * ((2 * chunk + 1) ^ sw)) = live ? u32x4{c2.x, c2.y, c3.x, c3.y} : z;
    }
  }
}

__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
}

// max of a value over lanes l and l ^ 32
__device__ __forceinline__ float max_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  const unsigned lo = r[0], hi = r[1];  // (bit_cast of a subscripted vector element reads element 0)
  return __builtin_fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

__device__ __forceinline__ float sum_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  const unsigned lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Workgroup barrier for LDS hand-off.  __syncthreads() would also wait for
// every outstanding global load, i.e. drain the tile fetches in flight; here
// only this wave's LDS accesses are completed (lgkmcnt(0)) and the fetched
// tiles are waited for explicitly with wait_vmem.  The "memory" clobber keeps
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding, N < 16)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Iteration t of the main loop (after a barrier) fetches K(t + NS) and
// V(t + NS - 2), computes the scores of tile t+1, adds P(t-1) V(t-1) into the
// output and turns the scores of tile t into P(t).  Tile j lives in ring slot
// j % NS; at the top of iteration t the ring holds K(t+1) and V(t-1), and no
// wave still reads the slots the iteration overwrites.
template <int ESZ, int D>
__global__ __launch_bounds__(256, 1) void prefill_kernel(AttnParams p) {
  constexpr int NKS = D / 16;              // score MFMA k-steps
  constexpr int NDB = D / 32;              // output dim blocks
  constexpr int NS = ESZ == 2 ? 4 : 2;     // K/V ring depth
  constexpr int TB = kKeyTile * D * 2;     // bytes per LDS tile
  using TL = TileLayout<D>;
  // one LDS variable per ring slot: the compiler tells LDS-DMA targets apart
  // by variable, so reads of one slot never wait for fetches into another
  __shared__ __attribute__((aligned(16))) char sk0[TB], sk1[TB], sk2[NS > 2 ? TB : 16], sk3[NS > 2 ? TB : 16];
  __shared__ __attribute__((aligned(16))) char sv0[TB], sv1[TB], sv2[NS > 2 ? TB : 16], sv3[NS > 2 ? TB : 16];
  char* const sk[4] = {sk0, sk1, sk2, sk3};
  char* const sv[4] = {sv0, sv1, sv2, sv3};

  const int rank = (int)(blockIdx.x / (unsigned)p.Hkv), h = (int)(blockIdx.x % (unsigned)p.Hkv);
  if (rank >= p.ws_plan[0]) return;
  const uint32_t item = (uint32_t)p.ws_plan[1 + rank];
  const int b = (int)(item >> 16), tile = (int)(item & 0xFFFF);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int tpt = kPrefillRows / G;  // tokens per tile

  const int64_t q0 = p.qsl[b];
  const int64_t n = p.qsl[b + 1] - q0;
  const int64_t L = p.seq_lens[b];
  const int64_t P = L - n;
  const int64_t tok0 = (int64_t)tile * tpt;
  const int64_t tok_end = min(tok0 + (int64_t)tpt, n);
  const int64_t kv_len = P + tok_end;  // keys some row of this tile sees
  const int n_tiles = (int)((kv_len + kKeyTile - 1) / kKeyTile);
  const int64_t first_pos = P + tok0;  // position of the tile's first token
  // first key tile that reaches past first_pos, i.e. needs the causal mask
  const int t_diag = first_pos >= kKeyTile - 1 ? (int)((first_pos - (kKeyTile - 1)) / kKeyTile) + 1 : 0;

  TileSrc c;
  c.row_stride = (uint32_t)p.Hkv * D * ESZ;
  c.page_stride = (int64_t)c.row_stride * kPageSize;
  c.kbase = (const char*)p.key_pool + (int64_t)h * D * ESZ;
  c.vbase = (const char*)p.value_pool + (int64_t)h * D * ESZ;
  c.bt = (const_i64_ptr)(p.block_table + (int64_t)b * p.max_blocks);
  c.L = (int)L;
  c.last_page = (int)((L + 15) >> 4) - 1;

  // logit scale in log2 units; its sign goes into q so maxima are taken on raw scores
  float cs = p.scale * kLog2e;
  if constexpr (ESZ == 1) cs *= p.k_scale[h];
  const uint32_t qflip = cs < 0.f ? 0x80008000u : 0u;
  cs = fabsf(cs);
  // a zero scale means uniform weights; any tiny scale gives the same exp2 values
  cs = fmaxf(cs, 1e-30f);

  // ---- query operand (B of S^T = K Q^T): lane l holds row (l & 31) of block
  // nb, dims [16 ks + 8 (l >> 5), +8)
  const int qcol = lane & 31, qgrp = lane >> 5;
  bf16x8 qb[2][NKS];
  int32_t qrel[2];  // row position - first_pos - 4 qgrp
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = wave * 64 + nb * 32 + qcol;
    const int64_t tok = tok0 + r / G;
    const bool live = r < tpt * G && tok < tok_end;
    qrel[nb] = (int32_t)((live ? tok : tok_end - 1) - tok0) - 4 * qgrp;
    const __bf16* qrow = (const __bf16*)p.q + ((q0 + (live ? tok : 0)) * p.Hq + h * G + r % G) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (live) x = *(const u32x4*)(qrow + 16 * ks + 8 * qgrp) ^ qflip;
      // park the query operand in AGPRs (MFMA reads A/B from either file),
      // leaving the VGPRs to the softmax and the LDS operand pipeline
      u32x4 xa;
      asm("" : "=a"(xa) : "0"(x));
      qb[nb][ks] = __builtin_bit_cast(bf16x8, xa);
    }
  }

  // ---- per-lane LDS byte offsets inside a tile.  The XOR swizzles act on
  // bits the k-step (K) or dim-block (V) index enters by XOR, so one base per
  // lane serves every read.
  // K operand (A of S^T): row qcol, chunk 2 ks + qgrp -> kA ^ (32 ks)
  const uint32_t kA = (uint32_t)qcol * 2 * D + 16u * (uint32_t)(qgrp ^ TL::swz_k(qcol));
  // V^T operand: row 16 hh + 8 hi + 4 qgrp + (li >> 2), dims 32 d + 16 (blk16 & 1) + 4 (li & 3)
  //   -> (vA ^ (64 d)) + (16 hh + 8 hi) * 2 D
  const int blk16 = lane >> 4, li = lane & 15;
  const int vrow = 4 * qgrp + (li >> 2);
  const uint32_t vA = (uint32_t)vrow * 2 * D +
                      16u * (uint32_t)((2 * (blk16 & 1) + ((li & 3) >> 1)) ^ TL::swz_v(vrow)) + 8u * (li & 1);

  f32x16 acc[NDB][2];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][nb][i] = 0.f;
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference max, log2 units
  float l_run[2] = {0.f, 0.f};

  // S^T of the K tile in ring slot `slot`: s[nb][i] = score of key 8 (i / 4) +
  // 4 qgrp + i % 4 of the tile and query row 32 nb + qcol
  auto scores = [&](int slot, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const char* k = sk[slot];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 ka = *(const bf16x8*)(k + (kA ^ (32u * ks)));
      s[0] = mfma32(ka, qb[0][ks], s[0]);
      s[1] = mfma32(ka, qb[1][ks], s[1]);
    }
  };

  // O^T += V^T P^T for the V tile in ring slot `slot`
  auto pv = [&](int slot, const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    const char* v = sv[slot];
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const char* vd = v + (vA ^ (64u * d));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x4 lo = lds_read_tr16(vd + (16 * hh) * 2 * D);
        const s16x4 hi = lds_read_tr16(vd + (16 * hh + 8) * 2 * D);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[d][0] = mfma32(va, pb[hh][0], acc[d][0]);
        acc[d][1] = mfma32(va, pb[hh][1], acc[d][1]);
      }
    }
  };

  // P(t) from the raw scores of tile t.  The reference max moves only when a
  // row's max passes it by more than kLazyRescale; alpha is the factor the
  // accumulator then needs (1 otherwise).  Returns whether any row moved.
  auto softmax = [&](auto mask_c, int t, f32x16 (&s)[2], bf16x8 (&pb)[2][2], float (&alpha)[2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    bool moved = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if constexpr (MASK) {
        const int32_t lim = (int32_t)(first_pos - (int64_t)t * kKeyTile) + qrel[nb];
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = 8 * (i >> 2) + (i & 3) > lim ? -INFINITY : s[nb][i];
      }
      float mx = __builtin_fmaxf(s[nb][0], s[nb][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[nb][i], s[nb][i + 1]));
      mx = max_pair(mx) * cs;
      const bool need = mx > m_ref[nb] + kLazyRescale;
      alpha[nb] = need ? __builtin_amdgcn_exp2f(m_ref[nb] - mx) : 1.0f;
      m_ref[nb] = need ? mx : m_ref[nb];
      moved |= need;
      float l = l_run[nb] * alpha[nb];
      const float neg_m = -m_ref[nb];
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][8 * hh + 2 * q], cs, neg_m));
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][8 * hh + 2 * q + 1], cs, neg_m));
          const uint32_t pk = pack_bf16x2(a, e);
          w[q] = pk;
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, l, false);
        }
        pb[hh][nb] = __builtin_bit_cast(bf16x8, w);
      }
      l_run[nb] = l;
    }
    return __builtin_amdgcn_ballot_w64(moved) != 0;
  };

  // (one 16-register block at a time, so the rare rescale needs few
  // temporaries beside the live state)
  auto rescale = [&](const float (&alpha)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        acc[d][nb] *= alpha[nb];
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // ---- tile fetches.  Tile j lives in ring slot j % NS.  bf16: DMA issued
  // for "virtual iteration" u (K(u+NS-1), V(u+NS-2)), so that every iteration
  // issues the same number of loads and vmcnt(LOADS_AFTER) leaves exactly the
  // tiles the next iteration needs in flight.
  constexpr int LOADS_AFTER = (NS - 2) * 2 * Dma<D>::LOADS;
  auto issue = [&](int u, int slot_k, int slot_v) __attribute__((always_inline)) {
    dma_tile<D, false>(c, (__bf16*)sk[slot_k], u + NS - 1, wave, lane);
    dma_tile<D, true>(c, (__bf16*)sv[slot_v], u + NS - 2, wave, lane);
  };
  Fp8Tile<D> fk, fv;  // fp8 staging: iteration t fetches K(t+1) and V(t)
  auto store8 = [&](int t, int slot_k, int slot_v) __attribute__((always_inline)) {
    fp8_store<D, false>(fk, (__bf16*)sk[slot_k], t + 1, L, tid);
    fp8_store<D, true>(fv, (__bf16*)sv[slot_v], t, L, tid);
  };

  // ---- prologue: K(0) resident, V(-1) zero (the PV of the first iteration
  // multiplies it by P(-1) = 0), later tiles in flight
  bf16x8 pb_prev[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) pb_prev[hh][nb] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  if constexpr (ESZ == 2) {
#pragma unroll
    for (int u = 1 - NS; u < 0; ++u) issue(u, (u + NS - 1) % NS, (u + 2 * NS - 2) % NS);
    wait_vmem<LOADS_AFTER + Dma<D>::LOADS>();  // K(0) landed (V(-1) is a zero fill)
  } else {
    fp8_fetch<D>(fk, c, c.kbase, 0, tid);
    fp8_store<D, false>(fk, (__bf16*)sk[0], 0, L, tid);
    for (int i = tid; i < TB / 16; i += 256) ((u32x4*)sv[NS - 1])[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // Iteration t, ring position R = t % NS (a compile-time constant at every
  // call, so every LDS access names its slot variable): scores of tile t,
  // then P(t-1) V(t-1) into the output while the softmax of tile t runs, so
  // MFMA and VALU work overlap.  At the top (after the barrier) K(t) and
  // V(t-1) are resident and no wave still reads K(t-1) or V(t-2), whose slots
  // the iteration's fetches overwrite.  Tiles past the sequence are zero
  // filled and fully masked, so iterations past the last tile add nothing.
  auto iteration = [&](auto mask_c, auto r_c, int t) __attribute__((always_inline)) {
    constexpr int R = decltype(r_c)::value;
    barrier_lds();
    if constexpr (ESZ == 2) {
      issue(t, (R + NS - 1) % NS, (R + NS - 2) % NS);
    } else {
      fp8_fetch<D>(fk, c, c.kbase, t + 1, tid);
      fp8_fetch<D>(fv, c, c.vbase, t, tid);
    }
    f32x16 s[2];
    scores(R, s);
    pv((R + NS - 1) % NS, pb_prev);
    float alpha[2];
    bf16x8 pb[2][2];
    if (softmax(mask_c, t, s, pb, alpha)) rescale(alpha);
    if constexpr (ESZ == 2) wait_vmem<LOADS_AFTER>();
    else store8(t, (R + 1) % NS, R);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      pb_prev[0][nb] = pb[0][nb];
      pb_prev[1][nb] = pb[1][nb];
    }
  };
  auto group = [&](auto mask_c, int t) __attribute__((always_inline)) {
    iteration(mask_c, std::integral_constant<int, 0>{}, t);
    iteration(mask_c, std::integral_constant<int, 1>{}, t + 1);
    if constexpr (NS == 4) {
      iteration(mask_c, std::integral_constant<int, 2>{}, t + 2);
      iteration(mask_c, std::integral_constant<int, 3>{}, t + 3);
    }
  };

  // iterations 0 .. n_tiles (the last one only adds P(n_tiles - 1) V), in
  // groups of NS: unmasked up to the group holding the diagonal, masked after
  const int t_split = t_diag / NS * NS;
  int t = 0;
  for (; t < t_split; t += NS) group(std::false_type{}, t);
  for (; t <= n_tiles; t += NS) group(std::true_type{}, t);
  if constexpr (ESZ == 2) wait_vmem<0>();  // no tile write may land after the workgroup ends

  // acc[d][nb][i] = O^T[dim 32 d + 8 (i / 4) + 4 qgrp + i % 4][row]
  float out_scale = 1.0f;
  if constexpr (ESZ == 1) out_scale = p.v_scale[h];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l = sum_pair(l_run[nb]);
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
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  const dim3 grid((unsigned)(prefill_max_items(p.T, p.B, p.G) * p.Hkv));
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
