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
//    that share a KV head share every K/V tile.  One workgroup of 8 waves per
//    item (two per SIMD), each wave owning 32 rows.  A one-workgroup plan
//    kernel lists the items longest first (their KV length sets their cost),
//    so in-order dispatch fills the CUs greedily.  When the items make fewer
//    than two rounds of workgroups (few KV heads per GPU), every item's keys
//    are cut into chunks that run as items of their own, each writing (m, l,
//    O) partials per row, which prefill_split_merge_kernel combines.
//  * Keys stream in tiles of 32 positions (2 pages) through LDS rings (K and
//    V).  bf16 tiles go from global memory straight into LDS (buffer_load ...
//    lds), 6 slots deep, two K and two V tiles behind each barrier; every page
//    gets a buffer descriptor whose range ends at the sequence's last valid
//    row, so rows at positions >= seq_lens read as zeros whatever the pool
//    holds.  fp8 codes take the same DMA path into code slots (half the
//    bytes), two sets of four tiles, and every wave widens its share of them
//    exactly to bf16 into 4-slot rings one hand-off later, with the same
//    barrier cadence.  LDS rows keep their 16-byte chunks XOR-swizzled so the
//    operand reads below are spread over the banks.
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from
//    LDS, B = 16 dims x 32 query rows held in registers): each lane owns 16 keys
//    of one query row, so a row max needs one cross-lane step.
//  * O^T = V^T . P^T with the same MFMA; V^T comes out of LDS through
//    ds_read_b64_tr_b16 (gfx950's transposing LDS read); P is rounded to bf16
//    and the softmax denominator sums the same rounded values.
//  * Software pipeline: the scores of tile t+1 and the PV product of tile t-1
//    are computed in the same iteration as the softmax of tile t, so MFMA and
//    VALU work of different tiles can overlap within a wave.
//  * Online softmax in the exp2 domain with a lazy reference max: P is taken
//    against a reference that moves (and the accumulator is rescaled) only
//    when some P of a tile could exceed 2^8, which the tile's own row sums
//    reveal, so the common step is one FMA, one exp2, half a conversion and
//    half a dot2 per score and no max.  The scale's sign is moved into q (an
//    exact sign flip), so maxima can be taken over raw scores.
//  * Masking selects -inf for keys after the row's position, only on tiles
//    that cross the diagonal.  The fp8 k scale joins the logit scale, the v
//    scale the output normalisation.
#include <math.h>

#include <algorithm>
#include <numeric>

#include <type_traits>

#include "common.h"
#include "decode_device.h"
#include "kernels.h"

namespace pkv {

constexpr int kPrefillRows = 256;      // query rows per workgroup
#ifndef PKV_PREFILL_ROW_BLOCKS
#define PKV_PREFILL_ROW_BLOCKS 1
#endif
constexpr int kPrefillRowBlocks = PKV_PREFILL_ROW_BLOCKS;  // 32-row blocks per wave (8 / NB waves)
constexpr int kKeyTile = 32;           // key positions per LDS tile (2 pages)
constexpr int kPlanSortMax = 2048;     // items the plan kernel orders by length
constexpr int kValuPerMfma = 4;        // softmax VALU instructions placed after each MFMA
constexpr float kLazyBound = 256.0f;   // largest P (= exp2 of 8) a tile may hold before the reference moves
constexpr int kRawBufferWord3 = 0x00020000;

int prefill_tokens_per_tile(int G) { return kPrefillRows / G; }

int64_t prefill_max_items(int64_t T, int64_t B, int G) {
  const int tpt = prefill_tokens_per_tile(G);
  return (T + tpt - 1) / tpt + B;
}

// Key split.  When the items (query tiles x KV heads) make fewer than
// kSplitRounds rounds of workgroups on kSplitCUs CUs, as with one to four KV
// heads per GPU, the longest item alone would set the kernel's time; the keys
// are then cut into chunks so that about kSplitRounds rounds of workgroups
// fill the CUs (if every sequence had max_blocks pages), each chunk at least
// kSplitMinKeys keys.  The CU count is MI355X's, fixed so that
// the workspace size does not depend on the device.
constexpr int kSplitCUs = 256;
constexpr int kSplitRounds = 2;
constexpr int kSplitMinKeys = 512;

void prefill_split_plan(AttnParams& p) {
  const int64_t tiles = prefill_max_items(p.T, p.B, p.G);
  p.plan_tiles_cap = tiles;
  p.split_keys = 0;
  p.split_max_chunks = 1;
  const int64_t wgs = tiles * p.Hkv;
  const int64_t max_kv = p.max_blocks * kPageSize;
  if (wgs >= kSplitRounds * kSplitCUs || max_kv <= 2 * kSplitMinKeys) return;
  const int64_t per_item = (kSplitRounds * kSplitCUs + wgs - 1) / wgs;
  int64_t c = std::max<int64_t>((max_kv + per_item - 1) / per_item, kSplitMinKeys);
  c = (c + kKeyTile - 1) / kKeyTile * kKeyTile;
  p.split_keys = (int)c;
  p.split_max_chunks = (int)((max_kv + c - 1) / c);
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

static size_t plan_bytes(const AttnParams& p) {
  const int64_t items = p.plan_tiles_cap * p.split_max_chunks;
  return align256((size_t)(2 + 2 * items + p.plan_tiles_cap) * sizeof(int32_t));
}

static size_t split_rows(const AttnParams& p) {
  return p.split_keys > 0 ? (size_t)p.plan_tiles_cap * p.Hkv * p.split_max_chunks * kPrefillRows : 0;
}

size_t prefill_workspace_bytes(const AttnParams& p) {
  const size_t rows = split_rows(p);
  return plan_bytes(p) + (rows ? align256(rows * 4 * sizeof(float)) + rows * p.D * sizeof(_Float16) : 0);
}

void prefill_workspace_carve(AttnParams& p, void* workspace) {
  char* w = (char*)workspace;
  p.ws_plan = (int32_t*)w;
  const size_t rows = split_rows(p);
  p.ws_split_ml = rows ? (float*)(w + plan_bytes(p)) : nullptr;
  p.ws_split_o = rows ? (_Float16*)(w + plan_bytes(p) + align256(rows * 4 * sizeof(float))) : nullptr;
}

// chunks of an item whose rows see kv keys (1 without the key split); kv <
// max_blocks * 16 < 2^31, so the division is a 32-bit one
__device__ __forceinline__ int item_chunks(const AttnParams& p, int64_t kv) {
  if (p.split_keys == 0) return 1;
  const uint32_t c = ((uint32_t)kv + (uint32_t)p.split_keys - 1u) / (uint32_t)p.split_keys;
  return (int)min(c, (uint32_t)p.split_max_chunks);
}

// ---------------------------------------------------------------------------
// Plan: enumerate the (sequence, query tile, key chunk) items, longest key
// range first, and the (sequence, query tile) pairs.  Layout in ws_plan:
//   [0] item count, [1] tile count,
//   [2 + 2 rank] = b << 16 | tile, [3 + 2 rank] = tile index * split_max_chunks + chunk,
//   [2 + 2 items_cap + tile index] = b << 16 | tile.
// Above kPlanSortMax items the natural order is kept.
//
// The natural order is by sequence, then query tile, then chunk.  Each thread
// first counts the tiles and items of its run of `per` sequences; block-wide
// prefix sums of both give every run's first tile and item.  Then one thread
// per tile finds its run by binary search over the tile sums, and the tile's
// first item by adding the chunk counts of the run's tiles before it, and
// lists the tile's items.  The ranking counts, for each item, the items with
// a larger 64-bit key (key range << 32 | ~index: longer first, then listed
// earlier).

// tiles and chunks of sequence b: the query tiles' key ranges P + min((t + 1)
// tpt, n), t < ceil(n / tpt)
struct PlanSeq {
  int64_t n, P;
  int nt;
};

__device__ __forceinline__ PlanSeq plan_seq(const AttnParams& p, int b, int tpt) {
  PlanSeq q;
  q.n = p.qsl[b + 1] - p.qsl[b];
  q.P = p.seq_lens[b] - q.n;
  q.nt = (int)((q.n + tpt - 1) / tpt);
  return q;
}

__device__ __forceinline__ int64_t plan_tile_kv(const PlanSeq& q, int t, int tpt) {
  return q.P + min((int64_t)(t + 1) * tpt, q.n);
}

// items of tiles 0 .. t - 1 of a sequence
__device__ __forceinline__ int32_t plan_items_before(const AttnParams& p, const PlanSeq& q, int t, int tpt) {
  if (p.split_keys == 0) return t;
  int32_t a = 0;
  for (int u = 0; u < t; ++u) a += item_chunks(p, plan_tile_kv(q, u, tpt));
  return a;
}

// Inclusive sums of a and c over the 1024 threads (lane shuffles within each
// wave, then the 16 wave totals through LDS: one barrier); returns them in
// a and c, and the totals.
__device__ __forceinline__ void plan_scan2(int32_t& a, int32_t& c, int32_t (&s_wave)[2][16], int32_t& total_a,
                                           int32_t& total_c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t ya = __shfl_up(a, off, 64), yc = __shfl_up(c, off, 64);
    if (lane >= off) {
      a += ya;
      c += yc;
    }
  }
  if (lane == 63) {
    s_wave[0][wave] = a;
    s_wave[1][wave] = c;
  }
  __syncthreads();
  total_a = 0;
  total_c = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int32_t ta = s_wave[0][w], tc = s_wave[1][w];
    a += w < wave ? ta : 0;
    c += w < wave ? tc : 0;
    total_a += ta;
    total_c += tc;
  }
}

__global__ __launch_bounds__(1024) void prefill_plan_kernel(AttnParams p) {
  __shared__ uint32_t s_item[kPlanSortMax];
  __shared__ int32_t s_tc[kPlanSortMax];
  __shared__ uint64_t s_key[kPlanSortMax];
  __shared__ int32_t s_scan[1024];   // items (inclusive sums over threads' runs)
  __shared__ int32_t s_tscan[1024];  // tiles
  __shared__ int32_t s_wave[2][16];
  const int tid = threadIdx.x;
  const int B = (int)p.B;
  const int tpt = kPrefillRows / p.G;
  const int MC = p.split_max_chunks;
  const int64_t tiles_cap = p.plan_tiles_cap, items_cap = tiles_cap * MC;
  int32_t* const list = p.ws_plan + 2;
  int32_t* const tiles = p.ws_plan + 2 + 2 * items_cap;
  const int per = (B + 1023) / 1024;  // sequences per thread
  int32_t mine = 0, mine_t = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b >= B) continue;
    const PlanSeq q = plan_seq(p, b, tpt);
    mine_t += q.nt;
    mine += plan_items_before(p, q, q.nt, tpt);
  }
  int32_t all_items, all_tiles;
  plan_scan2(mine, mine_t, s_wave, all_items, all_tiles);
  s_scan[tid] = mine;
  s_tscan[tid] = mine_t;
  __syncthreads();
  const int32_t total = (int32_t)min((int64_t)all_items, items_cap);
  const bool sort = total <= kPlanSortMax;
  for (int g = tid; g < all_tiles; g += 1024) {
    // the run holding tile g: the first thread whose inclusive tile sum exceeds g
    int lo = 0, hi = 1023;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_tscan[mid] > g) hi = mid;
      else lo = mid + 1;
    }
    int32_t local = g - (lo ? s_tscan[lo - 1] : 0);
    int32_t at = lo ? s_scan[lo - 1] : 0;
    int b = lo * per;
    PlanSeq q = plan_seq(p, b, tpt);
    while (local >= q.nt) {  // earlier sequences of the run
      local -= q.nt;
      at += plan_items_before(p, q, q.nt, tpt);
      q = plan_seq(p, ++b, tpt);
    }
    const int t = local;
    at += plan_items_before(p, q, t, tpt);
    const uint32_t item = ((uint32_t)b << 16) | (uint32_t)t;
    if (g < tiles_cap) tiles[g] = (int32_t)item;
    const int64_t kv = plan_tile_kv(q, t, tpt);
    const int nch = item_chunks(p, kv);
    for (int ch = 0; ch < nch; ++ch, ++at) {
      if (at >= total) break;
      const int32_t tc = g * MC + ch;
      if (sort) {
        const int64_t w = nch == 1 ? kv : (ch + 1 < nch ? (int64_t)p.split_keys : kv - (int64_t)ch * p.split_keys);
        s_item[at] = item;
        s_tc[at] = tc;
        s_key[at] = ((uint64_t)min(w, (int64_t)INT32_MAX) << 32) | (uint32_t)~at;
      } else {
        list[2 * at] = (int32_t)item;
        list[2 * at + 1] = tc;
      }
    }
  }
  if (tid == 0) {
    p.ws_plan[0] = total;
    p.ws_plan[1] = (int32_t)min((int64_t)all_tiles, tiles_cap);
  }
  if (!sort) return;
  __syncthreads();
  // rank = items with a larger key: longer, or as long and listed earlier
  for (int i = tid; i < total; i += 1024) {
    const uint64_t k = s_key[i];
    int32_t r0 = 0, r1 = 0;
    int j = 0;
    for (; j + 2 <= total; j += 2) {
      r0 += s_key[j] > k;
      r1 += s_key[j + 1] > k;
    }
    if (j < total) r0 += s_key[j] > k;
    const int rank = r0 + r1;
    list[2 * rank] = (int32_t)s_item[i];
    list[2 * rank + 1] = s_tc[i];
  }
}

// ---------------------------------------------------------------------------

template <int D>
struct TileLayout {
  static constexpr int NC = D / 8;  // 16-byte chunks per bf16 row
  // K: the rows one 32-lane operand read touches land on distinct chunk slots
  __device__ static int swz_k(int row) { return (row / (16 / NC)) % NC; }
  // V: one pass of a transposing read serves 32 lanes (256 bytes, all 64 banks)
  // and touches 4 rows x 4 chunks; each row's 4 chunks go to their own group
  // of 4 chunk slots, so the pass hits every bank once
  __device__ static int swz_v(int row) { return (4 * ((row / (16 / NC)) % (NC / 4))) % NC; }
};

typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;

// Raw buffer descriptor (stride 0, `bytes` addressable bytes) in scalar
// registers.  The range is uniform too, but may be computed on the VALU (e.g. a
// clamp): without the readfirstlane it would not be known to be scalar.
__device__ __forceinline__ u32x4 uniform_rsrc(const char* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)v);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) & 0xFFFFu;  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = kRawBufferWord3;
  return r;
}

// One 16-byte-per-lane global -> LDS transfer: lane l's 16 bytes at voff go to
// LDS byte lds + 16 l (buffer_load_dwordx4 ... lds, LDS base in M0).  Written
// as inline assembly so that the compiler does not track the transfer: its
// own tracking of LDS-DMA targets is coarse enough to put waits for unrelated
// transfers before operand reads of ring slots that have long landed.  The
// kernel orders these transfers itself (wait_vmem, then a barrier).  The
// s_nop covers the wait states between writing M0 (and, just before, the
// descriptor's scalar registers from the VALU) and the load reading them.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
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
// chunk each lane fetches.  The D / 16 loads of a tile are spread over the
// waves (waves past the last load fetch nothing).  Tiles before position 0 or
// past seq_lens read as zeros and touch no memory.
template <int D, int WAVES>
struct Dma {
  static constexpr int ROWS = 1024 / (2 * D);                 // rows per load: 4 (D = 128) or 8 (D = 64)
  static constexpr int TOTAL = kKeyTile / ROWS;               // loads per tile
  static constexpr int LOADS = TOTAL >= WAVES ? TOTAL / WAVES : 1;  // loads per active wave
  static constexpr int ACTIVE = TOTAL / LOADS;                // waves that load
  static constexpr int WROWS = LOADS * ROWS;                  // rows per active wave (within one page)
  static_assert(TOTAL % LOADS == 0 && kPageSize % WROWS == 0, "a wave's rows share a page");
};

// Page holding this wave's rows of tile t; tiles outside the sequence map to a
// page it owns, whose rows the descriptor range then excludes.
template <int D, int WAVES>
__device__ __forceinline__ int64_t wave_page(const TileSrc& c, int t, int wave) {
  const int lp = (t * kKeyTile + wave * Dma<D, WAVES>::WROWS) >> 4;
  const int lpc = lp < 0 ? 0 : (lp < c.last_page ? lp : c.last_page);
  return c.bt[lpc];
}

template <int D, int WAVES, bool IS_V>
__device__ __forceinline__ void dma_tile(const TileSrc& c, __bf16* tile, int t, int64_t page, int wave, int lane) {
  using TL = TileLayout<D>;
  using M = Dma<D, WAVES>;
  if (wave >= M::ACTIVE) return;
  const char* base = IS_V ? c.vbase : c.kbase;
  const int lp = (t * kKeyTile + wave * M::WROWS) >> 4;  // logical page (negative before position 0)
  int valid = c.L - (lp << 4);  // rows of this page the sequence holds
  valid = lp < 0 || valid < 0 ? 0 : (valid > kPageSize ? kPageSize : valid);
  const u32x4 r = uniform_rsrc(base + page * c.page_stride, (uint32_t)valid * c.row_stride);
#pragma unroll
  for (int i = 0; i < M::LOADS; ++i) {
    const int first_row = (wave * M::LOADS + i) * M::ROWS;
    const int row = first_row + lane / TL::NC;
    const int logical = (lane % TL::NC) ^ (IS_V ? TL::swz_v(row) : TL::swz_k(row));
    const uint32_t voff = (uint32_t)(row & 15) * c.row_stride + 16u * logical;
    dma16(r, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)(tile + first_row * D), voff);
  }
}

// fp8: a tile's codes (32 rows x D bytes) go straight into an LDS code slot.
// One load moves 1 KiB per wave (lane l -> LDS bytes 16 l after the wave's
// base), i.e. 1024 / D whole rows of one page; the codes keep the pool's row
// layout.  A hand-off fetches 4 tiles (two K, two V), its loads spread over
// the waves.  Rows past seq_lens read as zeros and touch no memory.
template <int D, int WAVES>
struct Dma8 {
  static constexpr int ROWS = 1024 / D;               // rows per load: 8 (D = 128) or 16 (D = 64)
  static constexpr int PER_TILE = kKeyTile / ROWS;    // loads per tile: 4 or 2
  static constexpr int PER_HANDOFF = 4 * PER_TILE;    // loads per hand-off: 16 or 8
  static constexpr int LOADS = PER_HANDOFF / WAVES;   // per wave
  static_assert(PER_HANDOFF % WAVES == 0 && kPageSize % ROWS == 0, "a load's rows share a page");
};

// Page holding rows part * ROWS .. of tile t (clamped into the sequence, as wave_page).
template <int D, int WAVES>
__device__ __forceinline__ int64_t page8(const TileSrc& c, int t, int part) {
  const int lp = (t * kKeyTile + part * Dma8<D, WAVES>::ROWS) >> 4;
  const int lpc = lp < 0 ? 0 : (lp < c.last_page ? lp : c.last_page);
  return c.bt[lpc];
}

template <int D, int WAVES>
__device__ __forceinline__ void dma8_rows(const TileSrc& c, const char* base, char* ctile, int t, int part,
                                          int64_t page, int lane) {
  using M = Dma8<D, WAVES>;
  constexpr int CPR = D / 16;  // 16-byte chunks per code row
  const int r0 = part * M::ROWS;
  const int lp = (t * kKeyTile + r0) >> 4;  // logical page (negative before position 0)
  int valid = c.L - (lp << 4);
  valid = lp < 0 || valid < 0 ? 0 : (valid > kPageSize ? kPageSize : valid);
  const u32x4 r = uniform_rsrc(base + page * c.page_stride, (uint32_t)valid * c.row_stride);
  const int row = r0 + lane / CPR;
  const uint32_t voff = (uint32_t)(row & 15) * c.row_stride + 16u * (lane % CPR);
  dma16(r, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ctile + r0 * D), voff);
}

// Widen one 16-code chunk (row r, chunk k of a code tile) into the bf16 tile
// at `dst`, laid out and swizzled as the bf16 tiles the DMA path fills (exact:
// every E4M3FN value is a bf16 value).
template <int D>
__device__ __forceinline__ void widen_chunk(const char* codes, char* dst, bool is_v, int r, int k) {
  using TL = TileLayout<D>;
  const u32x4 x = *(const u32x4*)(codes + r * D + 16 * k);
  const u32x2 c0 = fp8x4_to_bf16x4(x.x), c1 = fp8x4_to_bf16x4(x.y);
  const u32x2 c2 = fp8x4_to_bf16x4(x.z), c3 = fp8x4_to_bf16x4(x.w);
  const int sw = is_v ? TL::swz_v(r) : TL::swz_k(r);
  *(u32x4*)(dst + r * 2 * D + 16 * ((2 * k) ^ sw)) = u32x4{c0.x, c0.y, c1.x, c1.y};
  *(u32x4*)(dst + r * 2 * D + 16 * ((2 * k + 1) ^ sw)) = u32x4{c2.x, c2.y, c3.x, c3.y};
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

// PREFIX: the shared-prefix form of decode (see shared_prefix_decode_kernel).  An
// item is then (group of decode sequences, chunk of the shared prefix): its
// rows are the query rows of tpt consecutive sequences, its keys the chunk's
// positions of the prefix pages every block_table row starts with, and it
// writes an unnormalised partial (m, l, O) per row instead of the output.
// LDS of one prefill workgroup: the bf16 K and V rings and (fp8 pools) the
// code slots
template <int ESZ, int D>
struct PrefillLds {
  static constexpr int NS = ESZ == 2 ? 6 : 4;
  static constexpr int TB = kKeyTile * D * 2;
  alignas(16) char sk[NS][TB];
  alignas(16) char sv[NS][TB];
  alignas(16) char sc[ESZ == 1 ? 2 : 1][4][ESZ == 1 ? kKeyTile * D : 16];
};

// One work item, run by workgroup `block`: item rank0 + block / Hkv of KV
// head block % Hkv (prefill_kernel: rank0 = 0; the shared-prefix kernel's
// prefix workgroups run the PREFIX form for rank0 = 0, prefix_wgs / Hkv, ...).
template <int ESZ, int D, int NB, bool PREFIX>
__device__ __forceinline__ void prefill_item(const AttnParams& p, PrefillLds<ESZ, D>& lds, const unsigned block,
                                             const int rank0) {
  constexpr int WAVES = 8 / NB;            // 32 NB query rows per wave, 256 per workgroup
  constexpr int THREADS = 64 * WAVES;
  constexpr int NKS = D / 16;              // score MFMA k-steps
  constexpr int NDB = D / 32;              // output dim blocks
  // K/V ring depth: bf16 tiles arrive by DMA two at a time, one workgroup
  // barrier per two tiles, 6 slots deep; fp8 codes arrive by DMA into code
  // slots (two sets of four tiles) and are widened into 4-slot bf16 rings one
  // hand-off later, with the same barrier cadence
  constexpr int NS = ESZ == 2 ? 6 : 4;
  constexpr int TB = kKeyTile * D * 2;     // bytes per LDS tile
  using TL = TileLayout<D>;
  auto& sk = lds.sk;
  auto& sv = lds.sv;
  auto& sc = lds.sc;

  const int rank = rank0 + (int)(block / (unsigned)p.Hkv);
  const int h = (int)(block % (unsigned)p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int tpt = kPrefillRows / G;  // tokens per tile (PREFIX: sequences per item)

  // b: the sequence (PREFIX: the item's first sequence); tokens tok0 ..
  // tok_end - 1 of it are the tile's (PREFIX: sequences b + tok), sitting at
  // positions first_pos + (tok - tok0) (PREFIX: all at the chunk's last
  // position, so that every key of the chunk and none past it is visible)
  int b, chunk = 0;
  int64_t q0, n, L, P, tok0, tok_end;
  // key split: this item runs keys k0 .. k1 - 1 of the tile (all of them
  // unless the tile's keys are cut into n_chunks chunks); gtile = the tile's
  // index in the plan
  int64_t k0 = 0, k1 = 0;
  int n_chunks = 1, gtile = 0;
  if constexpr (PREFIX) {
    if (rank >= p.prefix_tiles * p.prefix_chunks) return;
    const int tile = rank / p.prefix_chunks;
    chunk = rank - tile * p.prefix_chunks;
    b = tile * tpt;
    q0 = 0;
    tok0 = 0;
    tok_end = min((int64_t)tpt, p.B - b);
    const int64_t c0 = (int64_t)chunk * p.prefix_chunk_len;
    L = min((int64_t)p.prefix_chunk_len, p.prefix_len - c0);  // the chunk's keys
    n = 0;
    P = L - 1;
  } else {
    if (rank >= p.ws_plan[0]) return;
    const uint32_t item = (uint32_t)p.ws_plan[2 + 2 * rank];
    const int32_t tc = p.ws_plan[3 + 2 * rank];
    b = (int)(item >> 16);
    const int tile = (int)(item & 0xFFFF);
    q0 = p.qsl[b];
    n = p.qsl[b + 1] - q0;
    L = p.seq_lens[b];
    P = L - n;
    tok0 = (int64_t)tile * tpt;
    tok_end = min(tok0 + (int64_t)tpt, n);
    gtile = tc / p.split_max_chunks;
    chunk = tc - gtile * p.split_max_chunks;
    const int64_t kv_all = P + tok_end;
    n_chunks = item_chunks(p, kv_all);
    k0 = (int64_t)chunk * p.split_keys;
    k1 = chunk + 1 < n_chunks ? k0 + p.split_keys : kv_all;
  }
  // keys some row of this item sees, counted from k0 (chunks before the last
  // end on a tile boundary, so no key past k1 enters a tile)
  const int64_t kv_len = PREFIX ? L : k1 - k0;
  const int n_tiles = (int)((kv_len + kKeyTile - 1) / kKeyTile);
  const int64_t first_pos = P + tok0 - k0;  // position of the tile's first token, from k0
  // the last key this item may use (a row past it, in a chunk before the
  // last, still stops there: the keys after it are the next chunks')
  const int64_t last_key = kv_len - 1;
  // first key tile that reaches past min(first_pos, last_key), i.e. needs the
  // mask; tiles past the item's keys are always masked
  const int64_t diag_pos = min(first_pos, last_key);
  const int t_diag = diag_pos >= kKeyTile - 1 ? (int)((diag_pos - (kKeyTile - 1)) / kKeyTile) + 1 : 0;

  TileSrc c;
  c.row_stride = (uint32_t)p.Hkv * D * ESZ;
  c.page_stride = (int64_t)c.row_stride * kPageSize;
  c.kbase = (const char*)p.key_pool + (int64_t)h * D * ESZ;
  c.vbase = (const char*)p.value_pool + (int64_t)h * D * ESZ;
  // (PREFIX: the chunk's pages, from the row of the item's first sequence)
  c.bt = (const_i64_ptr)(p.block_table + (int64_t)b * p.max_blocks +
                         (PREFIX ? (int64_t)chunk * p.prefix_chunk_len / kPageSize : k0 / kPageSize));
  c.L = (int)(L - k0);  // positions from k0 on
  c.last_page = (int)((L - k0 + 15) >> 4) - 1;

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
  bf16x8 qb[NB][NKS];
  int32_t qrel[NB];  // min(row position, last_key) - first_pos - 4 qgrp
  bool row_live[NB];
  // (called once the first tile fetches are in flight; every lane loads, rows
  // past the tile from the sequence's first token, so that the loads issue
  // together rather than one exec-masked load and wait at a time)
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = wave * 32 * NB + nb * 32 + qcol;
      const int64_t tok = tok0 + r / G;
      bool live = r < tpt * G && tok < tok_end;
      int64_t qidx;  // packed query row of this lane's row
      if constexpr (PREFIX) {
        // sequence b + tok, if it has a query row
        const int64_t bs = live ? b + tok : b;
        const int64_t qa = p.qsl[bs], qz = p.qsl[bs + 1];
        live = live && qz > qa;
        qidx = live ? qa : 0;
        qrel[nb] = -4 * qgrp;
      } else {
        qidx = q0 + (live ? tok : 0);
        qrel[nb] = (int32_t)min((live ? tok : tok_end - 1) - tok0, last_key - first_pos) - 4 * qgrp;
      }
      row_live[nb] = live;
      const __bf16* qrow = (const __bf16*)p.q + (qidx * p.Hq + h * G + r % G) * D;
      u32x4 raw[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) raw[ks] = *(const u32x4*)(qrow + 16 * ks + 8 * qgrp);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 x = live ? (raw[ks] ^ qflip) : u32x4{0u, 0u, 0u, 0u};
        if constexpr (NB > 1) {
          // park the query operand in AGPRs (MFMA reads A/B from either file),
          // leaving the VGPRs to the softmax and the LDS operand pipeline
          u32x4 xa;
          asm("" : "=a"(xa) : "0"(x));
          qb[nb][ks] = __builtin_bit_cast(bf16x8, xa);
        } else {
          qb[nb][ks] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }
  };

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

  f32x16 acc[NDB][NB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][nb][i] = 0.f;
  // reference max (log2 units); finite so that exp2(-inf - m_ref) stays 0
  float m_ref[NB];
  float l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_ref[nb] = -1e30f;
    l_run[nb] = 0.f;
  }

  // S^T of the K tile in ring slot `slot`: s[nb][i] = score of key 8 (i / 4) +
  // 4 qgrp + i % 4 of the tile and query row 32 nb + qcol
  auto read_k = [&](int slot, bf16x8 (&ka)[NKS]) __attribute__((always_inline)) {
    const char* k = sk[slot];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) ka[ks] = *(const bf16x8*)(k + (kA ^ (32u * ks)));
  };
  auto scores = [&](const bf16x8 (&ka)[NKS], f32x16 (&s)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = mfma32(ka[ks], qb[nb][ks], s[nb]);
  };

  // V^T operands of the V tile in ring slot `slot`, then O^T += V^T P^T
  auto read_v = [&](int slot, bf16x8 (&va)[NDB][2]) __attribute__((always_inline)) {
    const char* v = sv[slot];
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const char* vd = v + (vA ^ (64u * d));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x4 lo = lds_read_tr16(vd + (16 * hh) * 2 * D);
        const s16x4 hi = lds_read_tr16(vd + (16 * hh + 8) * 2 * D);
        va[d][hh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto scores_pv = [&](const bf16x8 (&ka)[NKS], const bf16x8 (&va)[NDB][2], f32x16 (&s)[NB],
                       const bf16x8 (&pb)[2][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
    static_assert(NKS == 2 * NDB, "one PV MFMA per score k-step");
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = mfma32(ka[ks], qb[nb][ks], s[nb]);
      const int d = ks / 2, hh = ks % 2;  // PV MFMA (d, hh) after score k-step ks
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[d][nb] = mfma32(va[d][hh], pb[hh][nb], acc[d][nb]);
    }
  };

  // P(t) = exp2(s * cs - m_ref) from the raw scores of tile t, rounded to
  // bf16; lt = this lane's share of the tile's row sums of the rounded P.
  auto exps = [&](const f32x16 (&s)[NB], bf16x8 (&pb)[2][NB], float (&lt)[NB]) __attribute__((always_inline)) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float neg_m = -m_ref[nb];
      float l = 0.f;
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
      lt[nb] = l;
    }
  };

  // Softmax of tile t with a lazy reference max m_ref.  The common step never
  // computes a max: P is taken against the current reference and, as long as
  // no lane's partial row sum exceeds kLazyBound (so no single P does),
  // the reference stands.  Otherwise (always on the first tile, where m_ref
  // starts at -1e30) the reference moves to the row max, P is recomputed and
  // alpha = exp2(m_old - m_new) is returned for the accumulator; the function
  // then returns true.
  auto softmax = [&](auto mask_c, int t, f32x16 (&s)[NB], bf16x8 (&pb)[2][NB], float (&alpha)[NB]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int32_t lim = (int32_t)(first_pos - (int64_t)t * kKeyTile) + qrel[nb];
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = 8 * (i >> 2) + (i & 3) > lim ? -INFINITY : s[nb][i];
      }
    }
    float lt[NB];
    exps(s, pb, lt);
    bool over = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) over |= lt[nb] > kLazyBound;
    const bool moved = __builtin_amdgcn_ballot_w64(over) != 0;
    // Instruction order of the iteration up to here: the first operand reads,
    // then each MFMA followed by the next operand reads and a run of softmax
    // VALU work that co-executes with it.
    constexpr int kMfma = NKS * NB + 2 * NDB * NB, kReads = NKS + 4 * NDB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (4 + 2 * i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    if (moved) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = __builtin_fmaxf(s[nb][0], s[nb][1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[nb][i], s[nb][i + 1]));
        mx = max_pair(mx) * cs;  // -inf if every key of the row is masked in this tile
        const float m_new = __builtin_fmaxf(m_ref[nb], mx);
        alpha[nb] = m_new == m_ref[nb] ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
        m_ref[nb] = m_new;
        l_run[nb] *= alpha[nb];
      }
      exps(s, pb, lt);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) l_run[nb] += lt[nb];
    return moved;
  };

  // (one 16-register block at a time, so the rare rescale needs few
  // temporaries beside the live state)
  auto rescale = [&](const float (&alpha)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[d][nb] *= alpha[nb];
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // ---- tile fetches.  Tile j lives in ring slot j % NS of its ring.
  using DM = Dma<D, WAVES>;
  // Page ids of this wave's rows; V(j) reuses the id fetched for K(j).
  int64_t page_k[2] = {0, 0}, page_v[2] = {0, 0};

  bf16x8 pb_prev[2][NB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pb_prev[hh][nb] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  f32x16 s_cur[NB];

  // One iteration's compute for tile t in ring position R = t % NS (a
  // compile-time constant, so every LDS address is a base plus an immediate):
  // K(t+1) and V(t-1) are resident.  The MFMAs (scores of tile t+1, P(t-1)
  // V(t-1) into the output) do not depend on the VALU work (the softmax of
  // tile t), and the two are interleaved instruction by instruction so that
  // they co-execute.  Tiles past the sequence are zero filled and fully
  // masked, so iterations past the last tile add nothing.
  // The iteration is fenced off from the code around it (the two iterations
  // of a hand-off share a basic block, and the scheduler would otherwise mix
  // them and undo the interleave), and runs at wave priority 1, so that a
  // wave in its MFMA stream wins the issue over one fetching or widening
  // tiles between iterations.
  auto compute = [&](auto mask_c, auto r_c, int t) __attribute__((always_inline)) {
    constexpr int R = decltype(r_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    bf16x8 ka[NKS], va[NDB][2];
    read_k((R + 1) % NS, ka);
    read_v((R + NS - 1) % NS, va);
    // score MFMAs (one accumulation chain per row block) alternate with the
    // independent PV MFMAs, so no MFMA waits for its predecessor's result
    f32x16 s_next[NB];
    scores_pv(ka, va, s_next, pb_prev);
    float alpha[NB];
    bf16x8 pb[2][NB];
    if (softmax(mask_c, t, s_cur, pb, alpha)) rescale(alpha);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s_cur[nb] = s_next[nb];
      pb_prev[0][nb] = pb[0][nb];
      pb_prev[1][nb] = pb[1][nb];
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // iterations 0 .. n_tiles (the last one only adds P(n_tiles - 1) V):
  // unmasked up to the group holding the diagonal, masked after
  int t = 0;
  if constexpr (ESZ == 2) {
    // bf16: a hand-off at every even iteration t.  After the barrier before
    // iteration t, K(t+1), K(t+2), V(t-1) and V(t) are resident (read by
    // iterations t and t+1), K(t+3), K(t+4), V(t+1) and V(t+2) may still be
    // in flight, and no wave reads any other slot any more: the hand-off
    // fetches K(t+5), K(t+6), V(t+3) and V(t+4) into those.  The fetches are
    // issued after iteration t, so that the iteration's MFMA stream starts
    // right after the barrier (2 % faster than issuing them first).  Every
    // hand-off issues the same number of transfers, so vmcnt(4 LOADS) before
    // the next barrier leaves exactly the latest hand-off's transfers in
    // flight.
    auto handoff = [&](auto r_c, int t) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      dma_tile<D, WAVES, false>(c, (__bf16*)sk[(R + 5) % NS], t + 5, page_k[0], wave, lane);
      dma_tile<D, WAVES, false>(c, (__bf16*)sk[R], t + 6, page_k[1], wave, lane);
      dma_tile<D, WAVES, true>(c, (__bf16*)sv[(R + 3) % NS], t + 3, page_v[0], wave, lane);
      dma_tile<D, WAVES, true>(c, (__bf16*)sv[(R + 4) % NS], t + 4, page_v[1], wave, lane);
      page_v[0] = page_k[0];
      page_v[1] = page_k[1];
    };
    auto pair = [&](auto mask_c, auto r_c, int t) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      barrier_lds();
      compute(mask_c, r_c, t);
      handoff(r_c, t);
      compute(mask_c, std::integral_constant<int, R + 1>{}, t + 1);
      wait_vmem<4 * DM::LOADS>();
      // the next page ids, loaded just before the barrier that waits for them
      // anyway (an earlier scalar load would force a full LDS drain at the
      // first operand wait after it)
      __builtin_amdgcn_sched_barrier(0);
      page_k[0] = wave_page<D, WAVES>(c, t + 7, wave);
      page_k[1] = wave_page<D, WAVES>(c, t + 8, wave);
    };

    // prologue: K(0), K(1), K(2), V(-1) (zero: the first PV multiplies it by
    // P(-1) = 0) and V(0) resident, the scores of tile 0, then the fetches of
    // the hand-off before iteration -2 (no wave reads their slots yet)
    dma_tile<D, WAVES, false>(c, (__bf16*)sk[0], 0, wave_page<D, WAVES>(c, 0, wave), wave, lane);
    dma_tile<D, WAVES, false>(c, (__bf16*)sk[1], 1, wave_page<D, WAVES>(c, 1, wave), wave, lane);
    dma_tile<D, WAVES, false>(c, (__bf16*)sk[2], 2, wave_page<D, WAVES>(c, 2, wave), wave, lane);
    dma_tile<D, WAVES, true>(c, (__bf16*)sv[NS - 1], -1, wave_page<D, WAVES>(c, -1, wave), wave, lane);
    dma_tile<D, WAVES, true>(c, (__bf16*)sv[0], 0, wave_page<D, WAVES>(c, 0, wave), wave, lane);
    load_q();
    wait_vmem<0>();
    barrier_lds();
    {
      bf16x8 ka[NKS];
      read_k(0, ka);
      scores(ka, s_cur);
    }
    dma_tile<D, WAVES, false>(c, (__bf16*)sk[3], 3, wave_page<D, WAVES>(c, 3, wave), wave, lane);
    dma_tile<D, WAVES, false>(c, (__bf16*)sk[4], 4, wave_page<D, WAVES>(c, 4, wave), wave, lane);
    dma_tile<D, WAVES, true>(c, (__bf16*)sv[1], 1, wave_page<D, WAVES>(c, 1, wave), wave, lane);
    dma_tile<D, WAVES, true>(c, (__bf16*)sv[2], 2, wave_page<D, WAVES>(c, 2, wave), wave, lane);
    page_v[0] = wave_page<D, WAVES>(c, 3, wave);
    page_v[1] = wave_page<D, WAVES>(c, 4, wave);
    page_k[0] = wave_page<D, WAVES>(c, 5, wave);
    page_k[1] = wave_page<D, WAVES>(c, 6, wave);

    using I0 = std::integral_constant<int, 0>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    const int t_split = t_diag / NS * NS;
    for (; t < t_split; t += NS) {
      pair(std::false_type{}, I0{}, t);
      pair(std::false_type{}, I2{}, t + 2);
      pair(std::false_type{}, I4{}, t + 4);
    }
    for (; t <= n_tiles; t += NS) {
      pair(std::true_type{}, I0{}, t);
      if (t + 2 > n_tiles) break;
      pair(std::true_type{}, I2{}, t + 2);
      if (t + 4 > n_tiles) break;
      pair(std::true_type{}, I4{}, t + 4);
    }
    wait_vmem<0>();  // no tile write may land after the workgroup ends
  } else {
    // fp8: a hand-off before every even iteration t.  After the barrier the
    // bf16 slots hold K(t+1), K(t+2), V(t-1) and V(t) (read by iterations t
    // and t+1), and the codes of K(t+5), K(t+6), V(t+3) and V(t+4) are
    // fetched into code set (t/2) % 2, whose codes were widened before this
    // barrier.  After iterations t and t+1, the codes the previous hand-off
    // fetched, K(t+3), K(t+4), V(t+1) and V(t+2) (landed in set (t/2 + 1) % 2
    // before the barrier), are widened into the four slots no wave reads any
    // more; vmcnt(0) then lands this hand-off's codes before the next barrier.
    // Widening there rather than right after the barrier measured 4 % faster
    // (the widening's LDS round trip no longer delays the MFMAs' operands).
    using M8 = Dma8<D, WAVES>;
    constexpr int CPR = D / 16;
    constexpr int TASKS = 4 * kKeyTile * CPR;  // 16-code chunks of a set
    static_assert(TASKS % THREADS == 0 && (kKeyTile * CPR) % 64 == 0, "each wave widens chunks of one tile");
    int64_t pg8[M8::LOADS];
    // tile of code slot q fetched at the hand-off before iteration t
    auto tile_of = [](int q, int t) { return q == 0 ? t + 5 : q == 1 ? t + 6 : q == 2 ? t + 3 : t + 4; };
    auto next_pages = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < M8::LOADS; ++k) {
        const int li = wave + WAVES * k, q = li / M8::PER_TILE, part = li % M8::PER_TILE;
        pg8[k] = page8<D, WAVES>(c, tile_of(q, t), part);
      }
    };
    auto fetch_codes = [&](int set, int t) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < M8::LOADS; ++k) {
        const int li = wave + WAVES * k, q = li / M8::PER_TILE, part = li % M8::PER_TILE;
        dma8_rows<D, WAVES>(c, q < 2 ? c.kbase : c.vbase, sc[set][q], tile_of(q, t), part, pg8[k], lane);
      }
    };
    // widen code set `set` (slots 0..3) into dst[q]; slots 2 and 3 hold V
    // tiles unless v2 is false (the prologue's K(2))
    auto widen = [&](int set, char* d0, char* d1, char* d2, char* d3, bool v2) __attribute__((always_inline)) {
#pragma unroll
      for (int j0 = 0; j0 < TASKS; j0 += THREADS) {
        const int j = j0 + tid, q = j / (kKeyTile * CPR), task = j % (kKeyTile * CPR);
        char* dst = q == 0 ? d0 : q == 1 ? d1 : q == 2 ? d2 : d3;
        widen_chunk<D>(sc[set][q], dst, q == 3 || (q == 2 && v2), task / CPR, task % CPR);
      }
    };
    auto pair8 = [&](auto mask_c, auto r_c, int t) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      barrier_lds();
      fetch_codes(R / 2, t);
      compute(mask_c, r_c, t);
      compute(mask_c, std::integral_constant<int, R + 1>{}, t + 1);
      // (after the pair's MFMAs, whose operand reads it would otherwise delay;
      // its writes reach the other waves through the next barrier)
      widen((R / 2 + 1) % 2, sk[(R + 3) % NS], sk[R], sv[(R + 1) % NS], sv[(R + 2) % NS], true);
      wait_vmem<0>();
      __builtin_amdgcn_sched_barrier(0);
      next_pages(t + 2);
    };

    // prologue: codes of K(0), K(1), K(2) and V(0) into set 0, of K(3), K(4),
    // V(1) and V(2) into set 1; set 0 widened into K slots 0..2 and V slot 0,
    // V slot 3 (V(-1), multiplied by P(-1) = 0) zeroed; the scores of tile 0
#pragma unroll
    for (int k = 0; k < M8::LOADS; ++k) {
      const int li = wave + WAVES * k, q = li / M8::PER_TILE, part = li % M8::PER_TILE;
      const int t0 = q == 3 ? 0 : q, t1 = q == 0 ? 3 : q == 1 ? 4 : q - 1;
      dma8_rows<D, WAVES>(c, q == 3 ? c.vbase : c.kbase, sc[0][q], t0, part, page8<D, WAVES>(c, t0, part), lane);
      dma8_rows<D, WAVES>(c, q >= 2 ? c.vbase : c.kbase, sc[1][q], t1, part, page8<D, WAVES>(c, t1, part), lane);
    }
    load_q();
    wait_vmem<0>();
    barrier_lds();
    widen(0, sk[0], sk[1], sk[2], sv[0], false);
    for (int i = tid; i < TB / 16; i += THREADS) ((u32x4*)sv[3])[i] = u32x4{0u, 0u, 0u, 0u};
    barrier_lds();
    {
      bf16x8 ka[NKS];
      read_k(0, ka);
      scores(ka, s_cur);
    }
    next_pages(0);

    using I0 = std::integral_constant<int, 0>;
    using I2 = std::integral_constant<int, 2>;
    const int t_split = t_diag / NS * NS;
    for (; t < t_split; t += NS) {
      pair8(std::false_type{}, I0{}, t);
      pair8(std::false_type{}, I2{}, t + 2);
    }
    for (; t <= n_tiles; t += NS) {
      pair8(std::true_type{}, I0{}, t);
      if (t + 2 > n_tiles) break;
      pair8(std::true_type{}, I2{}, t + 2);
    }
    wait_vmem<0>();  // no code fetch may land after the workgroup ends
  }


  // acc[d][nb][i] = O^T[dim 32 d + 8 (i / 4) + 4 qgrp + i % 4][row]
  float out_scale = 1.0f;
  if constexpr (ESZ == 1) out_scale = p.v_scale[h];
  if constexpr (PREFIX) {
    // partial of (chunk, sequence, query head) as the merge expects it: m_ref
    // in log2 units, the row sum of the rounded P, and the unnormalised O in
    // fp16 times a power of two that puts the row's largest magnitude in
    // [2^14, 2^15), with that power's inverse
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l = sum_pair(l_run[nb]);
      // (every lane takes part: the row's two lane groups exchange their maxima)
      float mx = 0.f;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(acc[d][nb][i]));
      mx = fmaxf(mx, xor_shuffle(mx, 32));
      const int k = min(max(__builtin_amdgcn_frexp_expf(mx * fabsf(out_scale)), -100), 128);
      const float sc = out_scale * __builtin_amdgcn_ldexpf(1.f, 15 - k);
      if (!row_live[nb]) continue;
      const int r = wave * 32 * NB + nb * 32 + qcol;
      const int64_t slot = ((int64_t)chunk * p.B + b + r / G) * p.Hq + h * G + r % G;
      _Float16* orow = p.ws_pre_o + slot * D;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16& a = acc[d][nb];
          *(u32x2*)(orow + d * 32 + 8 * i4 + 4 * qgrp) = u32x2{pack_f16x2(a[4 * i4] * sc, a[4 * i4 + 1] * sc),
                                                               pack_f16x2(a[4 * i4 + 2] * sc, a[4 * i4 + 3] * sc)};
        }
      if (qgrp == 0) *(f32x4*)(p.ws_pre_ml + 4 * slot) = f32x4{m_ref[nb], l, __builtin_amdgcn_ldexpf(1.f, k - 15), 0.f};
    }
    return;
  }
  if (n_chunks > 1) {
    // one chunk of a split item: its partial per row, combined by
    // prefill_split_merge_kernel (plans past the bound write nothing)
    if (gtile >= p.plan_tiles_cap) return;
    // (m_ref, l, inverse scale) and the unnormalised row in fp16 times a power
    // of two that puts its largest magnitude in [2^14, 2^15), as for the
    // shared prefix's partials
    const int64_t item_slot = ((int64_t)gtile * p.Hkv + h) * p.split_max_chunks + chunk;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l = sum_pair(l_run[nb]);
      float mx = 0.f;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(acc[d][nb][i]));
      mx = fmaxf(mx, xor_shuffle(mx, 32));
      const int k = min(max(__builtin_amdgcn_frexp_expf(mx * fabsf(out_scale)), -100), 128);
      const float sc = out_scale * __builtin_amdgcn_ldexpf(1.f, 15 - k);
      const int r = wave * 32 * NB + nb * 32 + qcol;
      const int64_t slot = item_slot * kPrefillRows + r;
      _Float16* orow = p.ws_split_o + slot * D;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16& a = acc[d][nb];
          *(u32x2*)(orow + d * 32 + 8 * i4 + 4 * qgrp) = u32x2{pack_f16x2(a[4 * i4] * sc, a[4 * i4 + 1] * sc),
                                                               pack_f16x2(a[4 * i4 + 2] * sc, a[4 * i4 + 3] * sc)};
        }
      if (qgrp == 0) *(f32x4*)(p.ws_split_ml + 4 * slot) = f32x4{m_ref[nb], l, __builtin_amdgcn_ldexpf(1.f, k - 15), 0.f};
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = sum_pair(l_run[nb]);
    const int r = wave * 32 * NB + nb * 32 + qcol;
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

template <int ESZ, int D, int NB>
__global__ __launch_bounds__(512 / NB) __attribute__((amdgpu_waves_per_eu(3 - NB, 3 - NB)))
void prefill_kernel(AttnParams p) {
  __shared__ PrefillLds<ESZ, D> lds;
  prefill_item<ESZ, D, NB, false>(p, lds, blockIdx.x, 0);
}

// Shared-prefix decode in one launch.  Workgroups 0 .. n_dec - 1 run the
// split-K pass over the positions past the prefix (n_dec =
// dk::decode_workgroups(p)), the next prefix_wgs workgroups the prefix items:
// workgroup j takes items j / Hkv, j / Hkv + per_head, ... of KV head
// j % Hkv, per_head = prefix_wgs / Hkv.  The two kinds are bound by different
// units (HBM; MFMA and exp) and start together, so the prefix's tiles run
// while the private positions stream.  n_dec and prefix_wgs are multiples of
// 8 and workgroups are dealt to the 8 XCDs in turn, so a prefix workgroup and
// its KV head keep to one XCD (the items of a head re-read its K/V from that
// XCD's L2).  Every workgroup has 8 waves: a decode workgroup whose groups
// use fewer leaves the others idle after the length scan.
template <int ESZ, int D>
union SharedPrefixLds {
  dk::DecodeLds<D> dec;
  PrefillLds<ESZ, D> pre;
};

template <int ESZ, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void shared_prefix_decode_kernel(AttnParams p) {
  __shared__ SharedPrefixLds<ESZ, D> lds;
  const unsigned n_dec = (unsigned)dk::decode_workgroups(p);
  if (blockIdx.x < n_dec) {
    dk::decode_body<ESZ, D>(p, lds.dec, blockIdx.x, n_dec);
    return;
  }
  const unsigned j = blockIdx.x - n_dec;
  const int per_head = p.prefix_wgs / p.Hkv;
  const int items = p.prefix_tiles * p.prefix_chunks;
  static_assert(kPrefillRowBlocks == 1, "prefix items run as 8 waves of 32 rows, like the decode workgroups");
  for (int r0 = 0; r0 < items; r0 += per_head) {
    if (r0 > 0) __syncthreads();  // every wave is done with the last item's tiles
    prefill_item<ESZ, D, 1, true>(p, lds.pre, j, r0);
  }
}

// Key-split prefill: combine the chunks' partials of every row of a split
// (sequence, query tile, KV head) with a log-sum-exp merge,
//   M = max_c m_c,  out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,
// one wave per row (4 per workgroup), lane i over elements i * PER .. + PER - 1
// of the head dimension.  O_c is stored in fp16 divided by a power of two, u_c
// (its partial's third value), and enters as u_c times the stored row.
// Chunk 0 starts at key 0, which every row sees, so M is finite; a chunk that
// lies wholly past a row's position left m = -1e30 and l = 0 there (weight 0).
template <int D>
__global__ __launch_bounds__(256) void prefill_split_merge_kernel(AttnParams p) {
  constexpr int PER = D / 64;
  const int g = (int)(blockIdx.x / (unsigned)p.Hkv), h = (int)(blockIdx.x % (unsigned)p.Hkv);
  if (g >= p.ws_plan[1]) return;
  const int64_t items_cap = p.plan_tiles_cap * p.split_max_chunks;
  const uint32_t item = (uint32_t)p.ws_plan[2 + 2 * items_cap + g];
  const int b = (int)(item >> 16), tile = (int)(item & 0xFFFF);
  const int G = p.G, tpt = kPrefillRows / G;
  const int64_t q0 = p.qsl[b], n = p.qsl[b + 1] - q0, P = p.seq_lens[b] - n;
  const int64_t tok0 = (int64_t)tile * tpt, tok_end = min(tok0 + (int64_t)tpt, n);
  const int nch = item_chunks(p, P + tok_end);
  if (nch <= 1) return;  // written directly by prefill_kernel
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int r = (int)blockIdx.y * 4 + wave;
  const int64_t tok = tok0 + r / G;
  if (r >= tpt * G || tok >= tok_end) return;
  const int64_t base = ((int64_t)g * p.Hkv + h) * p.split_max_chunks;
  const f32x4* ml = (const f32x4*)p.ws_split_ml;
  // chunks in groups of 8, every load of a group issued before any is used
  constexpr int CH = 8;
  float M = -INFINITY, l = 0.f, o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += CH) {
    f32x4 x[CH];
    float oc[CH][PER];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t slot = (base + min(c0 + k, nch - 1)) * kPrefillRows + r;
      x[k] = ml[slot];
      load_f16_elems<PER>(p.ws_split_o + slot * D, lane, oc[k]);
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      x[k][0] = c0 + k < nch ? x[k][0] : -INFINITY;  // repeats of the last chunk weigh 0
      Mc = fmaxf(Mc, x[k][0]);
    }
    const float alpha = M == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mc);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= alpha;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float f = __builtin_amdgcn_exp2f(x[k][0] - Mc);
      l += f * x[k][1];
      const float g = f * x[k][2];
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += g * oc[k][i];
    }
    M = Mc;
  }
  const float inv = 1.0f / l;
  __bf16* orow = (__bf16*)p.out + ((q0 + tok) * p.Hq + h * G + r % G) * D;
  if constexpr (PER == 2)
    ((uint32_t*)orow)[lane] = pack_bf16x2(o[0] * inv, o[1] * inv);
  else
    orow[lane] = (__bf16)(o[0] * inv);
}

// Shared-prefix decode, prefix part: one item per (group of prefill_tokens_per_tile
// sequences, chunk of the prefix).  The chunk count is chosen for about 256
// workgroups whatever the device, so the workspace size depends on the shapes
// only.
// Shared-prefix schedule (shared_prefix_decode_kernel).  The prefix items
// (group of sequences x chunk of the prefix x KV head) run on prefix_wgs
// workgroups while the decode of the private positions streams on the rest
// of the CUs.  The two are bound by different units: the items by their
// MFMAs and exps, the decode by the loads each CU keeps in flight.
//
// The split comes from a model fitted to measurements on MI355X:
//  * an item costs (its 32-key tiles + kPrefixItemTiles) x kPrefixTileNs (the
//    fixed part is its start-up and the write-back of its partials);
//  * the decode streams an estimate of the private bytes (half of what the
//    block table holds past the prefix, as seq_lens stays on the device) at
//    kDecodeBytesPerNs x n / (n + kDecodeHalfCus) on n CUs: each CU's rate
//    rises as fewer CUs share HBM;
//  * the merge then reads each prefix chunk's partials at kMergeBytesPerNs.
// For each number of items per head (a multiple of 8 / gcd(Hkv, 8), so that
// the decode part keeps a multiple of 8 workgroups) the chunk count with the
// fewest estimated tiles is taken (ties: fewer chunks), then the number with
// the least estimated time, max(decode, items) + merge (ties: fewer prefix
// workgroups); the decode keeps at least a quarter of the CUs.
constexpr int kPrefixItemTiles = 13;
constexpr double kPrefixTileNs = 950.0;      // one 32-key tile of a 256-row item, D = 128
constexpr double kDecodeBytesPerNs = 5600.0;
constexpr double kDecodeHalfCus = 75.0;
constexpr double kMergeBytesPerNs = 3000.0;

// chunk count and estimated tiles of the prefix items at per_head workgroups per KV head
static void prefix_chunking(int64_t n_tiles, int64_t groups, int64_t per_head, int64_t& chunks_out,
                            int64_t& cost_out) {
  const int64_t max_chunks = std::max<int64_t>(1, std::min<int64_t>(kMaxPrefixChunks, n_tiles));
  chunks_out = 1;
  cost_out = INT64_MAX;
  for (int64_t c = 1; c <= max_chunks; ++c) {
    const int64_t len = (n_tiles + c - 1) / c;  // tiles per chunk
    if ((n_tiles + len - 1) / len != c) continue;  // the same cut as a smaller count
    const int64_t rounds = (groups * c + per_head - 1) / per_head;
    const int64_t cost = rounds * (len + kPrefixItemTiles);
    if (cost < cost_out) {
      chunks_out = c;
      cost_out = cost;
    }
  }
}

size_t prefix_plan(AttnParams& p, int64_t prefix_len, int n_cu, bool tight) {
  const int tpt = prefill_tokens_per_tile(p.G);
  p.prefix_len = prefix_len;
  p.prefix_tiles = (int)((p.B + tpt - 1) / tpt);
  const int64_t n_tiles = prefix_len / kKeyTile;
  const double private_bytes = (double)p.B * std::max<int64_t>(0, p.max_blocks * kPageSize - prefix_len) / 2 * p.Hkv *
                               p.D * std::max(p.kv_bytes, 1) * 2;
  const double tile_ns = kPrefixTileNs * p.D / 128;
  const int64_t step = 8 / std::gcd<int64_t>(p.Hkv, 8);
  const int64_t max_per_head = std::max<int64_t>(step, ((int64_t)n_cu - n_cu / 4) / p.Hkv / step * step);
  int64_t per_head = step, chunks = 1;
  double best = INFINITY;
  for (int64_t k = step; k <= max_per_head; k += step) {
    int64_t c, tiles;
    prefix_chunking(n_tiles, p.prefix_tiles, k, c, tiles);
    const double cus = std::max<double>(1.0, (double)n_cu - (double)k * p.Hkv);
    const double t_dec = private_bytes * (cus + kDecodeHalfCus) / (kDecodeBytesPerNs * cus);
    const double t_merge = (double)c * p.B * p.Hq * (p.D + 2) * sizeof(float) / kMergeBytesPerNs;
    const double t = std::max(t_dec, tiles * tile_ns) + t_merge;
    if (t < best) {
      best = t;
      per_head = k;
      chunks = c;
    }
  }
  p.prefix_wgs = (int)(per_head * p.Hkv);
  const int64_t len = (n_tiles + chunks - 1) / chunks * kKeyTile;
  p.prefix_chunk_len = (int)len;
  p.prefix_chunks = (int)((prefix_len + len - 1) / len);
  const int64_t max_chunks = std::max<int64_t>(1, std::min<int64_t>(kMaxPrefixChunks, n_tiles));
  const size_t slots = (size_t)(tight ? p.prefix_chunks : max_chunks) * p.B * p.Hq;
  return (slots * 4 * sizeof(float) + 255) / 256 * 256 + slots * p.D * sizeof(_Float16);
}

void prefix_workspace_carve(AttnParams& p, void* region) {
  const size_t slots = (size_t)p.prefix_chunks * p.B * p.Hq;
  p.ws_pre_ml = (float*)region;
  p.ws_pre_o = (_Float16*)((char*)region + (slots * 4 * sizeof(float) + 255) / 256 * 256);
}

hipError_t launch_shared_prefix_decode(const AttnParams& p, hipStream_t stream) {
  const int n_dec = dk::decode_workgroups(p);
  const dim3 grid((unsigned)(n_dec + p.prefix_wgs)), block(512);
  const bool fp8 = p.kv_type == KV_FP8;
  if (p.D == 128) {
    if (fp8) hipLaunchKernelGGL((shared_prefix_decode_kernel<1, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((shared_prefix_decode_kernel<2, 128>), grid, block, 0, stream, p);
  } else {
    if (fp8) hipLaunchKernelGGL((shared_prefix_decode_kernel<1, 64>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((shared_prefix_decode_kernel<2, 64>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev) {
  if (p.T == 0 || p.B == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  if (ev.begin) (void)hipEventRecord(ev.begin, stream);
  // one workgroup per (item, KV head): at most plan_tiles_cap * split_max_chunks items
  const dim3 grid((unsigned)(p.plan_tiles_cap * p.split_max_chunks * p.Hkv));
  constexpr int NB = kPrefillRowBlocks;
  const dim3 block(512 / NB);
  const bool fp8 = p.kv_type == KV_FP8;
  if (p.D == 128) {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<1, 128, NB>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_kernel<2, 128, NB>), grid, block, 0, stream, p);
  } else {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<1, 64, NB>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_kernel<2, 64, NB>), grid, block, 0, stream, p);
  }
  if (ev.end) (void)hipEventRecord(ev.end, stream);
  if (p.split_keys > 0) {
    const dim3 mgrid((unsigned)(p.plan_tiles_cap * p.Hkv), kPrefillRows / 4);
    if (p.D == 128) hipLaunchKernelGGL(prefill_split_merge_kernel<128>, mgrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(prefill_split_merge_kernel<64>, mgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
