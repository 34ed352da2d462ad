// decode_device.h -- device code of the split-K paged decode pass (the
// kernel body and its helpers), shared by decode_kernel and the shared-prefix
// kernel.  What it computes and how it maps onto gfx950 is described at the
// top of decode.hip.
#pragma once
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pkv {
namespace dk {

constexpr int kUnit = 32;      // key positions per unit of work (two pages)
// dword 3 of a raw (unformatted, stride 0) buffer descriptor: 32-bit data format
constexpr int kBufferWord3 = 0x00020000;
// cache policy of the KV stream: non-temporal (each byte is read once)
constexpr int kStreamAux = 2;
constexpr int kMaxWaves = 8;   // waves per workgroup

constexpr int kCopyRegs = 2;   // fused write: 16-byte chunks per thread and pool

#ifndef PKV_DECODE_MAX_GROUPS
#define PKV_DECODE_MAX_GROUPS 8
#endif

__host__ __device__ inline int decode_heads_per_wave(int Hkv) { return (Hkv + kMaxWaves - 1) / kMaxWaves; }
// waves of one group: together they cover every KV head of a part
__host__ __device__ inline int decode_waves(int Hkv) {
  const int hpw = decode_heads_per_wave(Hkv);
  return (Hkv + hpw - 1) / hpw;
}
// groups (parts) per workgroup: with fewer KV heads than waves, the workgroup
// runs several parts side by side, so the CU keeps 8 waves' loads in flight
__host__ __device__ inline int decode_groups(int Hkv) {
  const int g = kMaxWaves / decode_waves(Hkv);
  return g < PKV_DECODE_MAX_GROUPS ? g : PKV_DECODE_MAX_GROUPS;
}
// workgroups of the decode launch of p: grid_parts / groups per workgroup,
// each group running decode_rounds consecutive parts
__host__ __device__ inline int decode_workgroups(const AttnParams& p) {
  return p.grid_parts / (decode_groups(p.Hkv) * (p.decode_rounds > 1 ? p.decode_rounds : 1));
}

// four accumulator values times inv, as two packed bf16 pairs
__device__ __forceinline__ u32x2 normalised(const f32x4 a, const float inv) {
  return u32x2{pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
}
// four accumulator values times s, as two packed fp16 pairs (round to nearest even)
__device__ __forceinline__ u32x2 scaled_f16(const f32x4 a, const float s) {
  return u32x2{pack_f16x2(a[0] * s, a[1] * s), pack_f16x2(a[2] * s, a[3] * s)};
}

// Units of sequence b: its 32-position blocks past the shared prefix (if
// any), or none when it has no query row.  len_out = seq_lens[b].
__device__ __forceinline__ int32_t seq_units(const AttnParams& p, int b, int64_t& len_out) {
  const int64_t qa = p.qsl[b], qz = p.qsl[b + 1], L = p.seq_lens[b];
  len_out = L;
  if (qz == qa) return 0;
  const int64_t keys = L - p.prefix_len;
  return keys > 0 ? (int32_t)((keys + kUnit - 1) / kUnit) : 0;
}

// K of a unit is read in whole-row runs (each load instruction covers RPI
// complete rows of the head's D*ESZ bytes), then transposed into the MFMA
// layout through a per-wave LDS tile of 32 bf16 rows.
template <int ESZ, int D>
struct KGeom {
  static constexpr int LPR = D * ESZ / 16;  // lanes per K row (16 bytes each)
  static constexpr int RPI = 64 / LPR;      // rows per load instruction
  static constexpr int NKI = kUnit / RPI;   // load instructions per unit
  static constexpr int IPP = NKI / 2;       // ... per page
  static constexpr int NC = D / 8;          // 16-byte bf16 chunks per LDS row
  // chunk swizzles.  K: the 16 rows an MFMA operand read touches land in 16
  // different bank groups.  V: one pass of a transposing read serves 32 lanes
  // (256 bytes, all 64 banks) and touches 8 rows x 2 chunks, which land in 16
  // different bank groups.
  __device__ static int swz(int row) { return (row / (16 / NC)) % NC; }
  __device__ static int swz_v(int row) { return (2 * ((row / (16 / NC)) % (NC / 2))) % NC; }
};

// Raw K and V bytes of one unit for one KV head, as one lane holds them
// (both read in whole-row runs).
template <int ESZ, int D>
struct UnitRegs {
  u32x4 k[KGeom<ESZ, D>::NKI];
  u32x4 v[KGeom<ESZ, D>::NKI];
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

// Per-lane address parts of a unit (32-bit offsets from a page base): load i
// of a page reads row (i*RPI + lane/LPR), bytes [16*(lane%LPR), +16).
struct LaneOffsets {
  uint32_t k[8];
};

// Loads of one unit: page bases live in buffer descriptors (scalar
// registers), the per-lane part of every address is a 32-bit offset.
template <int ESZ, int D>
__device__ __forceinline__ void issue_k(UnitRegs<ESZ, D>& u, __amdgpu_buffer_rsrc_t kp0, __amdgpu_buffer_rsrc_t kp1,
                                        const LaneOffsets& off) {
  using G = KGeom<ESZ, D>;
#pragma unroll
  for (int i = 0; i < G::NKI; ++i)
    u.k[i] = __builtin_amdgcn_raw_buffer_load_b128(i < G::IPP ? kp0 : kp1, (int)off.k[i % G::IPP], 0, kStreamAux);
}

// Raw K of the unit -> the wave's LDS tile (bf16, 32 rows x D, swizzled chunks).
template <int ESZ, int D>
__device__ __forceinline__ void stage_k(const UnitRegs<ESZ, D>& u, __bf16* __restrict__ tile, int lane) {
  using G = KGeom<ESZ, D>;
  const int cs = lane % G::LPR;
#pragma unroll
  for (int i = 0; i < G::NKI; ++i) {
    const int row = (i / G::IPP) * 16 + (i % G::IPP) * G::RPI + lane / G::LPR;
    __bf16* r = tile + row * D;
    if constexpr (ESZ == 2) {
      *(u32x4*)(r + 8 * (cs ^ G::swz(row))) = u.k[i];
    } else {
      const u32x2 c0 = fp8x4_to_bf16x4(u.k[i].x), c1 = fp8x4_to_bf16x4(u.k[i].y);
      const u32x2 c2 = fp8x4_to_bf16x4(u.k[i].z), c3 = fp8x4_to_bf16x4(u.k[i].w);
      *(u32x4*)(r + 8 * ((2 * cs) ^ G::swz(row))) = u32x4{c0.x, c0.y, c1.x, c1.y};
      *(u32x4*)(r + 8 * ((2 * cs + 1) ^ G::swz(row))) = u32x4{c2.x, c2.y, c3.x, c3.y};
    }
  }
}

template <int ESZ, int D>
__device__ __forceinline__ void issue_v(UnitRegs<ESZ, D>& u, __amdgpu_buffer_rsrc_t vp0, __amdgpu_buffer_rsrc_t vp1,
                                        const LaneOffsets& off) {
  using G = KGeom<ESZ, D>;
#pragma unroll
  for (int i = 0; i < G::NKI; ++i)
    u.v[i] = __builtin_amdgcn_raw_buffer_load_b128(i < G::IPP ? vp0 : vp1, (int)off.k[i % G::IPP], 0, kStreamAux);
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

// Raw V of the unit -> the wave's V tile (bf16, 32 rows x D, swizzled
// chunks).  Rows at positions >= len are stored as zeros: a masked key has
// P = 0, and 0 * NaN would poison the MFMA sum.
template <int ESZ, int D>
__device__ __forceinline__ void stage_v(const UnitRegs<ESZ, D>& u, __bf16* __restrict__ tile, int lane, int64_t pos0,
                                        int64_t len) {
  using G = KGeom<ESZ, D>;
  const int cs = lane % G::LPR;
#pragma unroll
  for (int i = 0; i < G::NKI; ++i) {
    const int row = (i / G::IPP) * 16 + (i % G::IPP) * G::RPI + lane / G::LPR;
    const bool live = pos0 + row < len;
    __bf16* r = tile + row * D;
    if constexpr (ESZ == 2) {
      *(u32x4*)(r + 8 * (cs ^ G::swz_v(row))) = live ? u.v[i] : u32x4{0u, 0u, 0u, 0u};
    } else {
      const u32x2 c0 = fp8x4_to_bf16x4(u.v[i].x), c1 = fp8x4_to_bf16x4(u.v[i].y);
      const u32x2 c2 = fp8x4_to_bf16x4(u.v[i].z), c3 = fp8x4_to_bf16x4(u.v[i].w);
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(r + 8 * ((2 * cs) ^ G::swz_v(row))) = live ? u32x4{c0.x, c0.y, c1.x, c1.y} : z;
      *(u32x4*)(r + 8 * ((2 * cs + 1) ^ G::swz_v(row))) = live ? u32x4{c2.x, c2.y, c3.x, c3.y} : z;
    }
  }
}

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<__bf16*>(p)));
}

// V^T operand of output MFMA t: dims [16t, 16t+16) as rows, the lane group's
// 8 keys (4*grp + e of page 0, then of page 1) as the reduction index, read
// with two transposing LDS reads of 4 keys each.
template <int ESZ, int D>
__device__ __forceinline__ bf16x8 v_operand(const __bf16* __restrict__ tile, int t, int lane) {
  using G = KGeom<ESZ, D>;
  const int grp = lane >> 4, li = lane & 15;
  const int dim = 16 * t + 4 * (li & 3);  // this lane's 4-element run
  const int c = dim / 8, within = dim % 8;
  const int k0 = 4 * grp + (li >> 2), k1 = k0 + 16;
  const s16x4 lo = lds_read_tr16(tile + k0 * D + 8 * (c ^ G::swz_v(k0)) + within);
  const s16x4 hi = lds_read_tr16(tile + k1 * D + 8 * (c ^ G::swz_v(k1)) + within);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// K operand of score MFMA kk on page pp: row 16*pp + (lane & 15), dims
// [32*kk + 8*grp, +8), read from the wave's LDS tile.
template <int ESZ, int D>
__device__ __forceinline__ bf16x8 k_operand(const __bf16* __restrict__ tile, int pp, int kk, int col, int grp) {
  using G = KGeom<ESZ, D>;
  const int row = 16 * pp + col;
  return *(const bf16x8*)(tile + row * D + 8 * ((4 * kk + grp) ^ G::swz(row)));
}

// Fused write: row `row` of the unit's K and V tiles replaced by the key the
// step writes at the sequence's last position, held in registers (lane c <
// D * ESZ / 16 holds bytes [16 c, 16 c + 16) of the K and V rows), laid out
// as stage_k / stage_v lay out a pool row (same wave, so these LDS writes
// land after the staged ones).
template <int ESZ, int D>
__device__ __forceinline__ void put_new_row(__bf16* __restrict__ ktile, __bf16* __restrict__ vtile, int row,
                                            const u32x4& nk, const u32x4& nv, int lane) {
  using G = KGeom<ESZ, D>;
  constexpr int NCH = D * ESZ / 16;
  if (lane >= NCH) return;
  __bf16* kr = ktile + row * D;
  __bf16* vr = vtile + row * D;
  if constexpr (ESZ == 2) {
    *(u32x4*)(kr + 8 * (lane ^ G::swz(row))) = nk;
    *(u32x4*)(vr + 8 * (lane ^ G::swz_v(row))) = nv;
  } else {
    const u32x2 k0 = fp8x4_to_bf16x4(nk.x), k1 = fp8x4_to_bf16x4(nk.y);
    const u32x2 k2 = fp8x4_to_bf16x4(nk.z), k3 = fp8x4_to_bf16x4(nk.w);
    const u32x2 v0 = fp8x4_to_bf16x4(nv.x), v1 = fp8x4_to_bf16x4(nv.y);
    const u32x2 v2 = fp8x4_to_bf16x4(nv.z), v3 = fp8x4_to_bf16x4(nv.w);
    *(u32x4*)(kr + 8 * ((2 * lane) ^ G::swz(row))) = u32x4{k0.x, k0.y, k1.x, k1.y};
    *(u32x4*)(kr + 8 * ((2 * lane + 1) ^ G::swz(row))) = u32x4{k2.x, k2.y, k3.x, k3.y};
    *(u32x4*)(vr + 8 * ((2 * lane) ^ G::swz_v(row))) = u32x4{v0.x, v0.y, v1.x, v1.y};
    *(u32x4*)(vr + 8 * ((2 * lane + 1) ^ G::swz_v(row))) = u32x4{v2.x, v2.y, v3.x, v3.y};
  }
}

// One unit of the online softmax for one KV head: stage the unit's K and V
// into the wave's LDS tiles, call next() (which issues the following unit's
// loads into the now free registers), then scores for 32 keys, the running
// max/sum update and the P.V accumulation.  pos0 = position of the unit's first
// key; keys at positions >= len are masked.  new_row >= 0 (fused write):
// that row of the tiles is the step's new key, taken from nk / nv.
template <int ESZ, int D, class Next>
__device__ __forceinline__ void consume_unit(UnitRegs<ESZ, D>& u, __bf16* __restrict__ ktile, __bf16* __restrict__ vtile,
                                             const bf16x8 (&qb)[D / 32], f32x4 (&acc)[D / 16], float& m_run,
                                             float& l_run, float logit_scale, int64_t pos0, int64_t len, int lane,
                                             int new_row, const u32x4& nk, const u32x4& nv, Next next) {
  constexpr int NKK = D / 32, NJ = D / 16;
  const int col = lane & 15, grp = lane >> 4;
  stage_k<ESZ, D>(u, ktile, lane);
  stage_v<ESZ, D>(u, vtile, lane, pos0, len);
  if (new_row >= 0) put_new_row<ESZ, D>(ktile, vtile, new_row, nk, nv, lane);
  next();
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    s0 = mfma16(k_operand<ESZ, D>(ktile, 0, kk, col, grp), qb[kk], s0);
    s1 = mfma16(k_operand<ESZ, D>(ktile, 1, kk, col, grp), qb[kk], s1);
  }
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
  // P.V: acc[t][i] = O^T[dim 16t + 4*grp + i][head col]
#pragma unroll
  for (int t = 0; t < NJ; ++t) acc[t] = mfma16(v_operand<ESZ, D>(vtile, t, lane), pb, acc[t]);
}

// Cut of U units into W contiguous ranges: the first r = U mod W workgroups
// take q + 1 = floor(U / W) + 1 units, the others q.  start() is
// division-free; owner(u) is the workgroup whose range holds unit u.
struct Partition {
  int32_t q, r;
  // (U < 2^31 units, W <= the grid size: 32-bit division)
  __device__ Partition(int32_t U, int32_t W) : q((int32_t)((uint32_t)U / (uint32_t)W)), r((int32_t)((uint32_t)U % (uint32_t)W)) {}
  __device__ int32_t start(int32_t w) const { return w * q + min(w, r); }
  __device__ int32_t owner(int32_t u) const {
    const int32_t big = r * (q + 1);  // units held by the q+1-unit ranges
    return u < big ? u / (q + 1) : r + (u - big) / q;
  }
  __device__ bool empty(int32_t w) const { return q == 0 && w >= r; }
};

// Stream-K decode.  The flattened list of (sequence, unit) pairs is cut into
// grid_parts equal contiguous ranges (parts).  Group gi of workgroup w runs
// the `rounds` = grid_parts / (nblocks * R) consecutive parts from
// (w * R + gi) * rounds on, as one stream; it walks the segments of its range:
// the pieces of a sequence that lie in one part.  Wave k of a group handles
// KV heads k, k + (waves per group), ... of every segment.  After the scan the
// groups share no barrier, so a group whose range is empty leaves.
//
// A segment that covers a whole sequence writes the normalised output;
// otherwise it writes a partial to slot (b + part), which merge_kernel
// combines.  Slots are unique because the ranges are ordered: a later
// sequence only meets later parts.  A partial is its (max, sum) in fp32 and
// its unnormalised output row in fp16, scaled by a power of two that puts
// the row's largest magnitude in [2^14, 2^15), with the inverse of that power
// as a third fp32.  Partial rows cost the stream far more HBM time than their
// bytes; fp16 halves the bytes of fp32 and keeps 11 significant bits (bf16
// keeps 8, which measurably raises the merged output's error).
//
// Each wave processes its work as one stream of units: a run is one KV head of
// one segment, runs follow segment by segment (heads inside a segment), and
// the loads of the next unit are issued while the current one is computed
// even when the next unit opens a new run.  Page ids are fetched two units
// ahead.  Lengths come from the scan's LDS tables, so opening a run needs no
// dependent global load.

// A position in a wave's stream: unit j of run (sequence b, head slot hk) of
// the segment of b that lies in part w, units [j0, j1) of b.  b < 0 past the
// end of the stream.
struct StreamPos {
  int b, hk;
  int32_t j, j0, j1;
  int w;
};

// LDS of one decode workgroup
template <int D>
struct DecodeLds {
  alignas(256) __bf16 ktile[kMaxWaves][kUnit * D];
  alignas(256) __bf16 vtile[kMaxWaves][kUnit * D];
  int32_t cum[kDecodeMaxSeqs + 1];
  // positions of each sequence's last unit (1..32), to rebuild its length
  uint8_t tail[kDecodeMaxSeqs];
  alignas(16) int32_t wave_units[kMaxWaves];
};

// The split-K pass as run by workgroup `block` of `nblocks` (decode_kernel:
// blockIdx.x of gridDim.x; the shared-prefix kernel runs it in its first
// nblocks workgroups).
template <int ESZ, int D>
__device__ __forceinline__ void decode_body(const AttnParams p, DecodeLds<D>& lds, const unsigned block,
                                            const unsigned nblocks) {
  constexpr int NKK = D / 32;
  constexpr int NJ = D / 16;
  auto& s_cum = lds.cum;
  auto& s_tail = lds.tail;
  auto& s_wave_units = lds.wave_units;
  auto& s_ktile = lds.ktile;
  auto& s_vtile = lds.vtile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nthreads = blockDim.x;
  const int col = lane & 15, grp = lane >> 4;
  const int B = (int)p.B;

  // ---- fused write: workgroup w writes new rows w, w + nblocks, ... to
  // their pool rows (the host checks that they fit in kCopyRegs chunks per
  // thread).  The rows are loaded here (their addresses do not depend on the
  // slots) and stored when the workgroup's stream is done, so neither waits.
  // No position this kernel reads is a written row (each is a sequence's
  // last position, whose key the kernel takes from the new rows), so the
  // stores need no ordering against the loads.
  u32x4 cpk[kCopyRegs], cpv[kCopyRegs];
  int64_t cpd[kCopyRegs];  // byte offset of the chunk in the pools, or -1
  if (p.n_new > 0) {
    const int64_t row_bytes = (int64_t)p.Hkv * D * ESZ;
    const int rc = (int)(row_bytes / 16);
#pragma unroll
    for (int i = 0; i < kCopyRegs; ++i) {
      const int f = tid + i * nthreads, k = f / rc, c = f - k * rc;
      const int64_t t = block + (int64_t)k * nblocks;
      cpd[i] = -1;
      if (t < p.n_new) {
        const int64_t slot = p.new_slots[t];
        cpk[i] = ((const u32x4*)((const char*)p.new_k + t * row_bytes))[c];
        cpv[i] = ((const u32x4*)((const char*)p.new_v + t * row_bytes))[c];
        cpd[i] = slot >= 0 ? slot * row_bytes + 16 * c : -1;
      }
    }
  }
  auto finish_copy = [&]() {
    if (p.n_new == 0) return;
#pragma unroll
    for (int i = 0; i < kCopyRegs; ++i)
      if (cpd[i] >= 0) {
        *(u32x4*)((char*)const_cast<void*>(p.key_pool) + cpd[i]) = cpk[i];
        *(u32x4*)((char*)const_cast<void*>(p.value_pool) + cpd[i]) = cpv[i];
      }
  };

  // ---- units before each sequence: a scan of each thread's run of
  // sequences, inclusive within the wave by lane shuffles, then over the wave
  // totals (one barrier).  The thread whose run holds the workgroup's first
  // unit also publishes that sequence.
  // parts: R groups of wpg waves per workgroup, group gi running part wg
  const int wpg = decode_waves(p.Hkv);
  const int R = (nthreads >> 6) / wpg;
  const int gi = wave / wpg, wig = wave - gi * wpg;
  const int W = p.grid_parts;
  int32_t U;
  {
    const int per = (B + nthreads - 1) / nthreads;
    const int b_lo = tid * per;
    int32_t run = 0;
    int64_t len;
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b < B) run += seq_units(p, b, len);
    }
    int32_t x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave_units[wave] = x;
    __syncthreads();
    int32_t acc_units = x - run;
    U = 0;
    for (int w = 0; w < (nthreads >> 6); ++w) {
      const int32_t t = s_wave_units[w];
      acc_units += w < wave ? t : 0;
      U += t;
    }
    if (tid == 0) s_cum[0] = 0;
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b < B) {
        const int32_t n = seq_units(p, b, len);
        // len = prefix_len + 32 (n - 1) + tail with tail in [1, 32]
        s_tail[b] = (uint8_t)(n > 0 ? len - p.prefix_len - (int64_t)kUnit * (n - 1) : 0);
        acc_units += n;
        s_cum[b + 1] = acc_units;
      }
    }
    __syncthreads();
  }
  if (block == 0)
    for (int b = tid; b <= B; b += nthreads) p.ws_cum[b] = s_cum[b];
  // waves past the R groups (a workgroup of more waves than its groups use,
  // as in the shared-prefix kernel) only took part in the scan
  if (gi >= R) {
    finish_copy();
    return;
  }
  // (the wave totals come through LDS: keep the range in scalar registers)
  U = (int32_t)__builtin_amdgcn_readfirstlane(U);
  if (U == 0) {
    finish_copy();
    return;
  }
  const Partition part(U, W);
  const int rounds = W / ((int)nblocks * R);
  const int g0 = ((int)block * R + gi) * rounds;  // the group's first part
  const int32_t u0 = (int32_t)__builtin_amdgcn_readfirstlane(part.start(g0));
  const int32_t u1 = (int32_t)__builtin_amdgcn_readfirstlane(part.start(g0 + rounds));
  if (u0 >= u1) {
    finish_copy();
    return;
  }
  auto part_end = [&](int w) { return (int32_t)__builtin_amdgcn_readfirstlane(part.start(w + 1)); };

  const int hpw = decode_heads_per_wave(p.Hkv);
  const uint32_t row_stride = (uint32_t)p.Hkv * D * ESZ;
  const int64_t page_stride = (int64_t)row_stride * kPageSize;
  const uint32_t page_bytes = (uint32_t)page_stride;
  const int64_t base = p.prefix_len;  // unit j of b covers positions base + 32 j ..
  LaneOffsets off;
  {
    using G = KGeom<ESZ, D>;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      off.k[i] = (uint32_t)((i % G::IPP) * G::RPI + lane / G::LPR) * row_stride + 16 * (lane % G::LPR);
  }
  __bf16* const ktile = s_ktile[wave];
  __bf16* const vtile = s_vtile[wave];

  // ---- the wave's stream (all of it wave-uniform)
  auto uniform = [](int32_t v) { return (int32_t)__builtin_amdgcn_readfirstlane(v); };
  auto seq_len = [&](int b) {  // from the scan's tables
    const int32_t n = uniform(s_cum[b + 1] - s_cum[b]), t = uniform(s_tail[b]);
    return base + (int64_t)kUnit * (n - 1) + t;
  };
  // the segment that starts at unit u of the group's range (u in part w or a
  // later one): the sequence holding u is the last b with cum[b] <= u, as
  // empty sequences share their cum with the next one
  auto segment_at = [&](int32_t u, int b, int w) {
    while (part_end(w) <= u) ++w;
    while (uniform(s_cum[b + 1]) <= u) ++b;
    const int32_t cb = uniform(s_cum[b]), ce = uniform(s_cum[b + 1]);
    const int32_t j = uniform(u - cb);
    return StreamPos{b, 0, j, j, uniform(min(part_end(w), ce) - cb), w};
  };
  auto advance = [&](StreamPos c) {
    if (c.b < 0) return c;
    if (++c.j < c.j1) return c;
    if (c.hk + 1 < hpw && wig + (c.hk + 1) * wpg < p.Hkv) {  // next head of the segment
      ++c.hk;
      c.j = c.j0;
      return c;
    }
    const int32_t u = uniform(s_cum[c.b]) + c.j1;  // the next segment's first unit
    if (u >= u1) {
      c.b = -1;
      return c;
    }
    return segment_at(u, c.b, c.w);
  };
  auto same_run = [](const StreamPos& a, const StreamPos& c) { return a.b == c.b && a.hk == c.hk && a.w == c.w; };
  // wave-uniform reads of metadata the kernel never writes, as scalar loads
  using c64p = const __attribute__((address_space(4))) int64_t*;
  using cf32p = const __attribute__((address_space(4))) float*;
  auto q_row_of = [&](int b) { return ((c64p)p.qsl)[b]; };
  auto run_scales = [&](int h, float& ls, float& os) {
    ls = p.scale * kLog2e;
    os = 1.0f;
    if constexpr (ESZ == 1) {
      ls *= ((cf32p)p.k_scale)[h];
      os = ((cf32p)p.v_scale)[h];
    }
  };
  auto bt_row = [&](int b) {
    return (const __attribute__((address_space(4))) int64_t*)(p.block_table + (int64_t)b * p.max_blocks +
                                                               base / kPageSize);
  };
  auto last_page = [&](int64_t L) { return ((L + 15) >> 4) - 1 - base / kPageSize; };
  auto pages_of = [&](const StreamPos& c, int64_t L) {
    if (c.b < 0) return UnitPages{0, 0};
    return unit_pages(bt_row(c.b), c.j, last_page(L));
  };
  auto head_of = [&](const StreamPos& c) { return wig + c.hk * wpg; };
  auto krsrc = [&](int h, int64_t pg) {
    return page_rsrc((const char*)p.key_pool + (int64_t)h * D * ESZ + pg * page_stride, page_bytes);
  };
  auto vrsrc = [&](int h, int64_t pg) {
    return page_rsrc((const char*)p.value_pool + (int64_t)h * D * ESZ + pg * page_stride, page_bytes);
  };
  // query operand of (row q_row, KV head h): head col of the group (zero for padding columns)
  auto load_q = [&](bf16x8(&qb)[NKK], int64_t q_row, int h) {
    const __bf16* qrow = (const __bf16*)p.q + (q_row * p.Hq + h * p.G + col) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (col < p.G) x = *(const u32x4*)(qrow + 32 * kk + 8 * grp);
      qb[kk] = __builtin_bit_cast(bf16x8, x);
    }
  };

  // fused write: the new key of the run's sequence (its query row's K and V
  // rows of the run's head), for the run's last unit
  u32x4 nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
  auto load_new = [&](int64_t q_row, int h) {
    constexpr int NCH = D * ESZ / 16;
    if (p.n_new > 0 && lane < NCH) {
      const int64_t off = (q_row * p.Hkv + h) * (int64_t)(D * ESZ) + 16 * lane;
      nk = *(const u32x4*)((const char*)p.new_k + off);
      nv = *(const u32x4*)((const char*)p.new_v + off);
    }
  };
  auto new_row_of = [&](int64_t pos0, int64_t len) {
    return p.n_new > 0 && pos0 + kUnit >= len ? (int)(len - 1 - pos0) : -1;
  };

  StreamPos c0;
  {
    // the sequence holding unit u0, by binary search over the unit counts
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (uniform(s_cum[mid]) <= u0) lo = mid; else hi = mid;
    }
    c0 = segment_at(u0, lo, g0);
  }
  int64_t L0 = seq_len(c0.b), q_row0 = q_row_of(c0.b);
  bf16x8 qb[NKK];
  load_q(qb, q_row0, head_of(c0));
  load_new(q_row0, head_of(c0));
  StreamPos c1 = advance(c0);
  int64_t L1 = same_run(c0, c1) || c1.b < 0 ? L0 : seq_len(c1.b);
  int64_t q_row1 = c1.b == c0.b || c1.b < 0 ? q_row0 : q_row_of(c1.b);
  UnitRegs<ESZ, D> u;
  {
    const UnitPages first = pages_of(c0, L0);
    const int h = head_of(c0);
    issue_k<ESZ, D>(u, krsrc(h, first.p0), krsrc(h, first.p1), off);
    issue_v<ESZ, D>(u, vrsrc(h, first.p0), vrsrc(h, first.p1), off);
  }
  UnitPages pg1 = pages_of(c1, L1);

  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  float logit_scale, out_scale;
  run_scales(head_of(c0), logit_scale, out_scale);
  // fp8 pools: the first partial that ends before the stream does is held in
  // registers (its fp16 row, max, sum and inverse scale) and stored with the
  // last one.  Partial stores made while the loads stream slow the stream far
  // more than their bytes would; that shows on long fp8 sequences split into
  // several parts per group.  The bf16 kernel has little register room, and
  // holding a partial there measured no gain on the bf16 decode workload.
  constexpr bool kHold = ESZ == 1;
  u32x2 hacc[kHold ? NJ : 1];
  float hm = 0.f, hl = 0.f, hu = 0.f;
  int64_t hslot = -1;  // the held partial's slot for the wave's first query head, or -1

  while (true) {
    // the unit after c1 (page ids fetched below, loads issued while c1 is computed)
    const StreamPos c2 = advance(c1);
    const int64_t L2 = c2.b == c1.b || c2.b < 0 ? L1 : seq_len(c2.b);
    const int64_t q_row2 = c2.b == c1.b || c2.b < 0 ? q_row1 : q_row_of(c2.b);
    const bool run_ends = !same_run(c0, c1);

    const int h0 = head_of(c0);
    const int h1 = head_of(c1);
    const int64_t pos0 = base + (int64_t)c0.j * kUnit;
    consume_unit<ESZ, D>(u, ktile, vtile, qb, acc, m_run, l_run, logit_scale, pos0, L0, lane, new_row_of(pos0, L0),
                         nk, nv, [&] {
                           if (c1.b >= 0) {
                             issue_k<ESZ, D>(u, krsrc(h1, pg1.p0), krsrc(h1, pg1.p1), off);
                             issue_v<ESZ, D>(u, vrsrc(h1, pg1.p0), vrsrc(h1, pg1.p1), off);
                           }
                         });
    const UnitPages pg2 = pages_of(c2, L2);

    if (run_ends) {
      // the next run's query (its latency overlaps the write-out below)
      if (c1.b >= 0) {
        load_q(qb, q_row1, head_of(c1));
        load_new(q_row1, head_of(c1));
      }
      // the four lane groups hold partial sums of the same head (same max)
      l_run += xor_shuffle(l_run, 16);
      l_run += xor_shuffle(l_run, 32);
      // (with a shared prefix, its partial joins in the merge: never whole)
      const int32_t cb = s_cum[c0.b], ce = s_cum[c0.b + 1];
      const bool whole = c0.j0 == 0 && cb + c0.j1 == ce && p.prefix_len == 0;
      const bool hold = kHold && !whole && hslot < 0 && c1.b >= 0;
      // a partial's power-of-two scale: the head's largest |value| (its 4
      // lane groups hold 32 dims each) lands in [2^14, 2^15) in fp16
      float sc = 1.f, unsc = 1.f;
      if (!whole) {
        float mx = 0.f;
#pragma unroll
        for (int t = 0; t < NJ; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[t][i]));
        mx = fmaxf(mx, xor_shuffle(mx, 16));
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        const int k = min(max(__builtin_amdgcn_frexp_expf(mx * fabsf(out_scale)), -100), 128);
        sc = out_scale * __builtin_amdgcn_ldexpf(1.f, 15 - k);
        unsc = __builtin_amdgcn_ldexpf(1.f, k - 15);
      }
      if (col < p.G) {
        const int hq = h0 * p.G + col;
        // acc[t][i] = O^T[dim 16t + 4*grp + i][head col]
        if (whole) {
          __bf16* orow = (__bf16*)p.out + (q_row0 * p.Hq + hq) * D;
#pragma unroll
          for (int t = 0; t < NJ; ++t) *(u32x2*)(orow + 16 * t + 4 * grp) = normalised(acc[t], out_scale / l_run);
        } else if (!hold) {
          const int64_t slot = ((int64_t)c0.b + c0.w) * p.Hq + hq;
          _Float16* orow = p.ws_o + slot * D;
#pragma unroll
          for (int t = 0; t < NJ; ++t) *(u32x2*)(orow + 16 * t + 4 * grp) = scaled_f16(acc[t], sc);
          if (grp == 0) *(f32x4*)(p.ws_ml + 4 * slot) = f32x4{m_run, l_run, unsc, 0.f};
        }
      }
      if constexpr (kHold) {
        if (hold) {
          hslot = ((int64_t)c0.b + c0.w) * p.Hq + h0 * p.G;
#pragma unroll
          for (int t = 0; t < NJ; ++t) hacc[t] = scaled_f16(acc[t], sc);
          hm = m_run;
          hl = l_run;
          hu = unsc;
        }
      }
      if (c1.b < 0) {
        if (kHold && hslot >= 0 && col < p.G) {
          const int64_t slot = hslot + col;
          _Float16* orow = p.ws_o + slot * D;
#pragma unroll
          for (int t = 0; t < NJ; ++t) *(u32x2*)(orow + 16 * t + 4 * grp) = hacc[t];
          if (grp == 0) *(f32x4*)(p.ws_ml + 4 * slot) = f32x4{hm, hl, hu, 0.f};
        }
        finish_copy();
        break;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
      run_scales(head_of(c1), logit_scale, out_scale);
    }
    c0 = c1;
    L0 = L1;
    q_row0 = q_row1;
    c1 = c2;
    L1 = L2;
    q_row1 = q_row2;
    pg1 = pg2;
  }
}

}  // namespace dk
}  // namespace pkv
