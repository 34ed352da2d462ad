// common.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kPageSize = 16;
constexpr float kLog2e = 1.4426950408889634f;

// element type tags
struct KvBf16 { static constexpr int bytes = 2; };
struct KvFp8 { static constexpr int bytes = 1; };

__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// elements lane * PER .. + PER - 1 of an fp16 row, widened
template <int PER>
__device__ __forceinline__ void load_f16_elems(const _Float16* row, const int lane, float (&o)[PER]) {
  if constexpr (PER == 2) {
    const f16x2 v = ((const f16x2*)row)[lane];
    o[0] = (float)v[0];
    o[1] = (float)v[1];
  } else {
    static_assert(PER == 1, "head_dim 64 or 128");
    o[0] = (float)row[lane];
  }
}

// Four OCP E4M3FN codes in one dword -> two dwords of packed bf16 (exact: every
// E4M3FN value is representable in bf16).  Uses gfx950's scaled conversion with
// a unit scale.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t codes) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace pkv
