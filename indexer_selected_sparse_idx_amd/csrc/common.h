// Shared device helpers for the gfx950 kernels: vector types, MFMA wrappers,
// number-format conversions and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int WAVE = 64;
constexpr int LATENT = 512;       // value width of a latent row
constexpr int ROPE = 64;          // rope width
constexpr int ROW = 576;          // key width of a latent row
constexpr int FP8_ROW_BYTES = 656;

// D += A * B on a 16x16 fp32 tile, K = 32 (bf16 operands).
//   a: lane l holds A[l % 16][8 * (l / 16) + 0..7]
//   b: lane l holds B[8 * (l / 16) + 0..7][l % 16]
//   d: lane l holds D[4 * (l / 16) + 0..3][l % 16]
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two OCP e4m3 codes (bytes 0,1 or 2,3 of `w`) -> two fp32 values (exact).
__device__ __forceinline__ f32x2 e4m3x2_lo(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}
__device__ __forceinline__ f32x2 e4m3x2_hi(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
}

// fp32 pair -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 4 e4m3 codes -> 4 bf16 values packed in two dwords, each multiplied by s.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w, float s) {
  f32x2 lo = e4m3x2_lo(w), hi = e4m3x2_hi(w);
  u32x2 r;
  r[0] = pack_bf16x2(lo[0] * s, lo[1] * s);
  r[1] = pack_bf16x2(hi[0] * s, hi[1] * s);
  return r;
}

// Cross-lane helpers through the LDS crossbar (no LDS memory is used).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), __builtin_bit_cast(int, v)));
}

// Order-preserving map fp32 -> uint32 (larger float => larger key); -0 and
// +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace idxs
