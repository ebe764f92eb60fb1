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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
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
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);  // -0 -> +0; every other value unchanged
  // negative: every bit flipped; otherwise: the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding; the
// 6-bit vmcnt saturates at 63, and waiting for fewer is always safe).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Global memory straight into LDS (global_load_lds): 16 bytes per lane land
// at lds_addr + 16 * lane (dma4: 4 bytes at lds_addr + 4 * lane); lds_addr is
// wave-uniform.  dma16_s takes a wave-uniform base address
// (SGPRs) and a 32-bit per-lane byte offset.  Written as inline asm so that the
// compiler does not turn later LDS reads of other ring slots into waits for
// every outstanding gather: completion is tracked with wait_vmcnt().
__device__ __forceinline__ void dma16(const uint8_t* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_s(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
  // (the base goes through readfirstlane as well: where the compiler cannot
  // prove it uniform it would otherwise hand the asm a VGPR pair)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t bs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"((const uint8_t*)(uintptr_t)bs), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace idxs
