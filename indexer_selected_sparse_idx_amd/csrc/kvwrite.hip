// FP8 latent-cache writer on gfx950.
//
// Also writes FP8 index keys (key_fp8_write_kernel, below) and MXFP8 index
// keys (key_mxfp8_write_kernel).
//
// Quantises latent rows (576 bf16: 512 latent values, 64 rope values) into
// the packed 656-byte FP8 row the sparse attention reads: per-token tiles of
// 128 latent values, each with its own fp32 scale computed online from the
// row ("Hierarchical Quantization", KV cache bullet, in Day 0 Inference
// Support for New LLM Architectures; section 4 of Day 0 Inference Adaptation
// and Performance Optimization for New Models).  Tile j of a row gets
// scale = amax / 448 and codes E4M3FN(clamp(value / scale, -448, 448)),
// rounded to the nearest value, ties to even (the gfx950 conversion); an
// all-zero tile gets scale 0 and codes 0; the rope values are copied.
//
// Each wave takes KVW_RPW rows and issues all their loads before using any.
// Per row, lane l holds latent values 8 l .. 8 l + 7 (one 16-byte load), so
// the 16 lanes of a row of the wave cover one tile and a 16-lane max
// reduction gives its amax; each lane stores its 8 codes (8 bytes), the
// first lane of each tile its scale, and lanes 0..7 copy the rope.  The
// kernel is HBM-bound: 1152 bytes read and 656 written per row.
#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int KVW_WAVES = 4;  // waves per workgroup
constexpr int KVW_RPW = 4;    // rows per wave
constexpr int KVW_ROWS = KVW_WAVES * KVW_RPW;
constexpr float E4M3_MAX_F = 448.0f;

__device__ __forceinline__ float clamp_e4m3(float q) { return fminf(fmaxf(q, -E4M3_MAX_F), E4M3_MAX_F); }

__global__ __launch_bounds__(KVW_WAVES * WAVE) void kv_fp8_write_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * KVW_WAVES + (threadIdx.x >> 6)) * KVW_RPW;
  u32x4 w[KVW_RPW], rope[KVW_RPW];
  int dst[KVW_RPW];
#pragma unroll
  for (int j = 0; j < KVW_RPW; ++j) {
    const int r = min(r0 + j, p.n - 1);  // (rows past n: a valid row, not stored)
    const uint16_t* src = p.src + (int64_t)r * ROW;
    dst[j] = r0 + j < p.n ? p.dst_row[r] : -1;
    w[j] = *(const u32x4*)(src + 8 * lane);
    rope[j] = *(const u32x4*)(src + LATENT + 8 * (lane & 7));
  }
#pragma unroll
  for (int j = 0; j < KVW_RPW; ++j) {
    if (dst[j] < 0) continue;
    uint8_t* out = p.kv + (int64_t)dst[j] * FP8_ROW_BYTES;
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[j][e] << 16);
      x[2 * e + 1] = __uint_as_float(w[j][e] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, shfl_xor(amax, off));
    const float scale = amax / E4M3_MAX_F;  // (fp32 division, correctly rounded)
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = scale > 0.0f ? clamp_e4m3(x[i] / scale) : 0.0f;
    // two codes per conversion: word_sel false fills bytes 0-1, true bytes 2-3
    uint32_t c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)c0, true);
    uint32_t c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)c1, true);
    *(u32x2*)(out + 8 * lane) = u32x2{c0, c1};
    if ((lane & 15) == 0) *(float*)(out + LATENT + 4 * (lane >> 4)) = scale;
    if (lane < 8) *(u32x4*)(out + LATENT + 16 + 16 * lane) = rope[j];
  }
}

// Index keys: a row of D bf16 keys spans D / 8 lanes (8 keys each), so a
// wave step covers 64 / (D / 8) rows; a wave takes KW_STEPS steps, all loads
// first.  With a scale array, each row's amax comes from a max reduction over
// its lanes and the row's scale goes to scale[dst]; without, the keys are
// stored with scale 1.0.
template <int D>
__global__ __launch_bounds__(KVW_WAVES * WAVE) void key_fp8_write_kernel(KeyWriteParams p) {
  constexpr int G = D / 8;        // lanes per row
  constexpr int RPS = WAVE / G;   // rows per wave step
  constexpr int KW_STEPS = 4;
  const int lane = threadIdx.x & 63;
  const int sub = lane / G, gl = lane % G;
  const int base = (blockIdx.x * KVW_WAVES + (threadIdx.x >> 6)) * RPS * KW_STEPS;
  u32x4 w[KW_STEPS];
  int dst[KW_STEPS];
#pragma unroll
  for (int j = 0; j < KW_STEPS; ++j) {
    const int r = base + j * RPS + sub;
    const int rr = min(r, p.n - 1);  // (rows past n: a valid row, not stored)
    dst[j] = r < p.n ? p.dst_row[rr] : -1;
    w[j] = *(const u32x4*)(p.src + (int64_t)rr * D + 8 * gl);
  }
#pragma unroll
  for (int j = 0; j < KW_STEPS; ++j) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[j][e] << 16);
      x[2 * e + 1] = __uint_as_float(w[j][e] & 0xffff0000u);
    }
    float q[8];
    float scale = 1.0f;
    if (p.scale) {  // (uniform: every lane reduces)
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
      for (int off = 1; off < G; off <<= 1) amax = fmaxf(amax, shfl_xor(amax, off));
      scale = amax / E4M3_MAX_F;
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = scale > 0.0f ? clamp_e4m3(x[i] / scale) : 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = clamp_e4m3(x[i]);
    }
    if (dst[j] < 0) continue;
    uint32_t c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)c0, true);
    uint32_t c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)c1, true);
    *(u32x2*)(p.k + (int64_t)dst[j] * D + 8 * gl) = u32x2{c0, c1};
    if (p.scale && gl == 0) p.scale[dst[j]] = scale;
  }
}

// MXFP8 index keys (d_I = 128): blocks of 32 values with a shared
// power-of-two scale ("Hierarchical Quantization", index-cache bullet, in
// Day 0 Inference Support for New LLM Architectures; section 4 of Day 0
// Inference Adaptation and Performance Optimization for New Models), by the
// OCP MX rule for E4M3 elements, the rule the MXFP8 indexer applies to its
// queries: e = floor(log2(amax)) - 8 clamped to [-127, 127] (E8M0 byte
// e + 127; an all-zero block gets byte 0 and codes 0), codes
// E4M3FN(clamp(k / 2^e, -448, 448)) -- the division by a power of two is
// exact.  Lane l of a row's 16 lanes holds keys 8 l .. 8 l + 7, so a block is
// 4 lanes and its amax a 4-lane max reduction.
__global__ __launch_bounds__(KVW_WAVES * WAVE) void key_mxfp8_write_kernel(KeyMxWriteParams p) {
  constexpr int D = 128, G = D / 8, RPS = WAVE / G, KW_STEPS = 4;
  const int lane = threadIdx.x & 63;
  const int sub = lane / G, gl = lane % G;
  const int base = (blockIdx.x * KVW_WAVES + (threadIdx.x >> 6)) * RPS * KW_STEPS;
  u32x4 w[KW_STEPS];
  int dst[KW_STEPS];
#pragma unroll
  for (int j = 0; j < KW_STEPS; ++j) {
    const int r = base + j * RPS + sub;
    const int rr = min(r, p.n - 1);  // (rows past n: a valid row, not stored)
    dst[j] = r < p.n ? p.dst_row[rr] : -1;
    w[j] = *(const u32x4*)(p.src + (int64_t)rr * D + 8 * gl);
  }
#pragma unroll
  for (int j = 0; j < KW_STEPS; ++j) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[j][e] << 16);
      x[2 * e + 1] = __uint_as_float(w[j][e] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, shfl_xor(amax, 1));
    amax = fmaxf(amax, shfl_xor(amax, 2));
    // amax = m 2^E with m in [0.5, 1): floor(log2 amax) = E - 1
    const int e = amax > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(amax) - 1 - 8, -127), 127) : -127;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = amax > 0.0f ? clamp_e4m3(__builtin_amdgcn_ldexpf(x[i], -e)) : 0.0f;
    if (dst[j] < 0) continue;
    uint32_t c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)c0, true);
    uint32_t c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)c1, true);
    *(u32x2*)(p.k + (int64_t)dst[j] * D + 8 * gl) = u32x2{c0, c1};
    if ((gl & 3) == 0) p.k_exp[(int64_t)dst[j] * 4 + (gl >> 2)] = (uint8_t)(amax > 0.0f ? e + 127 : 0);
  }
}

}  // namespace

hipError_t launch_key_mxfp8_write(const KeyMxWriteParams& p, hipStream_t stream) {
  constexpr int KW_STEPS = 4;
  const int rows_per_wg = KVW_WAVES * KW_STEPS * (WAVE / 16);
  hipLaunchKernelGGL(key_mxfp8_write_kernel, dim3(cdiv(p.n, rows_per_wg)), dim3(KVW_WAVES * WAVE), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_key_fp8_write(const KeyWriteParams& p, hipStream_t stream) {
  constexpr int KW_STEPS = 4;
  const int rows_per_wg = KVW_WAVES * KW_STEPS * (WAVE / (p.d == 64 ? 8 : 16));
  const dim3 grid(cdiv(p.n, rows_per_wg)), block(KVW_WAVES * WAVE);
  if (p.d == 64) hipLaunchKernelGGL(key_fp8_write_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(key_fp8_write_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_fp8_write(const KvWriteParams& p, hipStream_t stream) {
  const TimerEvents t = timer_take(4);
  return launch_kernel(kv_fp8_write_kernel, dim3(cdiv(p.n, KVW_ROWS)), dim3(KVW_WAVES * WAVE), stream, t.start,
                       t.stop, p);
}

}  // namespace idxs
