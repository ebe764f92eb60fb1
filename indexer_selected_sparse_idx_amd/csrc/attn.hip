// Sparse latent attention on gfx950.
//
// For each query token and head, over the selected positions s:
//   l_s = scale * (q[h, :] . c[s, 0:576]),  O[h, :] = sum_s softmax(l)_s c[s, 0:512]
// (the sparse attention core reads the KV entries at the selected indices
// and attends over them in blocks: "Index-Based Sparse Attention" in Day 0
// Inference Support for New LLM Architectures, section 3 of Day 0 Inference
// Acceleration for New LLM Architectures; one latent row shared by every
// head, MLA: section 1 of Day 0 Inference Adaptation and Performance
// Optimization for New Models).
//
// Work item: (token, split of the index list), every head of the token.  The
// workgroup has one wave per 32 heads.  The valid entries of the split are
// resolved to cache rows (block table included) and compacted into LDS, so
// entries that select nothing (-1, or past the context) cost no tile.  The
// selected latent rows are gathered 32 per tile into LDS, shared by all the
// waves, and each wave runs with its 32 heads on the MFMA N dimension
// (v_mfma_f32_32x32x16_bf16):
//   S^T[32 keys x 32 heads] = C_tile . Q^T   (keys on M, 36 k-steps over 576)
//   online softmax in fp32 registers (a lane holds 16 keys of one head; the
//   other 16 sit in lane ^ 32)
//   O^T[512 x 32 heads]   += V^T . P^T       (dv on M, 16 tiles of 32)
// The S^T accumulator is already the B operand of the second product once
// the key order inside its contraction is permuted to match (k-step kk takes
// accumulator registers 8 kk .. 8 kk + 7); the V^T operand is read from the
// key-major tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16),
// so each row is stored once.  Q^T stays in registers for the whole split and
// O^T in the accumulation registers.
//
// bf16 rows go from HBM straight into LDS (global_load_lds_dwordx4, one wave
// instruction per 1 KiB latent row) through a 4-deep ring with one barrier per
// tile, and the loop is software-pipelined: iteration k runs S of tile k
// with the gathers of tile k + 2 spread over its k-steps, then P.V of tile
// k - 1 with the softmax of tile k in the shadow of those MFMAs.  FP8 rows
// (656 bytes) go into a raw LDS ring the same way, each wave gathering whole
// rows of its own and dequantising them into the tile layout.  Splits
// (decode occupancy) are merged by combine_kernel.
//
// Products run in fp16: every wave converts the bf16 latent values its own
// gathers brought into LDS to fp16 in place (exact for |x| in [2^-14,
// 65504]; below that the absolute error is at most 2^-25), FP8 rows are
// dequantised to fp16, the queries' latent part is converted once, and the
// softmax numerators P go into the P.V product as fp16 (11 significant bits,
// where bf16 carries 8).  The rope part of S (4 of its 36 k-steps) stays in
// bf16 on both operands.  A value beyond the fp16 range makes the split's
// softmax sum or maximum non-finite, and a head whose whole output is below
// 2^-14 was computed from subnormal fp16 values; in both cases the
// workgroup recomputes the split with bf16 operands (and, for bf16 rows, P
// split into two bf16 parts, hi + lo, so the product runs twice on each V^T
// operand).
#include <math.h>

#include <algorithm>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TILE = ATTN_TILE;                 // selected rows per tile
constexpr int HPW = 32;                         // heads per wave
constexpr int LAT_STRIDE = 1024 + 64;           // 512 bf16 per row, padded by four 16-byte chunks
constexpr int LAT_TILE_BYTES = TILE * LAT_STRIDE;
constexpr int ROPE_TILE_BYTES = TILE * 128;     // 64 bf16 per row
constexpr int BUF_BYTES = LAT_TILE_BYTES + ROPE_TILE_BYTES;
constexpr int ROW_CHUNKS = FP8_ROW_BYTES / 16;   // 41 16-byte chunks of a packed FP8 row
constexpr int KSTEPS = ROW / 16;                // 36 k-steps of the S product
constexpr int LAT_KSTEPS = LATENT / 16;         // the first 32 cover the latent dims, the last 4 the rope
constexpr int DV_TILES = LATENT / 32;           // 16 dv tiles of the P.V product
constexpr float MAX_GROWTH = 64.0f;             // log2 growth of the max over the softmax reference tolerated
constexpr float LN2 = 0.69314718055994530942f;

constexpr float MAX_GROWTH_F16 = 15.0f;         // ... when P is fp16 (p <= 2^15 < 65504)
constexpr uint32_t RUN_GROWTH = 1u, RUN_NONFINITE = 2u;  // redo reasons

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// D += A * B on a 32x32 fp32 tile, K = 16 (fp16 operands when F16, else
// bf16; operands are passed as their raw 16-bit patterns).
//   a: lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   b: lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   d: register 4 i + j of lane l holds D[8 i + 4 * (l / 32) + j][l % 32]
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Two values as raw fp16 (or bf16) bits, round to nearest even.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// A dword of two bf16 values -> the same two values as fp16 (exact inside
// the fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack2<true>(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
}

// O^T accumulation: the same MFMA written as inline asm with the accumulator
// tied to AGPRs ("+a"), so the 256 registers of O^T stay in the accumulation
// file while the builtin MFMAs (this file is built with VGPR-form MFMAs) keep
// S^T in VGPRs.  The compiler does not see these as MFMAs, so the hazards it
// would otherwise pad are handled here: NOP_B adds the wait state needed when
// b was just written by a VALU instruction; back-to-back MFMAs accumulating
// into the same registers need none; o_fence() must separate the last of them
// from any other access to the accumulators.
template <bool F16, bool NOP_B>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (F16) {
    if (NOP_B)
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
      asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  } else {
    if (NOP_B)
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
}

// max / sum of v over lanes l and l ^ 32 (both lanes get the result).
// (v_permlane32_swap would do the exchange without the LDS crossbar, but the
// compiler folds the builtin's two results into one when both inputs are
// the same value.)
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, shfl_xor(v, 32)); }
__device__ __forceinline__ float pair_sum(float v) { return v + shfl_xor(v, 32); }

// LDS addresses of 16-byte chunk `ch` of tile row r.  The LDS has 64 banks
// of 4 bytes; a 128-bit read serves 16 lanes per cycle, a 64-bit transposing
// read 32.  Latent rows are padded to 68 chunks, so row r starts 4 r chunks
// into the 16-chunk bank window, and the two low bits of the chunk index are
// XOR-ed with bits 2-3 of the row.  Then
//   - 16 consecutive rows at one chunk (the S operand read) and
//   - 4 rows (4 m .. 4 m + 3) x 4 consecutive aligned chunks (the V^T
//     operand read of 32 lanes)
// each cover all 64 banks, and every per-lane address stays affine in the
// chunk index above bit 1 and in the row above bit 3 (immediate offsets).
// Rope rows (8 chunks) are XOR-swizzled with bits 1-3 of the row, so 16
// consecutive rows at one chunk cover the banks too.
__device__ __forceinline__ int lat_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int lat_off(int r, int ch) { return r * LAT_STRIDE + ((ch ^ lat_swz(r)) << 4); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int rope_off(int r, int ch) { return LAT_TILE_BYTES + r * 128 + ((ch ^ rope_swz(r)) << 4); }

// Per-wave state: Q^T operand (k-step ks: lane holds Q[head][16 ks + 8 h .. +8],
// h = lane / 32), the O^T accumulator (register 4 i + j of tile nt holds
// O^T[32 nt + 8 i + 4 h + j][head]) and the softmax state of the lane's head.
//
// The softmax runs against a fixed reference m_ref per head (the maximum of
// the first tile, base 2), so O^T never needs rescaling: p = 2^(x - m_ref)
// and O = sum p v / sum p is exact for any reference as long as nothing
// overflows.  m_max tracks the true maximum; if it outgrows the reference by
// more than MAX_GROWTH (p could then overflow), the workgroup recomputes the
// split with m_ref = m_max.
struct WaveAcc {
  u32x4 qb[KSTEPS];  // raw bf16 or fp16 bits
  f32x16 o[DV_TILES];
  float m_ref, m_max, l_run;
};

// Q^T operand of the lane's head, the stored bf16 bits (convert_q<true>
// turns them into fp16 once they have landed).
__device__ __forceinline__ void load_q(WaveAcc& a, const AttnParams& p, int tok, int head, bool head_ok, int h) {
  const uint16_t* qrow = p.q + ((int64_t)tok * p.H + (head_ok ? head : 0)) * ROW + h * 8;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (head_ok) v = *(const u32x4*)(qrow + ks * 16);
    a.qb[ks] = v;
  }
}
// (the latent k-steps only: the rope part of S stays bf16 on both sides)
template <bool F16>
__device__ __forceinline__ void convert_q(WaveAcc& a) {
  if constexpr (F16) {
#pragma unroll
    for (int ks = 0; ks < LAT_KSTEPS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) a.qb[ks][j] = bf16x2_to_f16x2(a.qb[ks][j]);
  }
}

// The 16 bytes at p (8 bf16 values) as fp16, in place.
__device__ __forceinline__ void bf16x8_to_f16_lds(uint8_t* p) {
  const u32x4 v = *(const u32x4*)p;
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = bf16x2_to_f16x2(v[j]);
  *(u32x4*)p = r;
}

// Start (or restart) the accumulation; m_ref < -FLT_MAX means "take the
// reference from the first tile".
// Wait states after the last accumulating MFMA before the accumulators are
// read or overwritten (the 32x32x16 result latency, with margin).
__device__ __forceinline__ void o_fence(WaveAcc& a) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7"
               : "+a"(a.o[0]), "+a"(a.o[1]), "+a"(a.o[2]), "+a"(a.o[3]), "+a"(a.o[4]), "+a"(a.o[5]),
                 "+a"(a.o[6]), "+a"(a.o[7]), "+a"(a.o[8]), "+a"(a.o[9]), "+a"(a.o[10]), "+a"(a.o[11]),
                 "+a"(a.o[12]), "+a"(a.o[13]), "+a"(a.o[14]), "+a"(a.o[15]));
}

__device__ __forceinline__ void reset_acc(WaveAcc& a, float m_ref) {
#pragma unroll
  for (int nt = 0; nt < DV_TILES; ++nt) a.o[nt] = f32x16{};
  a.m_ref = m_ref;
  a.m_max = -INFINITY;
  a.l_run = 0.0f;
}

// Per-lane LDS byte offsets inside a tile buffer.
struct TileAddr {
  int s_lat[2];   // S operand, latent k-step ks: s_lat[ks & 1] + 64 (ks >> 1)
  int s_rope[4];  // S operand, rope k-steps 32 .. 35
  int v[2];       // V^T operand, read r of k-step kk, dv tile nt: v[r] + 16 kk LAT_STRIDE + 64 nt
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, col = lane & 31;
    // k-step ks reads chunk 2 ks + h of row col; the swizzle only touches
    // the two low chunk bits (h and the parity of ks)
    s_lat[0] = lat_off(col, h);
    s_lat[1] = lat_off(col, 2 + h);
#pragma unroll
    for (int j = 0; j < 4; ++j) s_rope[j] = rope_off(col, 2 * j + h);
    // transposing read: 16-lane group G = lane / 16 reads keys 16 kk + 8 r +
    // 4 h + 0..3 (h = G / 2) at dv 32 nt + 16 (G % 2) + 0..15; lane k of the
    // group addresses key + k / 4, dv + 4 (k % 4)
    const int G = lane >> 4, k = lane & 15;
    const int hh = G >> 1, dvhalf = G & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r) v[r] = lat_off(8 * r + 4 * hh + (k >> 2), 2 * dvhalf + ((k & 3) >> 1)) + 8 * (k & 1);
  }
};

__device__ __forceinline__ u32x4 s_operand(const uint8_t* buf, const TileAddr& ad, int ks) {
  return *(const u32x4*)(buf + (ks < 32 ? ad.s_lat[ks & 1] + (ks >> 1) * 64 : ad.s_rope[ks - 32]));
}

__device__ __forceinline__ u32x4 v_operand(const uint8_t* buf, const TileAddr& ad, int nt, int kk) {
  const int off = kk * 16 * LAT_STRIDE + nt * 64;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + ad.v[0] + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + ad.v[1] + off));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T[32 keys x 32 heads] of one tile.  The operand of k-step ks + SPRE is
// read from LDS while the MFMA of k-step ks runs; the scheduling fences keep
// that order (left alone, the scheduler serialises read -> wait -> MFMA).
constexpr int SPRE = 3;

// at_step(std::integral_constant<int, ks>) runs after the MFMA of k-step ks
// is issued (the gathers of a later tile are spread over the k-steps this
// way).  The k-steps are expanded at compile time so that at_step sees a
// constant.
template <bool F16, int KS, typename F>
__device__ __forceinline__ void s_step(f32x16& acc, u32x4 (&op)[SPRE], const WaveAcc& a, const uint8_t* buf,
                                       const TileAddr& ad, F& at_step) {
  acc = mfma32<F16 && (KS < LAT_KSTEPS)>(op[KS % SPRE], a.qb[KS], acc);
  if constexpr (KS + SPRE < KSTEPS) op[KS % SPRE] = s_operand(buf, ad, KS + SPRE);
  at_step(std::integral_constant<int, KS>());
  __builtin_amdgcn_sched_barrier(0);
}

template <bool F16, typename F, int... KS>
__device__ __forceinline__ f32x16 s_steps(const WaveAcc& a, const uint8_t* buf, const TileAddr& ad, F& at_step,
                                          std::integer_sequence<int, KS...>) {
  f32x16 acc = {};
  u32x4 op[SPRE];
#pragma unroll
  for (int j = 0; j < SPRE; ++j) op[j] = s_operand(buf, ad, j);
  (s_step<F16, KS>(acc, op, a, buf, ad, at_step), ...);
  return acc;
}

template <bool F16, typename F>
__device__ __forceinline__ f32x16 s_phase(const WaveAcc& a, const uint8_t* buf, const TileAddr& ad, F&& at_step) {
  return s_steps<F16>(a, buf, ad, at_step, std::make_integer_sequence<int, KSTEPS>());
}

struct NoStep {
  template <int KS>
  __device__ __forceinline__ void operator()(std::integral_constant<int, KS>) const {}
};

// Why the workgroup must recompute the split, OR-ed over its waves:
// RUN_GROWTH when some head outgrew its reference (by more than max_growth,
// base 2), RUN_NONFINITE when some softmax sum or maximum is not finite (an
// operand outside the fp16 range).  `flags` is one int per wave in LDS that
// no wave reads or writes at this point.
template <int NW>
__device__ __forceinline__ uint32_t redo_reasons(const WaveAcc& a, float max_growth, int* flags, int wave, int lane) {
  const bool grew = __builtin_amdgcn_ballot_w64(a.m_max > a.m_ref + max_growth) != 0;
  // A non-finite operand gives a NaN or infinite score: a NaN or +inf one
  // reaches the softmax sum or the maximum.  (A -inf one gets p = 0, but 0
  // times the infinite value makes O NaN: write_result reports that.)
  const bool bad = __builtin_amdgcn_ballot_w64(
                       !__builtin_isfinite(a.l_run) ||
                       (a.l_run > 0.0f && !(__builtin_isfinite(a.m_max) && __builtin_isfinite(a.m_ref)))) != 0;
  __syncthreads();
  if (lane == 0) flags[wave] = (grew ? RUN_GROWTH : 0u) | (bad ? RUN_NONFINITE : 0u);
  __syncthreads();
  uint32_t any = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) any |= (uint32_t)flags[j];
  return any;
}

// true when `mine` holds in some lane of the workgroup (flags as above)
template <int NW>
__device__ __forceinline__ bool any_lane(bool mine, int* flags, int wave, int lane) {
  const bool w = __builtin_amdgcn_ballot_w64(mine) != 0;
  __syncthreads();
  if (lane == 0) flags[wave] = w ? 1 : 0;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) any |= flags[j];
  return any != 0;
}

// P^T operand of a tile (k-step kk takes p values 8 kk .. 8 kk + 7): fp16,
// or bf16.  With SPLITP (bf16 only), P = P_hi + P_lo, both bf16: the product
// then runs twice on the same V^T operand, so P carries ~16 mantissa bits
// instead of 8.
struct POp {
  u32x4 hi[2], lo[2];
};

// Softmax numerators of one S^T tile (base 2) against the reference, the
// first nv keys of the tile valid, in 16 stages: stage st can run after dv
// tile st of the previous tile's P.V MFMAs, whose shadow then hides the VALU
// work.  The scale is positive, so the maximum is taken over the raw scores
// and p = 2^(scale * x - m_ref) is one FMA and one exp2 per key.
//   0-3    mask invalid keys to -inf (partial tiles only), running maximum
//   4      start the exchange of the maximum with lane ^ 32 (same head)
//   6      reference (first tile) and running maximum
//   7-12   p and its sum
//   13     running sum
//   14-15  pack P^T (k-steps 0 and 1)
template <bool F16, bool SPLITP>
struct SoftmaxTile {
  static_assert(!(F16 && SPLITP), "P is split only in bf16");
  float x[16];
  float tmax, other, psum;
  POp op;

  __device__ __forceinline__ explicit SoftmaxTile(const f32x16& s) : tmax(-INFINITY), other(-INFINITY), psum(0.0f) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = s[j];
  }

  template <int ST>
  __device__ __forceinline__ void stage(WaveAcc& a, int nv, float scale_log2, int h) {
    if constexpr (ST < 4) {
      if (nv < TILE) {  // (uniform: only the last tile of a split is partial)
#pragma unroll
        for (int j = 4 * ST; j < 4 * ST + 4; ++j) {
          const int key = 8 * (j >> 2) + 4 * h + (j & 3);
          x[j] = key < nv ? x[j] : -INFINITY;
        }
      }
#pragma unroll
      for (int j = 4 * ST; j < 4 * ST + 4; ++j) tmax = fmaxf(tmax, x[j]);
    } else if constexpr (ST == 4) {
      other = shfl_xor(tmax, 32);
    } else if constexpr (ST == 6) {
      const float m = fmaxf(tmax, other) * scale_log2;
      if (a.m_ref == -INFINITY) a.m_ref = m == -INFINITY ? 0.0f : m;
      a.m_max = fmaxf(a.m_max, m);
    } else if constexpr (ST >= 7 && ST < 13) {
      constexpr int j0 = ST < 11 ? 3 * (ST - 7) : 12 + 2 * (ST - 11);
      constexpr int j1 = ST < 11 ? j0 + 3 : j0 + 2;
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], scale_log2, -a.m_ref));
        psum += x[j];
      }
    } else if constexpr (ST == 13) {
      a.l_run += psum;
    } else if constexpr (ST >= 14) {
      constexpr int kk = ST - 14;
      u32x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = x[8 * kk + 2 * j], p1 = x[8 * kk + 2 * j + 1];
        const uint32_t hw = pack2<F16>(p0, p1);
        hi[j] = hw;
        if (SPLITP) {
          const float h0 = __builtin_bit_cast(float, hw << 16), h1 = __builtin_bit_cast(float, hw & 0xffff0000u);
          lo[j] = pack2<false>(p0 - h0, p1 - h1);
        } else {
          lo[j] = 0u;
        }
      }
      op.hi[kk] = hi;
      op.lo[kk] = lo;
    }
  }

  template <int... ST>
  __device__ __forceinline__ void stages(WaveAcc& a, int nv, float scale_log2, int h,
                                         std::integer_sequence<int, ST...>) {
    (stage<ST>(a, nv, scale_log2, h), ...);
  }
  // every stage in order (no P.V to hide behind)
  __device__ __forceinline__ void run_all(WaveAcc& a, int nv, float scale_log2, int h) {
    stages(a, nv, scale_log2, h, std::make_integer_sequence<int, 16>());
  }
};

// O^T += V^T . P^T over the 16 dv tiles.  The operands of dv tile nt + VPRE
// are read while the MFMAs of tile nt run; between its two MFMAs at_step(nt)
// runs (the softmax stages of the next tile).
// The first MFMAs wait one state in case P was just written by VALU
// instructions.
constexpr int VPRE = 1;

template <bool F16, bool SPLITP, int NT, typename F>
__device__ __forceinline__ void v_step(WaveAcc& a, const uint8_t* buf, const TileAddr& ad, const POp& op,
                                       u32x4 (&v)[VPRE + 1][2], F& at_step) {
  constexpr int c = NT % (VPRE + 1);
  if constexpr (NT + VPRE < DV_TILES) {
    v[(NT + VPRE) % (VPRE + 1)][0] = v_operand(buf, ad, NT + VPRE, 0);
    v[(NT + VPRE) % (VPRE + 1)][1] = v_operand(buf, ad, NT + VPRE, 1);
  }
  constexpr bool NOP = NT == 0;
  // at_step(nt) goes between the tile's MFMAs: the wave issues in order, so
  // VALU work hides under an MFMA only when it sits between two of them
  mfma32_acc<F16, NOP>(a.o[NT], v[c][0], op.hi[0]);
  __builtin_amdgcn_sched_barrier(0);
  at_step(std::integral_constant<int, NT>());
  __builtin_amdgcn_sched_barrier(0);
  mfma32_acc<F16, NOP>(a.o[NT], v[c][1], op.hi[1]);
  if (SPLITP) {
    mfma32_acc<F16, NOP>(a.o[NT], v[c][0], op.lo[0]);
    mfma32_acc<F16, NOP>(a.o[NT], v[c][1], op.lo[1]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <bool F16, bool SPLITP, typename F, int... NT>
__device__ __forceinline__ void v_steps(WaveAcc& a, const uint8_t* buf, const TileAddr& ad, const POp& op,
                                        F& at_step, std::integer_sequence<int, NT...>) {
  u32x4 v[VPRE + 1][2];
#pragma unroll
  for (int j = 0; j < VPRE; ++j) {
    v[j][0] = v_operand(buf, ad, j, 0);
    v[j][1] = v_operand(buf, ad, j, 1);
  }
  (v_step<F16, SPLITP, NT>(a, buf, ad, op, v, at_step), ...);
}

template <bool F16, bool SPLITP, typename F>
__device__ __forceinline__ void v_phase(WaveAcc& a, const uint8_t* buf, const TileAddr& ad, const POp& op,
                                        F&& at_step) {
  v_steps<F16, SPLITP>(a, buf, ad, op, at_step, std::make_integer_sequence<int, DV_TILES>());
}

// Normalise and store the wave's O^T (and lse) for its 32 heads.  A split's
// partial O goes out as fp16 times a power-of-two scale per (token, split,
// head): the head's largest |O| is brought just below 2^15, so every value
// keeps 11 significant bits relative to that maximum (the split weights of
// the merge are at most 1), at half the bytes of fp32 partials.
// Returns false when the fp16 run's result must be recomputed in bf16 (the
// caller then writes again): some O value of the lane is not finite (a NaN
// from an operand outside the fp16 range), or, with tiny_check, the head's
// output is nonzero but below 2^-14 everywhere (its values came from fp16
// subnormals, whose absolute spacing of 2^-24 is no longer small against
// them; a whole output tensor that small would miss the tolerance).
constexpr float TINY_OUT = 0x1p-14f;

__device__ __forceinline__ bool write_result(const WaveAcc& a, const AttnParams& p, int tok, int split, int head,
                                             bool head_ok, int h, bool tiny_check) {
  const float l_tot = pair_sum(a.l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (a.m_ref + __builtin_amdgcn_logf(l_tot)) * LN2 : -INFINITY;
  float osum = 0.0f;
  float amax = 0.0f;
  if (p.num_splits == 1) {
    float* orow = p.out + ((int64_t)tok * p.H + (head_ok ? head : 0)) * LATENT;
#pragma unroll
    for (int nt = 0; nt < DV_TILES; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = {a.o[nt][4 * i], a.o[nt][4 * i + 1], a.o[nt][4 * i + 2], a.o[nt][4 * i + 3]};
        osum += (v[0] + v[1]) + (v[2] + v[3]);
        if (tiny_check) amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        if (head_ok) *(f32x4*)(orow + nt * 32 + i * 8 + h * 4) = v * inv;
      }
    if (head_ok && h == 0 && p.lse) p.lse[(int64_t)tok * p.H + head] = lse_v;
    amax = pair_max(amax) * inv;
    return __builtin_isfinite(osum) && !(tiny_check && head_ok && amax > 0.0f && amax < TINY_OUT);
  }
#pragma unroll
  for (int nt = 0; nt < DV_TILES; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      amax = fmaxf(amax, fabsf(a.o[nt][r]));
      osum += a.o[nt][r];
    }
  amax = pair_max(amax) * inv;
  const bool tiny = tiny_check && head_ok && amax > 0.0f && amax < TINY_OUT;
  // amax < 2^e; exponents below -100 are raised so the factor stays finite
  const int e = amax > 0.0f ? max(__builtin_amdgcn_frexp_expf(amax), -100) : 0;
  const float f = __builtin_amdgcn_ldexpf(inv, 15 - e);
  const float sc = amax > 0.0f ? __builtin_amdgcn_ldexpf(1.0f, e - 15) : 0.0f;
  if (!head_ok) return __builtin_isfinite(osum);
  const int64_t pi = ((int64_t)tok * p.num_splits + split) * p.H + head;
  uint16_t* orow = p.part_o + pi * LATENT;
#pragma unroll
  for (int nt = 0; nt < DV_TILES; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = f32x4{a.o[nt][4 * i], a.o[nt][4 * i + 1], a.o[nt][4 * i + 2], a.o[nt][4 * i + 3]} * f;
      *(f16x4*)(orow + nt * 32 + i * 8 + h * 4) = __builtin_convertvector(v, f16x4);
    }
  if (h == 0) *(f32x2*)(p.part_ls + 2 * pi) = f32x2{lse_v, sc};
  return __builtin_isfinite(osum) && !tiny;
}

// write_result for the ring kernels, the same values through LDS: every wave
// puts its heads' rows into `stage` (free once the split's tiles are done:
// ROWS x 1040 bytes, a row of 512 fp16 or half a row of fp32 plus 16 bytes
// of padding, so that the 16 lanes of a 128-bit write hit 16 bank groups),
// and each head's row then goes to memory as one 1 KiB wave store (fp32
// output in two halves).  Stored by lane, each 16-byte piece of a row is its
// own partial-line write.  All waves of the workgroup must call it.
template <int NW>
__device__ __forceinline__ bool write_result_staged(const WaveAcc& a, const AttnParams& p, int tok, int split,
                                                    int head, bool head_ok, int h, bool tiny_check, uint8_t* stage,
                                                    int wave, int lane) {
  constexpr int ROWS = NW * HPW;
  constexpr int SROW = 1040;
  const int r = wave * HPW + (lane & 31);  // this lane's head, the stage row
  const float l_tot = pair_sum(a.l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (a.m_ref + __builtin_amdgcn_logf(l_tot)) * LN2 : -INFINITY;
  float osum = 0.0f;
  float amax = 0.0f;
  if (p.num_splits == 1) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int nt = 8 * half; nt < 8 * half + 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = {a.o[nt][4 * i], a.o[nt][4 * i + 1], a.o[nt][4 * i + 2], a.o[nt][4 * i + 3]};
          osum += (v[0] + v[1]) + (v[2] + v[3]);
          if (tiny_check) amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
          *(f32x4*)(stage + r * SROW + ((nt - 8 * half) * 32 + i * 8 + h * 4) * 4) = v * inv;
        }
      __syncthreads();
      for (int rr = wave; rr < ROWS; rr += NW)
        if (rr < p.H)
          *(f32x4*)(p.out + ((int64_t)tok * p.H + rr) * LATENT + 256 * half + 4 * lane) =
              *(const f32x4*)(stage + rr * SROW + 16 * lane);
      __syncthreads();
    }
    if (head_ok && h == 0 && p.lse) p.lse[(int64_t)tok * p.H + head] = lse_v;
    amax = pair_max(amax) * inv;
    return __builtin_isfinite(osum) && !(tiny_check && head_ok && amax > 0.0f && amax < TINY_OUT);
  }
#pragma unroll
  for (int nt = 0; nt < DV_TILES; ++nt)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      amax = fmaxf(amax, fabsf(a.o[nt][q]));
      osum += a.o[nt][q];
    }
  amax = pair_max(amax) * inv;
  const bool tiny = tiny_check && head_ok && amax > 0.0f && amax < TINY_OUT;
  // amax < 2^e; exponents below -100 are raised so the factor stays finite
  const int e = amax > 0.0f ? max(__builtin_amdgcn_frexp_expf(amax), -100) : 0;
  const float f = __builtin_amdgcn_ldexpf(inv, 15 - e);
  const float sc = amax > 0.0f ? __builtin_amdgcn_ldexpf(1.0f, e - 15) : 0.0f;
#pragma unroll
  for (int nt = 0; nt < DV_TILES; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = f32x4{a.o[nt][4 * i], a.o[nt][4 * i + 1], a.o[nt][4 * i + 2], a.o[nt][4 * i + 3]} * f;
      *(f16x4*)(stage + r * SROW + (nt * 32 + i * 8 + h * 4) * 2) = __builtin_convertvector(v, f16x4);
    }
  __syncthreads();
  const int64_t pi0 = ((int64_t)tok * p.num_splits + split) * p.H;
  for (int rr = wave; rr < ROWS; rr += NW)
    if (rr < p.H) *(u32x4*)(p.part_o + (pi0 + rr) * LATENT + 8 * lane) = *(const u32x4*)(stage + rr * SROW + 16 * lane);
  __syncthreads();
  if (head_ok && h == 0) *(f32x2*)(p.part_ls + 2 * (pi0 + head)) = f32x2{lse_v, sc};
  return __builtin_isfinite(osum) && !tiny;
}

// Work item of a workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs; the splits of one token are placed 8 blocks apart so that they
// share an XCD (the token's queries are then read into one L2).
struct Work {
  int tok, split, b, ctx, e_lo, e_hi;
};

__device__ __forceinline__ bool map_work(const AttnParams& p, Work& w) {
  const int S = p.num_splits;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  w.tok = xcd + 8 * (slot / S);
  w.split = slot % S;
  if (w.tok >= p.sv.num_tokens) return false;
  w.b = seq_of_token(p.sv, w.tok);
  w.ctx = p.sv.ctx_len[w.b];
  w.e_lo = w.split * p.split_len;
  w.e_hi = min(p.top_k, w.e_lo + p.split_len);
  return true;
}

// Resolve the valid index entries of the split (0 <= s < ctx) to cache rows,
// compacted in entry order into rows[0 .. n); the tail of the last tile
// repeats rows[0] so every gather stays in bounds.  Returns n.  All index
// loads of the split are issued before the first is used (one memory
// latency, not one per round).
template <int NW, int MAXE>
__device__ __forceinline__ int resolve_rows(const AttnParams& p, const Work& w, int* rows, int* wsum, int tid) {
  constexpr int THREADS = NW * WAVE;
  constexpr int ROUNDS = (MAXE + THREADS - 1) / THREADS;
  const int32_t* idx_row = p.idx + (int64_t)w.tok * p.top_k;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  int sv[ROUNDS];
#pragma unroll
  for (int j = 0; j < ROUNDS; ++j) {
    const int e = w.e_lo + j * THREADS + tid;
    sv[j] = e < w.e_hi ? idx_row[e] : -1;
  }
  int n = 0;
#pragma unroll
  for (int j = 0; j < ROUNDS; ++j) {
    if (w.e_lo + j * THREADS >= w.e_hi) break;  // uniform
    const int s = sv[j];
    const bool valid = s >= 0 && s < w.ctx;
    const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
    if (lane == 0) wsum[(j & 1) * NW + wave] = __builtin_popcountll(m);
    __syncthreads();
    int off = n, tot = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const int c = wsum[(j & 1) * NW + q];
      off += q < wave ? c : 0;
      tot += c;
    }
    if (valid) rows[off + __builtin_popcountll(m & below)] = (int)cache_row(p.sv, w.b, s);
    n += tot;
  }
  __syncthreads();
  const int padded = cdiv(n, TILE) * TILE;
  if (n > 0)
    for (int i = n + tid; i < padded; i += THREADS) rows[i] = rows[0];
  __syncthreads();
  return n;
}

// ---------------------------------------------------------------------------
// Tile producers.  issue(k, slot) starts the gathers of tile k; for bf16 rows
// they land in the compute buffer, for FP8 rows in a raw staging buffer that
// convert() then dequantises.  LOADS is the per-wave count of gather
// instructions per tile that every wave has at least (for wait_vmcnt).
// ---------------------------------------------------------------------------
template <int NW>
struct Bf16Rows {
  static constexpr int INSTR = TILE + ROPE_TILE_BYTES / 1024;  // 32 latent rows + 4 rope KiB
  static constexpr int LOADS = INSTR / NW;
  static_assert(INSTR % NW == 0, "gathers must split evenly over the waves");

  // The gathers of a tile as 4 blocks of 9 instructions: 8 latent rows, then
  // the rope parts of those 8 rows.  Lane j (mod 32) reads the cache row of
  // tile row j once (prepare); a latent-row gather takes its row from that
  // register into a scalar register (v_readlane) and addresses the row with
  // an SGPR base, so only the lane's chunk offset lives in a VGPR; a rope
  // gather takes its per-lane rows through the LDS crossbar.
  struct Tile {
    int rowv;
    uint32_t buf;
  };
  __device__ __forceinline__ static Tile prepare(const int* rows, uint32_t buf, int lane) {
    return Tile{rows[lane & (TILE - 1)], buf};
  }
  // instruction i = 9 b + m of the tile (wave-uniform)
  template <int M>
  __device__ __forceinline__ static void issue_one(const AttnParams& p, const Tile& t, int b, int lane) {
    if constexpr (M < 8) {
      const int r = 8 * b + M;
      const int row = __builtin_amdgcn_readlane(t.rowv, r);
      dma16_s(p.kv + (int64_t)row * (ROW * 2), (uint32_t)((lane ^ lat_swz(r)) << 4), t.buf + r * LAT_STRIDE);
    } else {
      const int r = 8 * b + (lane >> 3);
      const int row = __builtin_amdgcn_ds_bpermute(r << 2, t.rowv);
      dma16(p.kv + (int64_t)row * (ROW * 2) + LATENT * 2 + (((lane & 7) ^ rope_swz(r)) << 4),
            t.buf + LAT_TILE_BYTES + b * 1024);
    }
  }
  // every gather of this wave for one tile: instructions wave * LOADS + j
  __device__ __forceinline__ static void issue(const AttnParams& p, const int* rows, uint32_t buf, int wave,
                                               int lane) {
    const Tile t = prepare(rows, buf, lane);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int i = wave * LOADS + j;
      const int b = i / 9, m = i - 9 * b;
      if (m < 8) {
        const int r = 8 * b + m;
        const int row = __builtin_amdgcn_readlane(t.rowv, r);
        dma16_s(p.kv + (int64_t)row * (ROW * 2), (uint32_t)((lane ^ lat_swz(r)) << 4), t.buf + r * LAT_STRIDE);
      } else {
        issue_one<8>(p, t, b, lane);
      }
    }
  }
  // With one block per wave (4 waves), the gathers of this wave
  // can be spread over the k-steps of an S phase: the j-th goes out after
  // k-step (j * KSTEPS) / LOADS, so the wave never stalls behind a full memory
  // queue while its MFMAs wait.
  static constexpr bool SPREAD = LOADS == 9;
  template <int KS>
  __device__ __forceinline__ static void issue_at_step(const AttnParams& p, const Tile& t, int wave, int lane) {
    constexpr int J = KS * LOADS / KSTEPS;  // KSTEPS = 4 LOADS
    if constexpr (KS % (KSTEPS / LOADS) == 0) issue_one<J>(p, t, wave, lane);
  }

  // fp16 copy, in place, of the 16 bytes that this lane's gather j of a tile
  // (instruction wave * LOADS + j) brought into the tile buffer `buf`.  A wave
  // converts only what its own gathers wrote, so its own vmcnt wait is all
  // the conversion needs; the next barrier publishes the result.
  __device__ __forceinline__ static int own_off(int j, int wave, int lane) {
    const int i = wave * LOADS + j;
    const int b = i / 9, m = i - 9 * b;
    return (m < 8 ? (8 * b + m) * LAT_STRIDE : LAT_TILE_BYTES + b * 1024) + 16 * lane;
  }
  // (latent chunks only: the rope stays bf16)
  __device__ __forceinline__ static void convert_own(uint8_t* buf, int j, int wave, int lane) {
    uint8_t* q = buf + own_off(j, wave, lane);
    if constexpr (LOADS % 9 == 0) {
      if (j % 9 < 8) bf16x8_to_f16_lds(q);
    } else {  // the gather's place in its block depends on the wave: a select, not a branch
      const bool lat = (wave * LOADS + j) % 9 < 8;
      const u32x4 v = *(const u32x4*)q;
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = lat ? bf16x2_to_f16x2(v[e]) : v[e];
      *(u32x4*)q = r;
    }
  }
  __device__ __forceinline__ static void convert_all(uint8_t* buf, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) convert_own(buf, j, wave, lane);
  }
  // The same conversion spread over the k-steps of an S phase: the wave
  // issues in order, so VALU work hides under the MFMAs only a few
  // instructions at a time, between them.  After the wave's own gathers of
  // the tile have landed (wait at k-step CONV_WAIT), chunk j is read at k-step
  // CONV0 + 3 j - 1, its dwords 0-1 converted at CONV0 + 3 j, dwords 2-3 and
  // the write at CONV0 + 3 j + 1 (two chunks in flight).
  static constexpr int CONV_WAIT = 4, CONV0 = 6;
  static_assert(CONV0 + 3 * LOADS - 1 <= KSTEPS || LOADS > 9, "conversion fits the S phase");
  // (with one block of 9 gathers per wave, gather 8 is the rope: not converted)
  template <int KS>
  __device__ __forceinline__ static void conv_step(u32x4 (&held)[2], uint8_t* buf, int wave, int lane) {
    constexpr int d = KS - CONV0 + 1;
    constexpr int j = d / 3, ph = d % 3;
    static_assert(!SPREAD || LOADS == 9, "one block of 9 gathers per wave");
    if constexpr (d >= 0 && j < 8) {
      if constexpr (ph == 0) held[j & 1] = *(const u32x4*)(buf + own_off(j, wave, lane));
      if constexpr (ph == 1) {
        held[j & 1][0] = bf16x2_to_f16x2(held[j & 1][0]);
        held[j & 1][1] = bf16x2_to_f16x2(held[j & 1][1]);
      }
      if constexpr (ph == 2) {
        held[j & 1][2] = bf16x2_to_f16x2(held[j & 1][2]);
        held[j & 1][3] = bf16x2_to_f16x2(held[j & 1][3]);
        *(u32x4*)(buf + own_off(j, wave, lane)) = held[j & 1];
      }
    }
  }
};

template <int NW>
struct Fp8Rows {
  // Wave w gathers and dequantises the tile rows w, w + NW, .. of its own:
  // the workgroup needs no barrier between a raw tile's arrival and its
  // dequantisation, only the one per tile that publishes the fp16 tile.
  static constexpr int ROWS = (TILE + NW - 1) / NW;               // rows of a wave (at most)
  static constexpr int LOADS = (ROWS * ROW_CHUNKS + 63) / 64;      // gathers of a wave per tile
  static constexpr int WAVE_BYTES = LOADS * 1024;                  // a wave's part of a raw slot
  static constexpr int SLOT_BYTES = NW * WAVE_BYTES;               // one raw ring slot

  // The wave's rows of one tile, packed at raw + wave * WAVE_BYTES (row j of
  // the wave at j * FP8_ROW_BYTES).  Every lane of every gather is active, so
  // each wave issues exactly LOADS gathers per tile (its waits count them):
  // lanes past the wave's rows fetch their own first row again into the
  // unused end of the wave's part.
  __device__ __forceinline__ static void issue(const AttnParams& p, const int* rows, uint32_t raw, int wave,
                                               int lane) {
    const int nrows = (TILE - wave + NW - 1) / NW;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = i * 64 + lane;
      const int j = q / ROW_CHUNKS, ch = q % ROW_CHUNKS;
      const int r = j < nrows ? wave + NW * j : wave;
      dma16(p.kv + (int64_t)rows[r] * FP8_ROW_BYTES + ch * 16, raw + wave * WAVE_BYTES + i * 1024);
    }
  }

  // 4 e4m3 codes times the tile scale s -> 4 fp16 (or bf16) values, two
  // dwords.  fp16: the gfx950 scaled conversion multiplies by the power of
  // two 2^floor(log2 s) (it reads only the exponent field of s; exact while
  // the product is an fp16 normal), then a packed fp16 multiply by the rest of
  // s, m = s / 2^floor(log2 s) in [1, 2) rounded to fp16: two roundings of
  // 2^-11 each instead of one, and a product beyond the fp16 range still ends
  // as infinity.  bf16: fp32 products, rounded once.
  template <bool F16>
  __device__ __forceinline__ static u32x2 dequant4(uint32_t w, float s, f16x2 m) {
    if constexpr (F16) {
      const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s, false) * m;
      const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s, true) * m;
      return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    } else {
      const f32x2 lo = e4m3x2_lo(w), hi = e4m3x2_hi(w);
      return u32x2{pack2<F16>(lo[0] * s, lo[1] * s), pack2<F16>(hi[0] * s, hi[1] * s)};
    }
  }

  // 16 codes (latent chunk ch of the wave's row j) -> two 16-byte chunks of
  // the tile layout.
  template <bool F16>
  __device__ __forceinline__ static void lat_item(const uint8_t* own, uint8_t* buf, int wave, int j, int ch) {
    const uint8_t* src = own + j * FP8_ROW_BYTES;
    const u32x4 codes = *(const u32x4*)(src + ch * 16);
    const float sc = *(const float*)(src + LATENT + (ch >> 3) * 4);
    // the mantissa of sc with a zero exponent: sc / 2^floor(log2 sc)
    const _Float16 mh = (_Float16)__builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, sc) & 0x007fffffu) | 0x3f800000u);
    const f16x2 m = {mh, mh};
    const u32x2 a0 = dequant4<F16>(codes[0], sc, m), a1 = dequant4<F16>(codes[1], sc, m);
    const u32x2 a2 = dequant4<F16>(codes[2], sc, m), a3 = dequant4<F16>(codes[3], sc, m);
    const int r = wave + NW * j;
    *(u32x4*)(buf + lat_off(r, 2 * ch)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *(u32x4*)(buf + lat_off(r, 2 * ch + 1)) = u32x4{a2[0], a2[1], a3[0], a3[1]};
  }

  // The wave's rows of a raw tile -> the fp16 (or bf16) tile layout; the rope
  // is copied, bf16 as stored.  The caller has waited for the wave's gathers.
  template <bool F16>
  __device__ __forceinline__ static void convert_own(const uint8_t* raw, uint8_t* buf, int wave, int lane) {
    const uint8_t* own = raw + wave * WAVE_BYTES;
    const int nrows = (TILE - wave + NW - 1) / NW;
    constexpr int LAT_IT = (ROWS * 32 + 63) / 64;
    if constexpr (LAT_IT <= 4) {
#pragma unroll
      for (int i = 0; i < LAT_IT; ++i) {
        const int q = i * 64 + lane;
        if (q < nrows * 32) lat_item<F16>(own, buf, wave, q >> 5, q & 31);
      }
    } else {
      // (two items at a time: the queries, O^T and P are live around this,
      // and a full unroll of 6 or more items spills)
#pragma unroll 2
      for (int i = 0; i < LAT_IT; ++i) {
        const int q = i * 64 + lane;
        if (q < nrows * 32) lat_item<F16>(own, buf, wave, q >> 5, q & 31);
      }
    }
#pragma unroll 2
    for (int i = 0; i < (ROWS * 8 + 63) / 64; ++i) {
      const int q = i * 64 + lane;
      if (q < nrows * 8) {
        const int j = q >> 3, ch = q & 7;
        *(u32x4*)(buf + rope_off(wave + NW * j, ch)) = *(const u32x4*)(own + j * FP8_ROW_BYTES + LATENT + 16 + ch * 16);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// bf16 rows: direct HBM -> LDS gathers through an NBUF-deep ring.
//
// fp16 run (the default): after the S phase of tile k, each wave waits for its
// own gathers of tile k + 1 and converts them to fp16 in place, in the shadow
// of the P.V MFMAs of tile k - 1 (the barrier at the top of iteration k + 1
// publishes them); tiles 0 and 1 are converted before the loop.  bf16 run
// (the fallback when an operand leaves the fp16 range): no conversion, P split
// into hi + lo.
// ---------------------------------------------------------------------------
template <int NW, int NBUF, int MAXE>
__global__ __launch_bounds__(NW * WAVE, 1) void attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * BUF_BYTES];
  __shared__ int rows_sh[MAXE];
  // per-wave scratch ints in the last ring slot: it is first filled by the
  // gathers of tile NBUF - 1, issued in the loop after every use of the scratch
  int* wsum = (int*)(smem + (NBUF - 1) * BUF_BYTES);
  typedef Bf16Rows<NW> R;
  static_assert(NBUF == 4, "two tiles in flight, one in S, one in P.V");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches)
  const int h = lane >> 5;
  Work w;
  if (!map_work(p, w)) return;
  const int head = wave * HPW + (lane & 31);
  const bool head_ok = head < p.H;

  // index entries first (they gate the gathers), then the queries and the
  // first gathers in flight together
  const int n = resolve_rows<NW, MAXE>(p, w, rows_sh, wsum, tid);
  const int ntiles = cdiv(n, TILE);
  WaveAcc a;
  load_q(a, p, w.tok, head, head_ok, h);

  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  TileAddr ad;
  ad.init(lane);
  float m_ref = -INFINITY;

  auto run = [&](auto f16_tag) -> uint32_t {
    constexpr bool F16 = decltype(f16_tag)::value;
    constexpr bool SPLITP = !F16;
    reset_acc(a, m_ref);
    for (int k = 0; k < NBUF - 2; ++k)
      if (k < ntiles) R::issue(p, rows_sh + k * TILE, smem_base + k * BUF_BYTES, wave, lane);
    // queries and the first tiles landed: no compiler-inserted waits in the loop
    wait_vmcnt<0>();
    if constexpr (F16) {
      if (m_ref == -INFINITY) convert_q<true>(a);  // (the first fp16 run)
      if (ntiles > 0) R::convert_all(smem, wave, lane);  // tile 0; S of tile k converts tile k + 1
    }
    // Iteration k: (bf16 run: wait for this wave's gathers of tile k, tile
    // k + 1 staying in flight) one barrier (tile k visible to every wave;
    // ring slot (k + 2) % NBUF, last read by P.V of tile k - 2, free again), S
    // of tile k with the gathers of tile k + 2 spread over its k-steps, then
    // P.V of tile k - 1 with the softmax of tile k (and, fp16 run, the
    // conversion of tile k + 1) in the shadow of its MFMAs.  Iteration 0 (no
    // P.V before it) is peeled: a branch around the P.V inside the loop makes
    // the compiler shuffle the AGPR-resident O^T.
    // fp16 run: S of tile k also converts tile k + 1 (this wave's gathers of
    // it are waited for at k-step CONV_WAIT, leaving the gathers of tile k + 2
    // issued so far in flight).  In the last iteration there is no tile k + 1:
    // the slot converted then holds tile k - 3, read by no one any more.
    auto s_of_tile = [&](int k) {
      if constexpr (!F16) {
        if (k + 1 < ntiles) wait_vmcnt<R::LOADS>();
        else wait_vmcnt<0>();
      }
      __syncthreads();
      const bool more = k + NBUF - 2 < ntiles;  // uniform
      const int slot_next = (k + NBUF - 2) % NBUF;
      const uint8_t* buf = smem + (k % NBUF) * BUF_BYTES;
      uint8_t* cbuf = smem + ((k + 1) % NBUF) * BUF_BYTES;
      u32x4 held[2];
      if (R::SPREAD && more) {
        // (the tile index goes through a scalar register so that the compiler
        // does not carry the row pointer as a VGPR induction variable)
        const int kn = __builtin_amdgcn_readfirstlane(k + NBUF - 2);
        const typename R::Tile nt = R::prepare(rows_sh + kn * TILE, smem_base + slot_next * BUF_BYTES, lane);
        return s_phase<F16>(a, buf, ad, [&](auto ks) {
          constexpr int KS = decltype(ks)::value;
          R::template issue_at_step<KS>(p, nt, wave, lane);
          if constexpr (F16) {
            // gathers of tile k + 2 issued so far: at k-steps 0, 4, .., CONV_WAIT
            if constexpr (KS == R::CONV_WAIT) wait_vmcnt<R::CONV_WAIT / 4 + 1>();
            R::template conv_step<KS>(held, cbuf, wave, lane);
          }
        });
      }
      if (more) R::issue(p, rows_sh + (k + NBUF - 2) * TILE, smem_base + slot_next * BUF_BYTES, wave, lane);
      const f32x16 sres = s_phase<F16>(a, buf, ad, [&](auto ks) {
        constexpr int KS = decltype(ks)::value;
        if constexpr (F16) {
          if constexpr (KS == R::CONV_WAIT) {
            if (more) wait_vmcnt<R::LOADS>();
            else wait_vmcnt<0>();
          }
          if constexpr (R::SPREAD) R::template conv_step<KS>(held, cbuf, wave, lane);
        }
      });
      if constexpr (F16 && !R::SPREAD) R::convert_all(cbuf, wave, lane);
      return sres;
    };
    POp op_prev;
    if (ntiles > 0) {
      SoftmaxTile<F16, SPLITP> sm(s_of_tile(0));
      sm.run_all(a, min(TILE, n), p.scale_log2, h);
      op_prev = sm.op;
    }
    for (int k = 1; k < ntiles; ++k) {
      SoftmaxTile<F16, SPLITP> sm(s_of_tile(k));
      const int nv = min(TILE, n - k * TILE);
      v_phase<F16, SPLITP>(a, smem + ((k - 1) % NBUF) * BUF_BYTES, ad, op_prev,
                           [&](auto st) { sm.template stage<decltype(st)::value>(a, nv, p.scale_log2, h); });
      op_prev = sm.op;
    }
    if (ntiles > 0) v_phase<F16, SPLITP>(a, smem + ((ntiles - 1) % NBUF) * BUF_BYTES, ad, op_prev, NoStep());
    o_fence(a);
    return redo_reasons<NW>(a, F16 ? MAX_GROWTH_F16 : MAX_GROWTH, wsum, wave, lane);
  };

  // Runs: a head that outgrew its reference (its p may then have
  // overflowed, making the run non-finite as well) runs again against its
  // true maximum (a second run's maximum is its reference: no further
  // growth); a run that is non-finite otherwise, or whose O is, had an
  // operand outside the fp16 range, and a run whose O is nonzero but below
  // 2^-14 for some head came from fp16 subnormals: the split runs again in
  // bf16 (writing its result over the first one).
  uint32_t why = run(std::true_type());
  if (why & RUN_GROWTH) {
    m_ref = a.m_max;
    why = run(std::true_type());
  }
  if (why == 0) {
    const bool ok = write_result_staged<NW>(a, p, w.tok, w.split, head, head_ok, h, true, smem, wave, lane);
    if (!any_lane<NW>(!ok, wsum, wave, lane)) return;
  }
  // bf16 operands (the result written over the fp16 one, if any)
  m_ref = -INFINITY;
  load_q(a, p, w.tok, head, head_ok, h);
  why = run(std::false_type());
  if (why & RUN_GROWTH) {
    m_ref = a.m_max;
    run(std::false_type());
  }
  write_result_staged<NW>(a, p, w.tok, w.split, head, head_ok, h, false, smem, wave, lane);
}

// ---------------------------------------------------------------------------
// bf16 rows, at most 32 heads, rows not split: one wave per workgroup and a
// single tile buffer (about 40 KiB of LDS with MAXE <= 256), so several
// tokens share a CU, one per SIMD, instead of one token holding the CU's
// whole LDS for its ring.  Each tile is gathered, waited for and computed in
// turn; the other tokens on the CU fill the gaps.  (Few heads make the
// per-token work small, so the loads' latency, not the MFMAs, bounds it.)
// ---------------------------------------------------------------------------
template <int MAXE>
__global__ __launch_bounds__(WAVE, 1) void attn_bf16_single_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BUF_BYTES];
  __shared__ int rows_sh[MAXE];
  __shared__ int wsum[4];
  typedef Bf16Rows<1> R;
  const int lane = threadIdx.x;
  const int h = lane >> 5;
  Work w;
  if (!map_work(p, w)) return;
  const int head = lane & 31;
  const bool head_ok = head < p.H;
  const int n = resolve_rows<1, MAXE>(p, w, rows_sh, wsum, lane);
  const int ntiles = cdiv(n, TILE);
  WaveAcc a;
  load_q(a, p, w.tok, head, head_ok, h);
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  TileAddr ad;
  ad.init(lane);
  float m_ref = -INFINITY;
  // bf16 operands, P split into hi + lo (these tokens are latency-bound: few
  // heads, short lists)
  for (int attempt = 0; attempt < 2; ++attempt) {
    reset_acc(a, m_ref);
    for (int k = 0; k < ntiles; ++k) {
      // the previous tile's operand reads have all returned (their values
      // fed its MFMAs), so the buffer can be overwritten
      R::issue(p, rows_sh + k * TILE, smem_base, 0, lane);
      wait_vmcnt<0>();
      const f32x16 sc = s_phase<false>(a, smem, ad, NoStep());
      SoftmaxTile<false, true> sm(sc);
      sm.run_all(a, min(TILE, n - k * TILE), p.scale_log2, h);
      v_phase<false, true>(a, smem, ad, sm.op, NoStep());
    }
    o_fence(a);
    if (!(redo_reasons<1>(a, MAX_GROWTH, wsum, 0, lane) & RUN_GROWTH)) break;
    m_ref = a.m_max;
  }
  write_result(a, p, w.tok, w.split, head, head_ok, h, false);
}

// ---------------------------------------------------------------------------
// FP8 rows: gathers into a raw NRAW-deep ring, each wave dequantising the
// rows it gathered into a double-buffered tile: fp16 values (the codes times
// their tile scale, within two fp16 roundings inside the fp16 range) and fp16
// P; bf16 values and bf16 P when a value leaves the fp16 range.
// ---------------------------------------------------------------------------
template <int NW, int NRAW, int MAXE>
__global__ __launch_bounds__(NW * WAVE, 1) void attn_fp8_kernel(AttnParams p) {
  typedef Fp8Rows<NW> R;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * BUF_BYTES + NRAW * R::SLOT_BYTES];
  __shared__ int rows_sh[MAXE];
  // per-wave scratch ints in the last raw ring slot: it is first filled by
  // the gather issued in iteration 0, after every use of the scratch
  int* wsum = (int*)(smem + 2 * BUF_BYTES + (NRAW - 1) * R::SLOT_BYTES);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches)
  const int h = lane >> 5;
  Work w;
  if (!map_work(p, w)) return;
  const int head = wave * HPW + (lane & 31);
  const bool head_ok = head < p.H;

  WaveAcc a;
  load_q(a, p, w.tok, head, head_ok, h);
  const int n = resolve_rows<NW, MAXE>(p, w, rows_sh, wsum, tid);
  const int ntiles = cdiv(n, TILE);
  wait_vmcnt<0>();

  uint8_t* raw = smem + 2 * BUF_BYTES;
  const uint32_t raw_base = (uint32_t)(uintptr_t)(lds_void*)raw;
  TileAddr ad;
  ad.init(lane);
  float m_ref = -INFINITY;

  auto run = [&](auto f16_tag) -> uint32_t {
    constexpr bool F16 = decltype(f16_tag)::value;
    reset_acc(a, m_ref);
#pragma unroll
    for (int k = 0; k < NRAW - 1; ++k)
      if (k < ntiles) R::issue(p, rows_sh + k * TILE, raw_base + k * R::SLOT_BYTES, wave, lane);
    // this wave's rows of tile 0 (the gathers of tile 1 stay in flight)
    if (ntiles > 0) {
      if (ntiles > 1) wait_vmcnt<R::LOADS>();
      else wait_vmcnt<0>();
      R::template convert_own<F16>(raw, smem, wave, lane);
    }
    // Iteration k: one barrier (every wave's rows of tile k are in tile slot
    // k % 2; every wave is done with tile k - 1, so slot (k + 1) % 2 is free),
    // this wave's gathers of tile k + NRAW - 1 (into the raw slot of tile
    // k - 1, which this wave dequantised in iteration k - 2), S and softmax
    // of tile k, this wave's rows of tile k + 1 dequantised (its gathers
    // waited for, those of the next tile left in flight), P.V of tile k.
    // (Dequantising between the P.V MFMAs instead spilled registers and
    // measured slower.)
    for (int k = 0; k < ntiles; ++k) {
      __syncthreads();
      if (k + NRAW - 1 < ntiles)
        R::issue(p, rows_sh + (k + NRAW - 1) * TILE, raw_base + ((k + NRAW - 1) % NRAW) * R::SLOT_BYTES, wave,
                 lane);
      const uint8_t* buf = smem + (k & 1) * BUF_BYTES;
      const f32x16 sc = s_phase<F16>(a, buf, ad, NoStep());
      SoftmaxTile<F16, false> sm(sc);
      sm.run_all(a, min(TILE, n - k * TILE), p.scale_log2, h);
      if (k + 1 < ntiles) {
        const int later = min(NRAW - 2, ntiles - 2 - k);  // tiles issued after tile k + 1
        if (later >= 2) wait_vmcnt<2 * R::LOADS>();
        else if (later == 1) wait_vmcnt<R::LOADS>();
        else wait_vmcnt<0>();
        R::template convert_own<F16>(raw + ((k + 1) % NRAW) * R::SLOT_BYTES, smem + ((k + 1) & 1) * BUF_BYTES,
                                     wave, lane);
      }
      v_phase<F16, false>(a, buf, ad, sm.op, NoStep());
    }
    o_fence(a);
    return redo_reasons<NW>(a, F16 ? MAX_GROWTH_F16 : MAX_GROWTH, wsum, wave, lane);
  };

  // attempts as in attn_bf16_kernel
  convert_q<true>(a);
  uint32_t why = run(std::true_type());
  if (why & RUN_GROWTH) {
    m_ref = a.m_max;
    why = run(std::true_type());
  }
  if (why == 0) {
    const bool ok = write_result_staged<NW>(a, p, w.tok, w.split, head, head_ok, h, true, smem, wave, lane);
    if (!any_lane<NW>(!ok, wsum, wave, lane)) return;
  }
  m_ref = -INFINITY;
  load_q(a, p, w.tok, head, head_ok, h);  // the stored bf16 queries again
  wait_vmcnt<0>();
  why = run(std::false_type());
  if (why & RUN_GROWTH) {
    m_ref = a.m_max;
    run(std::false_type());
  }
  write_result_staged<NW>(a, p, w.tok, w.split, head, head_ok, h, false, smem, wave, lane);
}

// Merge split partials: lse = log sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s,
// with O_s = scale_s * (stored fp16 values).
// One workgroup per (token, 4 heads), a wave per head, each lane 8 of the
// 512 values (16-byte loads of the partials, two 16-byte stores).  The
// (lse, scale) pairs and partials of COMBINE_BATCH splits are loaded before
// any is used, so with at most COMBINE_BATCH splits the merge waits for one
// memory latency; a split whose weight is zero (no valid entry) contributes
// nothing even if its values are not finite.
constexpr int COMBINE_BATCH = 4;
constexpr int COMBINE_HEADS = 4;  // heads (waves) per workgroup

__global__ __launch_bounds__(COMBINE_HEADS * WAVE) void combine_kernel(AttnParams p) {
  const int th = blockIdx.x * COMBINE_HEADS + (threadIdx.x >> 6);
  if (th >= p.sv.num_tokens * p.H) return;
  const int lane = threadIdx.x & 63;
  const int tok = th / p.H, h = th % p.H;
  const int S = p.num_splits;
  const int64_t base = (int64_t)tok * S * p.H + h;
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  float wsum = 0.0f, mx = -INFINITY;
  // (more splits than a batch: the maximum first, over every split)
  if (S > COMBINE_BATCH)
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.part_ls[2 * (base + (int64_t)s * p.H)]);
  for (int s0 = 0; s0 < S; s0 += COMBINE_BATCH) {
    f16x8 v[COMBINE_BATCH];
    f32x2 ls[COMBINE_BATCH];
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j) {
      const int64_t pi = base + (int64_t)min(s0 + j, S - 1) * p.H;
      v[j] = *(const f16x8*)(p.part_o + pi * LATENT + lane * 8);
      ls[j] = *(const f32x2*)(p.part_ls + 2 * pi);
    }
    if (S <= COMBINE_BATCH) {
#pragma unroll
      for (int j = 0; j < COMBINE_BATCH; ++j) mx = fmaxf(mx, s0 + j < S ? ls[j][0] : -INFINITY);
    }
    if (mx == -INFINITY) break;
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j) {
      const float wgt = s0 + j < S ? expf(ls[j][0] - mx) : 0.0f;
      if (wgt > 0.0f) {
        wsum += wgt;
        const float f = wgt * ls[j][1];
        acc0 += f * f32x4{(float)v[j][0], (float)v[j][1], (float)v[j][2], (float)v[j][3]};
        acc1 += f * f32x4{(float)v[j][4], (float)v[j][5], (float)v[j][6], (float)v[j][7]};
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float* orow = p.out + ((int64_t)tok * p.H + h) * LATENT + lane * 8;
  *(f32x4*)orow = acc0 * inv;
  *(f32x4*)(orow + 4) = acc1 * inv;
  if (lane == 0 && p.lse) p.lse[(int64_t)tok * p.H + h] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
}

template <typename K>
hipError_t launch_grid(K kernel, const AttnParams& p, int waves, hipStream_t stream, const TimerEvents& t) {
  const int blocks = cdiv(p.sv.num_tokens, 8) * 8 * p.num_splits;
  return launch_kernel(kernel, dim3(blocks), dim3(waves * WAVE), stream, t.start, t.stop, p);
}

template <int NW>
hipError_t launch_nw(const AttnParams& p, bool fp8, hipStream_t stream, const TimerEvents& t) {
  if (fp8) return launch_grid(attn_fp8_kernel<NW, 3, 2048>, p, NW, stream, t);
  if (NW == 1 && p.num_splits == 1 && p.split_len <= 256)
    return launch_grid(attn_bf16_single_kernel<256>, p, 1, stream, t);
  if (p.split_len <= 1024) return launch_grid(attn_bf16_kernel<NW, 4, 1024>, p, NW, stream, t);
  return launch_grid(attn_bf16_kernel<NW, 4, 2048>, p, NW, stream, t);
}

}  // namespace

int attn_num_splits(int num_tokens, int H, int top_k) {
  (void)H;
  // one workgroup per (token, split); aim for one per CU (256), splits of at
  // least four tiles
  const int max_splits = std::max(1, cdiv(top_k, 4 * TILE));
  const int s = cdiv(256, std::max(1, num_tokens));
  return std::min(std::max(s, 1), max_splits);
}

hipError_t launch_attn(const AttnParams& p, bool kv_fp8, hipStream_t stream) {
  const TimerEvents t = timer_take(2);
  hipError_t e;
  if (p.H <= 32) e = launch_nw<1>(p, kv_fp8, stream, t);
  else if (p.H <= 64) e = launch_nw<2>(p, kv_fp8, stream, t);
  else if (p.H <= 96) e = launch_nw<3>(p, kv_fp8, stream, t);
  else e = launch_nw<4>(p, kv_fp8, stream, t);
  if (e != hipSuccess || p.num_splits == 1) return e;
  const TimerEvents tc = timer_take(3);
  return launch_kernel(combine_kernel, dim3(cdiv(p.sv.num_tokens * p.H, COMBINE_HEADS)), dim3(COMBINE_HEADS * WAVE),
                       stream, tc.start, tc.stop, p);
}

}  // namespace idxs
