// Lightweight-indexer score on gfx950.
//
// For a query at position t and every causal position s <= t:
//   S[s] = sum_h w[h] * ReLU(k_scale[s] * (q_I[h, :] . k_I[s, :]))
// (relevance scoring, then head-weight weighting: "Internal Fusion of the
// Indexer" in Day 0 Inference Support for New LLM Architectures; section 3
// of Day 0 Inference Acceleration for New LLM Architectures).
//
// The per-head dot products are one MFMA contraction per 16 keys: indexer
// heads sit on the MFMA M dimension (16 per tile), keys on N and d_I on K.
// Each lane then holds 4 heads x 1 key per tile, so ReLU, the head weights
// and most of the head sum stay in registers; two cross-lane adds finish the
// sum.  Per-head values never leave registers; only the fp32 score of each
// key is written (to the workspace row that the selection kernel reads).
//
// The kernel also histograms the top 11 bits of each score's order-preserving
// key per row (LDS per workgroup, merged into the row's global histogram with
// one atomic per occupied bin), so the selection kernel knows the bucket that
// holds the K-th largest score before it reads the row.
//
// Keys stream from HBM straight into the MFMA B-operand registers (16 bytes
// per lane per load).  The contraction order over d_I is free, so the dims a
// lane loads are chosen for wide loads: for bf16 keys lane group g = l/16
// takes dims 32*ks + 8*g .. +8 at k-step ks; for e4m3 keys one 16-byte load
// covers two k-steps (dims 64*j + 16*g .. +16).  The query operand uses the
// same permutation.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int SCORE_WAVES = 4;
constexpr int NT = 2;            // key tiles (16 keys each) per pipeline stage
// keys per workgroup of the decode kernel: each wave loads its token's whole
// query first, so FP8 keys (half the bytes per key) take longer runs to keep
// that prologue small against the key stream
template <bool FP8>
constexpr int decode_kpw() { return FP8 ? 2048 : 1024; }
// keys per workgroup of the multi-token kernel
constexpr int MT_KPW = 1024;
// query tokens per workgroup of the multi-token kernel: 4 (one per wave,
// every wave over all the workgroup's keys), or 2 when no sequence has more
// than 2 query tokens (waves w and w + 2 take token w over the two halves of
// the keys, so no wave idles)
__host__ __device__ __forceinline__ int mt_tokens_per_wg(int max_q_len) { return max_q_len <= 2 ? 2 : 4; }

// max(x, 0) as one integer max on the bit pattern: negative floats (-0
// included) are negative integers (fmaxf costs a second instruction that
// quiets NaN inputs)
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// First dim of the 8-wide slice that lane group g holds at k-step ks.
template <bool FP8>
__device__ __forceinline__ int kdim(int ks, int g) {
  return FP8 ? (ks >> 1) * 64 + g * 16 + (ks & 1) * 8 : ks * 32 + g * 8;
}

// MT: 16-head tiles (ceil(H_I / 16)); KS: 32-dim k-steps (d_I / 32).
// decode: the 4 waves of a workgroup split one token's key block.
// prefill: the 4 waves are 4 consecutive query tokens of one sequence and
//          all scan the workgroup's key block (shared through L1/L2).
//
// Each wave runs a two-stage register pipeline over its keys: the 16-byte
// loads of the next NT key tiles are issued before the MFMAs and the
// epilogue of the current ones, so a wave always has a stage of keys in
// flight (a wave that waited for its loads and then computed left HBM idle
// whenever the waves of a SIMD all computed at once).  A paged cache's block
// table entries for the workgroup's key block are staged in LDS first, so no
// key address waits on a dependent global load, and the scores are collected
// in LDS and written once the wave's keys are done: a global store inside the
// loop would make the next stage's address registers wait for the store, and
// so for every load issued before it.
template <int MT, int KS, bool FP8, bool DECODE>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p, int keys_per_wg) {
  constexpr int LD = FP8 ? KS / 2 : KS;  // 16-byte loads per key tile and lane
  // decode: one histogram shared by the 4 waves (one token);
  // prefill: one histogram per wave (one token each)
  __shared__ uint32_t lhist[DECODE ? 1 : SCORE_WAVES][SCORE_HIST_BINS];
  // LDS page table and score staging: a workgroup's keys (decode, split
  // over the waves), or MT_KPW keys for every wave (the multi-token kernel)
  constexpr int MAXK = DECODE ? decode_kpw<FP8>() : MT_KPW;
  constexpr int WAVE_KEYS = DECODE ? MAXK / SCORE_WAVES : MT_KPW;
  __shared__ int pages[MAXK];
  __shared__ float sbuf[SCORE_WAVES][WAVE_KEYS];
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) so that the key loop is a uniform loop: a divergent
  // one merges its exit paths and waits for every load at the loop head
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c = lane & 15;
  const SeqView& sv = p.sv;

  for (int i = threadIdx.x; i < (DECODE ? 1 : SCORE_WAVES) * SCORE_HIST_BINS; i += 256) (&lhist[0][0])[i] = 0;

  int b, tok, t, key_lo, key_hi;  // wave's keys: [key_lo, key_hi]
  bool active = true;
  const int wg_lo = blockIdx.x * keys_per_wg;
  if (DECODE) {
    b = blockIdx.y;
    tok = first_token(sv, b);
    t = sv.ctx_len[b] - 1;
    const int per_wave = keys_per_wg / SCORE_WAVES;
    key_lo = wg_lo + wave * per_wave;
    key_hi = min(t, key_lo + per_wave - 1);
  } else {
    const int tpw = mt_tokens_per_wg(sv.max_q_len);
    const int nqb = cdiv(sv.max_q_len, tpw);
    b = blockIdx.y / nqb;
    const int i = (blockIdx.y % nqb) * tpw + wave % tpw;
    const int ql = q_len(sv, b);
    active = i < ql;
    tok = first_token(sv, b) + (active ? i : 0);
    t = sv.ctx_len[b] - ql + i;
    const int span = keys_per_wg / (SCORE_WAVES / tpw);
    key_lo = wg_lo + (wave / tpw) * span;
    key_hi = min(t, key_lo + span - 1);
  }
  active = active && key_lo <= key_hi;
  // block table entries of the pages that hold keys wg_lo .. min(ctx_len, wg_lo + keys_per_wg) - 1
  const int page0 = wg_lo >> sv.page_shift;
  if (sv.block_table) {
    const int last = min(sv.ctx_len[b], wg_lo + keys_per_wg) - 1;
    const int np = last >= wg_lo ? (last >> sv.page_shift) - page0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += 256) pages[i] = sv.block_table[(int64_t)b * sv.bt_stride + page0 + i];
  }
  uint32_t* my_hist = lhist[DECODE ? 0 : wave];
  __syncthreads();

  if (active) {
    // ---- query operand (A): Q[h = 16 mt + c][kdim(ks, g) .. +8] -------------
    bf16x8 qa[MT][KS];
    float w[MT][4];
    const uint16_t* qrow = p.q_idx + (int64_t)tok * p.H_I * p.d_I;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 16 + c;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < p.H_I) v = *(const u32x4*)(qrow + (int64_t)h * p.d_I + kdim<FP8>(ks, g));
        qa[mt][ks] = as_bf16x8(v);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hr = mt * 16 + g * 4 + r;
        w[mt][r] = hr < p.H_I ? p.head_w[(int64_t)tok * p.H_I + hr] : 0.0f;
      }
    }

    const int row_bytes = FP8 ? p.d_I : p.d_I * 2;
    float* srow = p.scores + (int64_t)tok * p.score_stride;
    const int pmask = (1 << sv.page_shift) - 1;
    const int64_t seq_base = (int64_t)b * sv.seq_stride;

    // keys s0 + 16 nt + c (clamped to key_hi: rows past it are masked at the
    // store) -> raw 16-byte words; bf16 keys: word j = dims kdim(j, g) .. +8,
    // e4m3 keys: word j = dims 64 j + 16 g .. +16 (k-steps 2j and 2j + 1)
    auto load = [&](int s0, u32x4 (&raw)[NT][LD], float (&ksc)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int s = min(s0 + nt * 16 + c, key_hi);
        const int64_t row = sv.block_table ? ((int64_t)pages[(s >> sv.page_shift) - page0] << sv.page_shift) + (s & pmask)
                                           : seq_base + s;
        const uint8_t* krow = p.k_idx + row * row_bytes;
        ksc[nt] = p.k_scale ? p.k_scale[row] : 1.0f;
#pragma unroll
        for (int j = 0; j < LD; ++j)
          raw[nt][j] = *(const u32x4*)(krow + (FP8 ? j * 64 + g * 16 : kdim<false>(j, g) * 2));
      }
    };
    auto compute = [&](int s0, const u32x4 (&raw)[NT][LD], const float (&ksc)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 kb[KS];
#pragma unroll
        for (int j = 0; j < LD; ++j) {
          if (FP8) {
            const u32x2 a0 = e4m3x4_to_bf16(raw[nt][j][0], 1.0f), a1 = e4m3x4_to_bf16(raw[nt][j][1], 1.0f);
            const u32x2 a2 = e4m3x4_to_bf16(raw[nt][j][2], 1.0f), a3 = e4m3x4_to_bf16(raw[nt][j][3], 1.0f);
            kb[2 * j] = as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]});
            kb[2 * j + 1] = as_bf16x8(u32x4{a2[0], a2[1], a3[0], a3[1]});
          } else {
            kb[j] = as_bf16x8(raw[nt][j]);
          }
        }
        float v = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16(qa[mt][ks], kb[ks], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) v += w[mt][r] * relu(acc[r] * ksc[nt]);
        }
        v += shfl_xor(v, 16);
        v += shfl_xor(v, 32);
        const int s = s0 + nt * 16 + c;
        if (g == 0 && s <= key_hi) {
          sbuf[wave][s - key_lo] = v;
          atomicAdd(&my_hist[score_key(v) >> (32 - SCORE_HIST_BITS)], 1u);
        }
      }
    };

    // stage pairs in a loop with its one exit at the bottom (a second exit
    // would join the back edge with the other stage's loads still pending,
    // and the loop head would then wait for all of them), odd stage after it
    u32x4 ra[NT][LD], rb[NT][LD];
    float sa[NT], sb[NT];
    const int stages = (key_hi - key_lo) / (16 * NT) + 1;
    int s0 = key_lo;
    load(s0, ra, sa);
    for (int i = 0; i + 2 <= stages; i += 2) {
      load(s0 + 16 * NT, rb, sb);
      compute(s0, ra, sa);
      load(s0 + 32 * NT, ra, sa);
      compute(s0 + 16 * NT, rb, sb);
      s0 += 32 * NT;
    }
    if (stages & 1) compute(s0, ra, sa);
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i <= key_hi - key_lo; i += WAVE) srow[key_lo + i] = sbuf[wave][i];
  }

  // ---- merge the workgroup's histogram(s) into the row histogram(s) ---------
  __syncthreads();
  if (DECODE) {
    uint32_t* gh = p.hist + (int64_t)tok * SCORE_HIST_BINS;
    for (int i = threadIdx.x; i < SCORE_HIST_BINS; i += 256) {
      const uint32_t v = lhist[0][i];
      if (v) atomicAdd(&gh[i], v);
    }
  } else if (active) {
    uint32_t* gh = p.hist + (int64_t)tok * SCORE_HIST_BINS;
    for (int i = lane; i < SCORE_HIST_BINS; i += WAVE) {
      const uint32_t v = my_hist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
}

// ---------------------------------------------------------------------------
// Indexer over MXFP8 keys (d_I = 128), any batch: the index quantised in
// blocks of 32 values sharing a power-of-two scale ("Hierarchical
// Quantization", index-cache bullet, in Day 0 Inference Support for New LLM
// Architectures; section 4 of Day 0 Inference Adaptation and Performance
// Optimization for New Models).  A key is a row of 128 E4M3FN codes and 4
// E8M0 bytes in a separate [rows, 4] array.  The query is quantised
// on the fly, per head and block of 32, by the OCP MX rule for E4M3
// elements: shared exponent floor(log2(amax)) - 8, codes E4M3(clamp(q / 2^e,
// +-448)).  One v_mfma_scale_f32_16x16x128_f8f6f4 covers 16 heads x 16 keys
// x all 128 dims: lane (c, g) holds head / key c of its tile, dims
// 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15, and, as its scale
// operand, the E8M0 byte of block g of that head / key (the instruction
// takes block s of row c from lane c + 16 s).  The rest (pipeline,
// epilogue, histogram) is the decode kernel's.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// keys per workgroup of the MXFP8 kernel (the LDS page table and score
// staging are sized for it): every wave quantises its token's whole query
// before its keys, so long runs keep that prologue small (on 64 x 32768
// positions, with key runs on grid x: 1024 keys per workgroup 73 us, 4096
// keys 59 us)
constexpr int MX_KPW = 4096;

// The query operand of the scaled MFMA, quantised by the MX rule.  The
// instruction reads, in lane group g, the values k = 16 g .. +15 from bytes
// 0..15 and k = 64 + 16 g .. +15 from bytes 16..31, and takes the exponent of
// the 32-value block s of row m from lane m + 16 s.  So lane (c, g) finds the
// exponent of block g of head 16 mt + c, passes it as its scale operand (qe),
// and quantises its two 16-value halves with the exponents of blocks g >> 1
// and 2 + (g >> 1), fetched from the lanes that own them; w gets the head
// weights of heads 16 mt + 4 g + r (the rows of the lane's accumulator).
template <int MT>
__device__ __forceinline__ void mx_query(const ScoreParams& p, int tok, int g, int c, i32x8 (&qa)[MT], int (&qe)[MT],
                                         float (&w)[MT][4]) {
  const uint16_t* qrow = p.q_idx + (int64_t)tok * p.H_I * 128;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + c;
    const uint16_t* qh = qrow + (int64_t)h * 128;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (h < p.H_I) raw = *(const u32x4*)(qh + 32 * g + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[e] << 16)), fabsf(__uint_as_float(raw[e] & 0xffff0000u))));
    }
    // shared exponent floor(log2 amax) - 8 (frexp: amax = m 2^E, m in [0.5, 1))
    const int e = amax > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(amax) - 9, -127), 127) : -127;
    qe[mt] = e + 127;
    const int e_lo = __shfl(e, c + 16 * (g >> 1));
    const int e_hi = __shfl(e, c + 16 * (2 + (g >> 1)));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int eh = half ? e_hi : e_lo;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (h < p.H_I) raw = *(const u32x4*)(qh + 64 * half + 16 * g + 8 * j);
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          float x[4];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t r = raw[2 * e2 + k];
            x[2 * k] = fminf(fmaxf(__builtin_amdgcn_ldexpf(__uint_as_float(r << 16), -eh), -448.0f), 448.0f);
            x[2 * k + 1] = fminf(fmaxf(__builtin_amdgcn_ldexpf(__uint_as_float(r & 0xffff0000u), -eh), -448.0f), 448.0f);
          }
          qa[mt][4 * half + 2 * j + e2] = (int)fp8x4(x[0], x[1], x[2], x[3]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = mt * 16 + g * 4 + r;
      w[mt][r] = hr < p.H_I ? p.head_w[(int64_t)tok * p.H_I + hr] : 0.0f;
    }
  }
}

template <int MT>
__global__ __launch_bounds__(256) void score_mx_kernel(ScoreParams p, int keys_per_wg) {
  __shared__ uint32_t lhist[SCORE_HIST_BINS];
  __shared__ int pages[MX_KPW];
  __shared__ float sbuf[SCORE_WAVES][MX_KPW / SCORE_WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c = lane & 15;
  const SeqView& sv = p.sv;
  for (int i = threadIdx.x; i < SCORE_HIST_BINS; i += 256) lhist[i] = 0;
  // grid x: query tokens (a decode batch: one per sequence), so that
  // neighbouring workgroups of a prefill chunk read the same keys; grid y:
  // runs of keys_per_wg keys of the token's causal range [0, t]
  const int tok = blockIdx.x;
  const int b = seq_of_token(sv, tok);
  const int t = sv.ctx_len[b] - q_len(sv, b) + (tok - first_token(sv, b));
  const int wg_lo = blockIdx.y * keys_per_wg;
  const int per_wave = keys_per_wg / SCORE_WAVES;
  const int key_lo = wg_lo + wave * per_wave;
  const int key_hi = min(t, key_lo + per_wave - 1);
  const bool active = key_lo <= key_hi;
  const int page0 = wg_lo >> sv.page_shift;
  if (sv.block_table) {
    const int last = min(sv.ctx_len[b], wg_lo + keys_per_wg) - 1;
    const int np = last >= wg_lo ? (last >> sv.page_shift) - page0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += 256) pages[i] = sv.block_table[(int64_t)b * sv.bt_stride + page0 + i];
  }
  __syncthreads();

  if (active) {
    i32x8 qa[MT];
    int qe[MT];
    float w[MT][4];
    mx_query<MT>(p, tok, g, c, qa, qe, w);

    float* srow = p.scores + (int64_t)tok * p.score_stride;
    const int pmask = (1 << sv.page_shift) - 1;
    const int64_t seq_base = (int64_t)b * sv.seq_stride;

    // key s0 + 16 nt + c (clamped to key_hi: rows past it are masked at the
    // store): its codes 16 g .. +15 and 64 + 16 g .. +15, and block g's
    // exponent byte
    auto load = [&](int s0, i32x8 (&kb)[NT], int (&ke)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int s = min(s0 + nt * 16 + c, key_hi);
        const int64_t row = sv.block_table ? ((int64_t)pages[(s >> sv.page_shift) - page0] << sv.page_shift) + (s & pmask)
                                           : seq_base + s;
        const u32x4* kw = (const u32x4*)(p.k_idx + row * 128 + 16 * g);
        const u32x4 lo = kw[0], hi = kw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kb[nt][j] = (int)lo[j];
          kb[nt][4 + j] = (int)hi[j];
        }
        ke[nt] = p.k_exp[row * 4 + g];
      }
    };
    auto compute = [&](int s0, const i32x8 (&kb)[NT], const int (&ke)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float v = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb[nt], f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                            0, 0, 0, qe[mt], 0, ke[nt]);
#pragma unroll
          for (int r = 0; r < 4; ++r) v += w[mt][r] * relu(acc[r]);
        }
        v += shfl_xor(v, 16);
        v += shfl_xor(v, 32);
        const int s = s0 + nt * 16 + c;
        if (g == 0 && s <= key_hi) {
          sbuf[wave][s - key_lo] = v;
          atomicAdd(&lhist[score_key(v) >> (32 - SCORE_HIST_BITS)], 1u);
        }
      }
    };

    // stage pairs in a loop with its one exit at the bottom, odd stage after it
    i32x8 ra[NT], rb[NT];
    int ea[NT], eb[NT];
    const int stages = (key_hi - key_lo) / (16 * NT) + 1;
    int s0 = key_lo;
    load(s0, ra, ea);
    for (int i = 0; i + 2 <= stages; i += 2) {
      load(s0 + 16 * NT, rb, eb);
      compute(s0, ra, ea);
      load(s0 + 32 * NT, ra, ea);
      compute(s0 + 16 * NT, rb, eb);
      s0 += 32 * NT;
    }
    if (stages & 1) compute(s0, ra, ea);
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i <= key_hi - key_lo; i += WAVE) srow[key_lo + i] = sbuf[wave][i];
  }

  __syncthreads();
  uint32_t* gh = p.hist + (int64_t)tok * SCORE_HIST_BINS;
  for (int i = threadIdx.x; i < SCORE_HIST_BINS; i += 256) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

__global__ void zero_kernel(uint32_t* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    ((u32x4*)p)[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Prefill: a workgroup takes PF_TOKS consecutive query tokens of one sequence
// (one per wave, two waves per SIMD) and walks their whole causal key range
// [0, t_last] in tiles of PF_KT keys that every wave reads from LDS.  The
// tiles come from HBM / L2 straight into an LDS ring (global_load_lds), so
// each key row is read once per workgroup instead of once per token.
//
// Per wave and tile: for each 16-key sub-tile, MT x KS MFMAs (16 heads x 16
// keys x 32 dims) with the query operand in registers and the key operand
// read from LDS; ReLU and the head weights fold into registers; the 4 lane
// groups (4 heads each per M-tile) are summed across lanes.  Lane (g, c)
// keeps sub-tile g: the wave's 64 scores of a tile, one per lane in position
// order, go into the row's LDS histogram and, where they reach the running
// threshold bound, into the row's candidate list (one ballot, one store).
// Because the workgroup covers the whole row of each of its tokens, each
// wave then selects its token's Top-K itself from the list (wave_select_list
// above): no global atomics, no clearing pass and no separate selection
// launch.
//
// Key rows in LDS: the 16-byte chunk ch of key row r sits at chunk
// ch ^ swz(r) of the row, so the 16 keys of a sub-tile read at one logical
// chunk (16 lanes of a 128-bit read) hit 16 different bank windows.
// ---------------------------------------------------------------------------
constexpr int PF_TOKS = PREFILL_TOKS;  // tokens (= waves) per workgroup
constexpr int PF_KT = 128;        // keys per tile (one barrier per tile)
constexpr int PF_NBUF = 2;        // tile ring depth (tile k + 1 loads while tile k is computed)
constexpr int PF_MAX_PAGES = 4096;  // block-table entries a workgroup can stage
constexpr int PF_SUB_BITS = 8;      // finer bins inside the bound's bucket: key bits 20 .. 13
constexpr int PF_SUB_BINS = 1 << PF_SUB_BITS;

template <int CPR>
__device__ __forceinline__ int pf_swz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

// Reduce-scatter over the 4 lane groups (rows of 16 lanes; the prefill
// kernel's quad_part): x[st] holds the group's partial for sub-tile st; the
// result at lane (g, c) is the sum over the four groups of x[g].  Two
// butterfly steps with the gfx950 row swaps: v_permlane16_swap exchanges rows
// 1, 3 of its first operand with rows 0, 2 of its second (rows 2 r and 2 r + 1
// exchange: even rows keep sub-tiles 0 and 2, odd rows 1 and 3),
// v_permlane32_swap the upper half of the first with the lower half of the
// second (rows r and r + 2 exchange: rows 0, 1 keep the first sum, rows 2, 3
// the second).  (Inline asm: the builtins fold their two results into one
// when both inputs are the same value.)
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// ---------------------------------------------------------------------------
// Top-K of a complete score row by one wave, at the end of the prefill
// kernel: the m = min(K, t + 1) largest scores, ties to the lower position
// (the selection of the fused indexer: "Internal Fusion of the Indexer" in
// Day 0 Inference Support for New LLM Architectures; the tie rule is this
// library's reading).
//
// The score loop keeps, per row, a candidate list instead of the scores: in
// position order, (order-preserving key, position) for every key whose top
// 11 bits reach a running lower bound of the row's threshold bucket (the
// bucket of the K-th largest key seen so far, refreshed from the row's LDS
// histogram every 1024 keys).  The K-th largest of a prefix never exceeds
// the K-th largest of the row, so the list holds every key the selection can
// take.  The histogram counts the candidates only; its bins at or above the
// bound, the only ones read, hold the counts of the whole row.  They fix the
// threshold bucket d1; one pass over the list writes the positions above d1
// and compacts the d1 keys in place (still in position order) while
// histogramming their next 11 bits; a pass over those picks the 22-bit
// prefix and keeps the keys with it (usually a handful: one score value for
// integer-valued scores) in LDS, where a 10-bit histogram fixes the exact
// threshold key tau and the first keys equal to it are taken.  When the
// prefix holds more keys than the LDS list, two more passes over the d1 keys
// do the same without it.
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: four
// shifts inside each row of 16 lanes (lanes without a source add 0), then
// the last lane of row 0 (and of row 2) added to rows 1 (and 3), then lane 31
// to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The bin d of an NB-bin LDS histogram (bins in key order) holding the
// want-th largest key: S(> d) < want <= S(>= d); above = S(> d), cnt = h[d].
// Returns false (d, above, cnt unset) when the histogram holds fewer than
// want keys.  Lane l sums bins PER l .. PER l + PER - 1; a wave scan finds
// the lane whose bins hold the want-th largest key, and its PER bins, read
// again one per lane, a second scan.
template <int NB, typename H>
__device__ __forceinline__ bool wave_pick(const H* h, uint32_t want, int lane, uint32_t& d, uint32_t& above,
                                          uint32_t& cnt) {
  constexpr int PER = NB / WAVE;
  static_assert(PER >= 1 && PER <= WAVE, "one to 64 bins per lane");
  uint32_t tot = 0;
  if constexpr (PER % 4 == 0) {
    // 16-byte reads, lane l's chunks in the order (c + l / (16 / CH)) mod CH:
    // the 16 lanes of one LDS cycle then cover 16 distinct bank groups
    // (lanes PER words apart would otherwise collide CH ways)
    constexpr int CH = PER / 4;
    constexpr int SPAN = CH >= 16 ? 1 : 16 / CH;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = (c + lane / SPAN) % CH;
      const u32x4 v = *(const u32x4*)(h + PER * lane + 4 * cc);
      tot += (v[0] + v[1]) + (v[2] + v[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) tot += h[PER * lane + j];
  }
  const uint32_t incl = wave_prefix_incl(tot);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, WAVE - 1);
  const uint32_t suf = total - incl + tot;  // keys in the bins of lanes >= this one
  const uint64_t m = __builtin_amdgcn_ballot_w64(suf >= want && suf - tot < want);
  if (m == 0) return false;
  const int L = __builtin_ctzll(m);
  const uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(suf - tot), L);  // keys above lane L's bins
  const uint32_t bv = lane < PER ? h[PER * L + lane] : 0u;
  const uint32_t bincl = wave_prefix_incl(bv);
  const uint32_t btot = (uint32_t)__builtin_amdgcn_readlane((int)bincl, PER - 1);
  const uint32_t bsuf = run + btot - bincl + bv;  // keys in bins >= PER L + lane
  const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < PER && bsuf >= want && bsuf - bv < want);
  const int i = __builtin_ctzll(m2);
  d = (uint32_t)(PER * L + i);
  above = (uint32_t)__builtin_amdgcn_readlane((int)(bsuf - bv), i);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)bv, i);
  return true;
}

// The selection reads and writes the score rows and the output through
// global-address-space pointers (plain global loads and stores; through a
// generic pointer every access is a FLAT one that also waits on the LDS
// counter).
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) int32_t g_i32;
typedef __attribute__((address_space(3))) uint32_t l_u32;   // LDS
__device__ __forceinline__ void lds_inc(l_u32* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// h: the row's 2048-bin LDS histogram of the top 11 key bits (the whole
// row); cand: the row's L candidate pairs (key, position) in position order;
// list: the wave's LDS scratch of list_cap words.
__device__ void wave_select_list(uint32_t* cand_, uint32_t L, int n, int K, int32_t* out_, uint32_t* h_,
                                 uint32_t* list_, int list_cap, int lane) {
  l_u32* h = (l_u32*)h_;
  l_u32* list = (l_u32*)list_;
  g_u32* cand = (g_u32*)cand_;
  g_i32* out = (g_i32*)out_;
  const int m = min(K, n);
  for (int i = m + lane; i < K; i += WAVE) out[i] = -1;
  if (m == n) {
    for (int i = lane; i < n; i += WAVE) out[i] = i;
    return;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t d1, above1, cnt1, d2, above2, cnt2, d3, above3, cnt3;
  wave_pick<SCORE_HIST_BINS>(h, (uint32_t)m, lane, d1, above1, cnt1);
  const uint32_t rem1 = (uint32_t)m - above1;
  for (int j = lane; j < SCORE_HIST_BINS; j += WAVE) h[j] = 0u;

  // Pass over the list, 128 pairs per 16-byte load of the wave (lane l holds
  // pairs 2 l and 2 l + 1 of a group, so lane order is position order), the
  // next batch of groups loaded before the current one is processed:
  // positions above d1 to out[0 .. above1); d1 pairs compacted in place at
  // the front of the list (they land behind every pair still to be read),
  // their key bits 20..10 into the histogram.
  constexpr int UB = 4;  // groups per batch
  // groups past the list load its last pairs (the row holds one spare pair
  // beyond the longest list, so a load never leaves the row)
  const uint32_t last = L > 0 ? (L - 1) & ~1u : 0u;
  auto load_batch = [&](uint32_t b0, u32x4 (&r)[UB]) {
#pragma unroll
    for (int u = 0; u < UB; ++u) r[u] = *(const __attribute__((address_space(1))) u32x4*)(
        cand + 2 * min(b0 + 128u * u + 2u * lane, last));
  };
  uint32_t og = 0, cw = 0;
  auto do_batch = [&](uint32_t b0, const u32x4 (&r)[UB]) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const uint32_t j = b0 + 128u * u + 2u * lane;
      const uint32_t key[2] = {r[u][0], r[u][2]};
      const uint32_t pos[2] = {r[u][1], r[u][3]};
      uint64_t ba[2], bd[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = j + e < L;
        ba[e] = __builtin_amdgcn_ballot_w64(ok && (key[e] >> 21) > d1);
        bd[e] = __builtin_amdgcn_ballot_w64(ok && (key[e] >> 21) == d1);
      }
      uint32_t pa = og + __popcll(ba[0] & below) + __popcll(ba[1] & below);
      uint32_t pd = cw + __popcll(bd[0] & below) + __popcll(bd[1] & below);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (((ba[e] >> lane) & 1ull) && pa < above1) out[pa] = (int32_t)pos[e];
        pa += (ba[e] >> lane) & 1ull;
        if ((bd[e] >> lane) & 1ull) {
          *(__attribute__((address_space(1))) u32x2*)(cand + 2 * pd++) = u32x2{key[e], pos[e]};
          lds_inc(&h[(key[e] >> 10) & 2047u]);
        }
      }
      og += __popcll(ba[0]) + __popcll(ba[1]);
      cw += __popcll(bd[0]) + __popcll(bd[1]);
    }
  };
  if (L > 0) {
    // straight-line body (loads clamped, entries past the list are no-ops):
    // with a conditional half the compiler waits for every load in flight
    // at the loop head
    u32x4 ra[UB], rb[UB];
    constexpr uint32_t STEP = 128u * UB;
    load_batch(0, ra);
    for (uint32_t b0 = 0; b0 < L; b0 += 2 * STEP) {
      load_batch(b0 + STEP, rb);
      do_batch(b0, ra);
      load_batch(b0 + 2 * STEP, ra);
      do_batch(b0 + STEP, rb);
    }
  }
  wave_pick<SCORE_HIST_BINS>(h, rem1, lane, d2, above2, cnt2);
  const uint32_t rem2 = rem1 - above2;
  for (int j = lane; j < 1024; j += WAVE) h[j] = 0u;
  g_i32* out_2 = out + above1;  // d1 keys above d2, then what the last bits decide
  wait_vmcnt<0>();  // the compacted pairs are written
  // (the list holds every key of the row at or above d1, so og == above1
  // and cw == cnt1; the passes below go by the pairs actually compacted and
  // the writes stay inside the row's m entries regardless)
  const uint32_t nd1 = min(cw, cnt1);

  // f(key, position, valid) over the nd1 compacted d1 pairs, 4 per lane in
  // flight (read at device scope: this wave's own stores must not be
  // shadowed by lines of the list it read before)
  auto over_d1 = [&](auto&& f) {
    const uint64_t* pairs = (const uint64_t*)cand_;
    for (uint32_t j0 = 0; j0 < nd1; j0 += 4 * WAVE) {
      uint64_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t j = j0 + WAVE * u + lane;
        w[u] = j < nd1 ? __hip_atomic_load(pairs + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) f((uint32_t)w[u], (uint32_t)(w[u] >> 32), j0 + WAVE * u + lane < nd1);
    }
  };
  if (cnt2 <= (uint32_t)list_cap && n <= (1 << 22)) {
    // d1 keys above d2 to the output; those in d2 to the list as (low 10
    // key bits << 22 | position), with their low bits into the histogram
    uint32_t oa = 0, ol = 0;
    over_d1([&](uint32_t key, uint32_t pos, bool ok) {
      const uint32_t sub = (key >> 10) & 2047u;
      const uint64_t ma = __builtin_amdgcn_ballot_w64(ok && sub > d2);
      const uint64_t mb = __builtin_amdgcn_ballot_w64(ok && sub == d2);
      const uint32_t ra = oa + __popcll(ma & below), rb = ol + __popcll(mb & below);
      if (((ma >> lane) & 1ull) && ra < above2) out_2[ra] = (int32_t)pos;
      if (((mb >> lane) & 1ull) && rb < cnt2) {
        list[rb] = ((key & 1023u) << 22) | pos;
        lds_inc(&h[key & 1023u]);
      }
      oa += __popcll(ma);
      ol += __popcll(mb);
    });
    wave_pick<1024>(h, rem2, lane, d3, above3, cnt3);
    const uint32_t need = rem2 - above3;  // list keys equal to tau taken, lowest positions first
    g_i32* out_a = out_2 + above2;
    g_i32* out_e = out_a + above3;
    uint32_t oa3 = 0, oe = 0;
    for (uint32_t j0 = 0; j0 < cnt2; j0 += WAVE) {
      const uint32_t j = j0 + lane;
      const uint32_t v = j < cnt2 ? list[j] : 0u;
      const uint32_t low = v >> 22;
      const uint64_t ma = __builtin_amdgcn_ballot_w64(j < cnt2 && low > d3);
      const uint64_t me = __builtin_amdgcn_ballot_w64(j < cnt2 && low == d3);
      const int32_t pos = (int32_t)(v & ((1u << 22) - 1u));
      const uint32_t ra = oa3 + __popcll(ma & below);
      if (((ma >> lane) & 1ull) && ra < above3) out_a[ra] = pos;
      if ((me >> lane) & 1ull) {
        const uint32_t r = oe + __popcll(me & below);
        if (r < need) out_e[r] = pos;
      }
      oa3 += __popcll(ma);
      oe += __popcll(me);
    }
    return;
  }
  // d2 holds more keys than the list: the low 10 bits over the d1 keys, then
  // the positions above tau and the first `need` equal to it
  over_d1([&](uint32_t key, uint32_t, bool ok) {
    if (ok && ((key >> 10) & 2047u) == d2) lds_inc(&h[key & 1023u]);
  });
  wave_pick<1024>(h, rem2, lane, d3, above3, cnt3);
  const uint32_t lowtau = (d2 << 10) | d3;  // key bits 20..0 of tau
  const uint32_t need = rem2 - above3;
  const uint32_t n_gt = above2 + above3;  // d1 keys above tau
  uint32_t og2 = 0, oe = 0;
  over_d1([&](uint32_t key, uint32_t pos, bool ok) {
    const uint32_t low21 = key & 0x1FFFFFu;
    const uint64_t mg = __builtin_amdgcn_ballot_w64(ok && low21 > lowtau);
    const uint64_t me = __builtin_amdgcn_ballot_w64(ok && low21 == lowtau);
    const uint32_t rg = og2 + __popcll(mg & below);
    if (((mg >> lane) & 1ull) && rg < n_gt) out_2[rg] = (int32_t)pos;
    if ((me >> lane) & 1ull) {
      const uint32_t r = oe + __popcll(me & below);
      if (r < need) out_2[n_gt + r] = (int32_t)pos;
    }
    og2 += __popcll(mg);
    oe += __popcll(me);
  });
}

// MX: MXFP8 keys (E4M3FN codes in the tile, the 4 E8M0 block exponents of
// each key staged beside it) and an MX-quantised query, one scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, as score_mx_kernel) per 16 heads x 16
// keys x 128 dims instead of four bf16 ones.
template <int MT, int KS, bool FP8, bool MX = false>
__global__ __launch_bounds__(PF_TOKS * WAVE, 1) void score_prefill_kernel(ScoreParams p) {
  static_assert(!MX || (FP8 && KS == 4), "MXFP8 keys are e4m3 rows of 128");
  constexpr int ROWB = FP8 ? KS * 32 : KS * 64;  // key row bytes
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
  constexpr int TILEB = PF_KT * ROWB;
  constexpr int INSTR = TILEB / 1024;            // 1 KiB gathers per tile
  constexpr int RPI = 1024 / ROWB;               // key rows per gather
  constexpr int LOADS = INSTR / PF_TOKS;         // gathers per tile every wave has at least
  __shared__ uint32_t hist[PF_TOKS][SCORE_HIST_BINS];
  __shared__ uint32_t subh[PF_TOKS][PF_SUB_BINS];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[PF_NBUF * TILEB];
  __shared__ float ksc[PF_NBUF][PF_KT];  // per-key fp32 scale, or (MX) the key's 4 exponent bytes
  __shared__ int pages[PF_MAX_PAGES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const SeqView& sv = p.sv;

  // ---- work items: token blocks, heaviest first, taken from a counter ---------
  // Item i is block nqb - 1 - i / num_seqs of sequence i % num_seqs (the
  // last blocks of every sequence first).  The loop ends for every wave of
  // the workgroup at the same item (the counter passes pf_items).
  __shared__ int next_item;
  for (;;) {
  if (tid == 0) next_item = (int)atomicAdd(p.pf_counter, 1u);
  __syncthreads();  // (also: the previous item's selection is done with the ring and the histograms)
  const int item = next_item;
  __syncthreads();  // every wave holds the item before thread 0 takes the next one
  if (item >= p.pf_items) break;
  const int b = item % sv.num_seqs;
  const int ql = q_len(sv, b);
  const int nqb = cdiv(ql, PF_TOKS);
  const int qb = nqb - 1 - item / sv.num_seqs;
  if (qb < 0) continue;
  const int ctx = sv.ctx_len[b];
  const int i_tok = qb * PF_TOKS + wave;           // query index inside the sequence
  const bool active = i_tok < ql;
  const int tok = first_token(sv, b) + (active ? i_tok : 0);
  const int t = ctx - ql + i_tok;                  // this wave's query position
  const int t_last = ctx - ql + min(ql, (qb + 1) * PF_TOKS) - 1;
  const int ntiles = cdiv(t_last + 1, PF_KT);
  const bool paged = sv.block_table != nullptr;

  for (int i = tid; i < PF_TOKS * SCORE_HIST_BINS; i += PF_TOKS * WAVE) (&hist[0][0])[i] = 0u;
  for (int i = tid; i < PF_TOKS * PF_SUB_BINS; i += PF_TOKS * WAVE) (&subh[0][0])[i] = 0u;
  if (paged) {
    const int np = (t_last >> sv.page_shift) + 1;
    for (int i = tid; i < np; i += PF_TOKS * WAVE) pages[i] = sv.block_table[(int64_t)b * sv.bt_stride + i];
  }

  // ---- query operand: Q[h = 16 mt + c][kdim(ks, g) .. +8], head weights ------
  // (MX: the quantised query of mx_query)
  bf16x8 qa[MT][KS];
  i32x8 qx[MT];
  int qe[MT];
  float w[MT][4];
  const uint16_t* qrow = p.q_idx + (int64_t)tok * p.H_I * p.d_I;
  if constexpr (MX) mx_query<MT>(p, tok, g, c, qx, qe, w);
#pragma unroll
  for (int mt = 0; mt < MT && !MX; ++mt) {
    const int hq = mt * 16 + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hq < p.H_I) v = *(const u32x4*)(qrow + (int64_t)hq * p.d_I + kdim<FP8>(ks, g));
      qa[mt][ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = mt * 16 + g * 4 + r;
      w[mt][r] = hr < p.H_I ? p.head_w[(int64_t)tok * p.H_I + hr] : 0.0f;
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // histograms cleared, block-table entries staged

  // ---- gathers of tile k into ring slot k % PF_NBUF --------------------------
  // Wave w issues the 1 KiB instructions w, w + 8, ... of the tile; lane l of
  // instruction i reads one 16-byte chunk of key row i * RPI + l / CPR.  A
  // contiguous cache whose tile lies wholly inside the causal range takes a
  // scalar base per tile and a fixed 32-bit offset per lane and instruction.
  constexpr int NG = INSTR / PF_TOKS;  // instructions per wave and tile
  static_assert(INSTR % PF_TOKS == 0, "the gathers of a tile split evenly over the waves");
  const uint32_t ring_base = lds_addr(ring);
  auto cache_row_of = [&](int s) -> int64_t {
    s = min(s, t_last);  // keys past the last token are masked later; stay in bounds
    if (!paged) return (int64_t)b * sv.seq_stride + s;
    return ((int64_t)pages[s >> sv.page_shift] << sv.page_shift) + (s & ((1 << sv.page_shift) - 1));
  };
  const uint8_t* seq_keys = p.k_idx + (int64_t)b * sv.seq_stride * ROWB;
  uint32_t goff[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int r = (wave + PF_TOKS * j) * RPI + lane / CPR;
    goff[j] = (uint32_t)(r * ROWB + (((lane % CPR) ^ pf_swz<CPR>(r)) << 4));
  }
  auto issue = [&](int k) {
    const uint32_t slot = ring_base + (k % PF_NBUF) * TILEB;
    if (!paged && (k + 1) * PF_KT - 1 <= t_last) {
      const uint8_t* tb = seq_keys + (int64_t)k * TILEB;
#pragma unroll
      for (int j = 0; j < NG; ++j) dma16_s(tb, goff[j], slot + (wave + PF_TOKS * j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int i = wave + PF_TOKS * j;
        const int r = i * RPI + lane / CPR;
        const int ch = (lane % CPR) ^ pf_swz<CPR>(r);
        dma16(p.k_idx + cache_row_of(k * PF_KT + r) * ROWB + ch * 16, slot + i * 1024);
      }
    }
    if ((MX || p.k_scale) && wave == PF_TOKS - 1) {
#pragma unroll
      for (int j = 0; j < PF_KT / 64; ++j) {
        const int64_t row = cache_row_of(k * PF_KT + j * 64 + lane);
        dma4(MX ? (const void*)(p.k_exp + row * 4) : (const void*)(p.k_scale + row), lds_addr(&ksc[k % PF_NBUF][j * 64]));
      }
    }
  };

  // per-lane LDS offsets of the key operand: key c of the sub-tile, logical
  // chunk (bf16) 4 ks + g, (e4m3) 4 j + g for k-steps 2 j, 2 j + 1
  constexpr int NLD = FP8 ? KS / 2 : KS;  // 16-byte operand loads per sub-tile
  int boff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) boff[j] = c * ROWB + (((4 * j + g) ^ pf_swz<CPR>(c)) << 4);

  // the row's candidate pairs (key, position) in this wave's score row; the
  // row pitch holds two words per position
  uint32_t* cand = (uint32_t*)(p.scores + ((int64_t)blockIdx.x * PF_TOKS + wave) * p.score_stride);
  uint32_t* my_hist = hist[wave];
  uint32_t* my_sub = subh[wave];
  // The running bound: a lower bound of the K-th largest key of the row,
  // from the histogram (the K-th largest key seen so far lies in bucket
  // d1_cur) refined by my_sub, the histogram of key bits 20 .. 13 of the
  // candidates of bucket d1_cur that arrived since it became the bucket.
  // Those are a subset of the bucket's keys, so the threshold they give
  // (enough keys above it, with the exact count of the buckets above) never
  // exceeds the K-th largest.
  uint32_t bound = 0;              // every key at or above it is a candidate
  uint32_t d1_cur = 0xffffffffu;   // bucket that my_sub refines (none yet)
  uint32_t above_cur = 0;          // candidates in the buckets above d1_cur
  uint32_t ncand = 0;              // candidate pairs written (wave-uniform)

  // the 64 scores of quad qd of tile k (xs[st]: this lane group's partial of
  // sub-tile st) into the histogram and the candidate list
  // (sc: the fp32 scale of the lane's key, e4m3 keys only)
  auto quad_sc = [&](int k, int qd) { return (!MX && p.k_scale) ? ksc[k % PF_NBUF][qd * 64 + 16 * g + c] : 1.0f; };
  // The quad's arithmetic in five pieces (quad_part(s), s = 0 .. 4: the
  // reduce-scatter over the lane groups, then the key scale), so that a
  // pipeline step can spread them over its MFMA slots; then quad_emit.
  struct QuadState {
    float a0, b0, a1, b1, y, z, keep;
  };
  auto quad_part = [&](int s, QuadState& q, const float* xs, float sc) {
    if (s == 0) {
      q.a0 = xs[0];
      q.b0 = xs[1];
      permlane16_swap(q.a0, q.b0);
    } else if (s == 1) {
      q.a1 = xs[2];
      q.b1 = xs[3];
      permlane16_swap(q.a1, q.b1);
    } else if (s == 2) {
      q.y = (g & 1) ? xs[1] + q.a0 : xs[0] + q.b0;
    } else if (s == 3) {
      q.z = (g & 1) ? xs[3] + q.a1 : xs[2] + q.b1;
    } else if (s == 4) {
      float ya = q.y, zb = q.z;
      permlane32_swap(ya, zb);
      q.keep = (g < 2 ? q.y + zb : q.z + ya) * sc;
    }
  };
  constexpr int QPARTS = 5;
  auto quad_emit = [&](int k, int qd, float keep) {
    const int sk = k * PF_KT + qd * 64 + 16 * g + c;  // this lane's key
    // only candidates enter the histogram: every key at or above the
    // bound is a candidate, so the counts of the bins at or above it (all
    // that the bound refresh and the selection read) are the row's own
    const uint32_t key = score_key(keep);
    const uint32_t bin = key >> (32 - SCORE_HIST_BITS);
    const bool take = sk <= t && key >= bound;
    const uint64_t cm = __builtin_amdgcn_ballot_w64(take);
    if (take) {
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
      *(u32x2*)(cand + 2 * (ncand + rank)) = u32x2{key, (uint32_t)sk};
      atomicAdd(&my_hist[bin], 1u);
      if (bin == d1_cur) atomicAdd(&my_sub[(key >> (32 - SCORE_HIST_BITS - PF_SUB_BITS)) & (PF_SUB_BINS - 1)], 1u);
    }
    ncand += __popcll(cm);
    if (d1_cur != 0xffffffffu) above_cur += __popcll(__builtin_amdgcn_ballot_w64(take && bin > d1_cur));
  };
  auto quad_out = [&](int k, int qd, const float* xs, float sc) {
    QuadState q;
#pragma unroll
    for (int s = 0; s < QPARTS; ++s) quad_part(s, q, xs, sc);
    quad_emit(k, qd, q.keep);
  };

  // Software pipeline over the NST sub-tiles of 16 keys from `tile` (4: one
  // quad; 8: both quads of the tile): step st issues the key operand reads of
  // sub-tile st + 1, the MFMAs of sub-tile st and, one value per slot between
  // them, the ReLU / head-weight epilogue of sub-tile st - 1, whose MFMA
  // results have long landed (in-order issue hides VALU work only between
  // MFMAs).  The k-steps go outermost, so the MT accumulation chains
  // interleave.  With both quads, the first quad's scores go out after step 4
  // (its last epilogue then sits under the MFMAs of sub-tile 4), and the
  // tile's last sub-tile is carried into the next tile: its epilogue runs
  // under the MFMAs of the next tile's sub-tile 0 and the second quad's scores
  // go out after them (carry: the tile index, or -1; acc[1] and xs[4 .. 6]
  // hold its state, csc the key scale).  A partial tile, or the end of the
  // row, flushes the carry first.
  auto load_kb = [&](const uint8_t* tile, int st, bf16x8 (&kb)[KS]) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const u32x4 raw = *(const u32x4*)(tile + st * 16 * ROWB + boff[j]);
      if (FP8) {
        const u32x2 a0 = e4m3x4_to_bf16(raw[0], 1.0f), a1 = e4m3x4_to_bf16(raw[1], 1.0f);
        const u32x2 a2 = e4m3x4_to_bf16(raw[2], 1.0f), a3 = e4m3x4_to_bf16(raw[3], 1.0f);
        kb[2 * j] = as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]});
        kb[2 * j + 1] = as_bf16x8(u32x4{a2[0], a2[1], a3[0], a3[1]});
      } else {
        kb[j] = as_bf16x8(raw);
      }
    }
  };
  constexpr int NMF = MT * KS, NV = MT * 4;  // MFMAs, epilogue values per sub-tile
  constexpr int NSLOT = NMF > NV ? NMF : NV;
  float xs[8] = {};
  f32x4 acc[2][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[1][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int carry = -1;
  float csc = 1.0f;
  auto epilogue = [&](const f32x4 (&a)[MT]) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) v += w[i / 4][i % 4] * relu(a[i / 4][i % 4]);
    return v;
  };
  auto flush = [&]() {
    if (carry >= 0) {
      xs[7] = epilogue(acc[1]);
      quad_out(carry, 1, xs + 4, csc);
      carry = -1;
    }
  };
  auto pipeline = [&](auto nst_tag, int k, const uint8_t* tile) {
    constexpr int NST = decltype(nst_tag)::value;
    constexpr bool CARRY = NST == 8;
    bf16x8 kb[2][KS];
    // with both quads: the carried quad's pieces go into the slots of step 1,
    // the first quad's into those of step 5; each is emitted after its step
    QuadState qc, q0;
    const float sc0 = quad_sc(k, 0);
    load_kb(tile, 0, kb[0]);
    // (unrolled in full: the indices of the operand and accumulator arrays
    // must be constants, or the arrays leave the registers)
#pragma clang loop unroll(full)
    for (int st = 0; st <= (CARRY ? NST - 1 : NST); ++st) {
      if (st + 1 < NST) load_kb(tile, st + 1, kb[(st + 1) & 1]);
      float v = 0.0f;
#pragma clang loop unroll(full)
      for (int e = 0; e < NSLOT; ++e) {
        if (st < NST && e < NMF) {
          const int ks = e / MT, mt = e % MT;
          acc[st & 1][mt] = mfma16(qa[mt][ks], kb[st & 1][ks],
                                   ks == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[st & 1][mt]);
        }
        // (step 0 of a carrying pipeline: the carried sub-tile, in acc[1])
        if (st > 0 || CARRY) {
#pragma unroll
          for (int i = 0; i < NV; ++i)
            if (i * NSLOT / NV == e) v += w[i / 4][i % 4] * relu(acc[(st + 1) & 1][i / 4][i % 4]);
        }
        if (CARRY && st == 1 && e < QPARTS) quad_part(e, qc, xs + 4, csc);
        if (CARRY && st == 5 && e < QPARTS) quad_part(e, q0, xs, sc0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = NSLOT; e < QPARTS; ++e) {  // (pieces beyond the step's slots)
        if (CARRY && st == 1) quad_part(e, qc, xs + 4, csc);
        if (CARRY && st == 5) quad_part(e, q0, xs, sc0);
      }
      // (kept here: a value used only on a conditional path would be computed
      // there, after the MFMAs instead of between them)
      asm volatile("" ::"v"(v));
      if (st > 0) xs[st - 1] = v;
      if (CARRY && st == 0) xs[7] = v;
      if (CARRY && st == 1) {
        asm volatile("" ::"v"(qc.keep));
        if (carry >= 0) quad_emit(carry, 1, qc.keep);
      }
      if (CARRY && st == 5) {
        asm volatile("" ::"v"(q0.keep));
        quad_emit(k, 0, q0.keep);
      }
      if (!CARRY && st == 4) quad_out(k, 0, xs, sc0);
    }
    if constexpr (CARRY) {
      carry = k;
      csc = quad_sc(k, 1);
    }
  };

#pragma unroll
  for (int k = 0; k < PF_NBUF - 1; ++k)
    if (k < ntiles) issue(k);

  for (int k = 0; k < ntiles; ++k) {
    const int later = min(PF_NBUF - 2, ntiles - 1 - k);
    if (later >= 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    __syncthreads();  // tile k visible; slot (k - 1) % PF_NBUF free
    if (k + PF_NBUF - 1 < ntiles) issue(k + PF_NBUF - 1);
    const uint8_t* tile_k = ring + (k % PF_NBUF) * TILEB;
    if constexpr (!MX) {
      // 64-key quads inside the causal range of the wave's token
      if constexpr (PF_KT == 128) {
        if (active && k * PF_KT + 64 <= t) {
          pipeline(std::integral_constant<int, 8>(), k, tile_k);
        } else if (active && k * PF_KT <= t) {
          flush();
          pipeline(std::integral_constant<int, 4>(), k, tile_k);
        }
      } else {
        static_assert(PF_KT == 64, "tiles of one or two quads");
        if (active && k * PF_KT <= t) pipeline(std::integral_constant<int, 4>(), k, tile_k);
      }
    } else {
#pragma unroll
      for (int qd = 0; qd < PF_KT / 64; ++qd) {  // 64-key quads of the tile
        if (active && k * PF_KT + qd * 64 <= t) {
          const uint8_t* tile = tile_k + qd * 64 * ROWB;
          float xs[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            // key c of the sub-tile: codes 16 g .. +15 (chunk g) and 64 + 16 g
            // .. +15 (chunk 4 + g), and the exponent byte of its block g
            const u32x4 lo = *(const u32x4*)(tile + st * 16 * ROWB + boff[0]);
            const u32x4 hi = *(const u32x4*)(tile + st * 16 * ROWB + boff[1]);
            const i32x8 kb = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int ke = (int)((__float_as_uint(ksc[k % PF_NBUF][qd * 64 + st * 16 + c]) >> (8 * g)) & 0xffu);
            float v = 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const f32x4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qx[mt], kb, f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                                0, 0, 0, qe[mt], 0, ke);
#pragma unroll
              for (int r = 0; r < 4; ++r) v += w[mt][r] * relu(acc[r]);
            }
            xs[st] = v;
          }
          quad_out(k, qd, xs, quad_sc(k, qd));
        }
      }
    }
    // refresh the bound every 1024 keys: the bucket of the K-th largest key
    // of the row so far (all candidates: the K largest keys of a prefix are
    // at or above the bound); within an unchanged bucket, the finer bins
    if (active && ((k + 1) * PF_KT) % 1024 == 0 && min(t + 1, (k + 1) * PF_KT) > p.top_k) {
      // The bucket moves up from d1_cur while the candidates above it are
      // K or more: a window of the 64 buckets above it and one wave scan
      // find the new bucket (a pick over the whole histogram the first time,
      // or when it moves further).
      const uint32_t K = (uint32_t)p.top_k;
      uint32_t d = d1_cur, above = above_cur;
      bool moved = false;
      if (d1_cur == 0xffffffffu) {
        uint32_t cnt;
        wave_pick<SCORE_HIST_BINS>(my_hist, K, lane, d, above, cnt);
        moved = true;
      } else if (above_cur >= K) {
        const uint32_t b = d1_cur + 1 + lane;
        const uint32_t wv = b < SCORE_HIST_BINS ? my_hist[b] : 0u;
        const uint32_t pw = wave_prefix_incl(wv);  // candidates in buckets d1_cur + 1 .. b
        const uint64_t mv = __builtin_amdgcn_ballot_w64(above_cur - pw < K);
        if (mv != 0) {
          const int i = __builtin_ctzll(mv);
          d = d1_cur + 1 + i;
          above = above_cur - (uint32_t)__builtin_amdgcn_readlane((int)pw, i);
        } else {
          uint32_t cnt;
          wave_pick<SCORE_HIST_BINS>(my_hist, K, lane, d, above, cnt);
        }
        moved = true;
      }
      constexpr int SUB_SHIFT = 32 - SCORE_HIST_BITS - PF_SUB_BITS;
      if (moved) {
        for (int j = lane; j < PF_SUB_BINS; j += WAVE) my_sub[j] = 0u;
        d1_cur = d;
        above_cur = above;
        bound = max(bound, d << (32 - SCORE_HIST_BITS));
      } else {
        uint32_t sd, sa, sc_;
        if (wave_pick<PF_SUB_BINS>(my_sub, K - above, lane, sd, sa, sc_))
          bound = max(bound, (d << (32 - SCORE_HIST_BITS)) | (sd << SUB_SHIFT));
      }
    }
  }

  if constexpr (!MX) flush();

  // ---- each wave selects the Top-K of its token's complete row -----------------
  __syncthreads();
  if (active) {
    wait_vmcnt<0>();  // the wave's candidate stores have completed
    // the tile ring is free now: each wave takes an equal share as its list
    constexpr int LIST = PF_NBUF * TILEB / 4 / PF_TOKS;
    wave_select_list(cand, ncand, t + 1, p.top_k, p.out_idx + (int64_t)tok * p.top_k, my_hist,
                     (uint32_t*)ring + wave * LIST, LIST, lane);
  }
  wait_vmcnt<0>();  // this row's stores are done before the next item writes it
  }
}

// true when the prefill kernel can stage the block table of every row
bool prefill_fits(const SeqView& sv) {
  return sv.block_table == nullptr || cdiv(sv.max_ctx_len, 1 << sv.page_shift) <= PF_MAX_PAGES;
}

}  // namespace

// Batches of at most PF_MIN_Q - 1 tokens per sequence (decode, multi-token
// decode rows of speculative verification) take the streaming kernel and the
// separate Top-K: the prefill kernel gives each sequence one workgroup per 8
// tokens, so a batch of short rows leaves most CUs idle (64 requests x 2
// tokens at 32768 positions: 617 us in the prefill kernel).
constexpr int PF_MIN_Q = 9;
bool score_selects(const SeqView& sv) { return sv.max_q_len >= PF_MIN_Q && prefill_fits(sv); }

int prefill_workgroups(int num_seqs, int max_q_len) {
  const int64_t items = (int64_t)std::max(num_seqs, 1) * cdiv(std::max(max_q_len, 1), PF_TOKS);
  return (int)std::min<int64_t>(items, PREFILL_ROW_BUDGET / PF_TOKS);
}

namespace {

// The prefill kernel: its work counter cleared (a kernel, not a memset, so
// the call stays safe to capture in a graph), then prefill_workgroups
// workgroups.
template <typename K>
hipError_t launch_prefill(K kernel, const ScoreParams& p, hipStream_t stream, const TimerEvents& t) {
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, stream, p.pf_counter, (int64_t)1);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const dim3 grid(prefill_workgroups(p.sv.num_seqs, p.sv.max_q_len));
  return launch_kernel(kernel, grid, dim3(PF_TOKS * WAVE), stream, t.start, t.stop, p);
}

}  // namespace

namespace {

template <int MT, int KS, bool FP8>
hipError_t launch_mt(const ScoreParams& p, hipStream_t stream, const TimerEvents& t) {
  const SeqView& sv = p.sv;
  const bool decode = sv.max_q_len == 1;
  if (score_selects(sv)) return launch_prefill(score_prefill_kernel<MT, KS, FP8>, p, stream, t);
  if (decode) {
    const int kpw = decode_kpw<FP8>();
    dim3 grid(cdiv(sv.max_ctx_len, kpw), sv.num_seqs);
    return launch_kernel(score_kernel<MT, KS, FP8, true>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
  }
  const int kpw = MT_KPW;
  dim3 grid(cdiv(sv.max_ctx_len, kpw), sv.num_seqs * cdiv(sv.max_q_len, mt_tokens_per_wg(sv.max_q_len)));
  return launch_kernel(score_kernel<MT, KS, FP8, false>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
}

template <bool FP8>
hipError_t launch_dt(const ScoreParams& p, hipStream_t stream, const TimerEvents& t) {
  const int mt = cdiv(p.H_I, 16);
  if (p.d_I == 128) {
    switch (mt) {
      case 1: return launch_mt<1, 4, FP8>(p, stream, t);
      case 2: return launch_mt<2, 4, FP8>(p, stream, t);
      case 3: return launch_mt<3, 4, FP8>(p, stream, t);
      default: return launch_mt<4, 4, FP8>(p, stream, t);
    }
  }
  switch (mt) {
    case 1: return launch_mt<1, 2, FP8>(p, stream, t);
    case 2: return launch_mt<2, 2, FP8>(p, stream, t);
    case 3: return launch_mt<3, 2, FP8>(p, stream, t);
    default: return launch_mt<4, 2, FP8>(p, stream, t);
  }
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, int k_format, hipStream_t stream) {
  const bool k_fp8 = k_format == 1;
  // the decode kernel accumulates the row histograms with atomics: clear
  // them first (a kernel, not a memset, so the call stays safe to capture in
  // a graph); the prefill kernel keeps its histograms in LDS
  if (!score_selects(p.sv)) {
    const int64_t n4 = (int64_t)p.sv.num_tokens * SCORE_HIST_BINS / 4;
    const int64_t zblocks = std::min<int64_t>((n4 + 255) / 256, 2048);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zblocks), dim3(256), 0, stream, p.hist, n4);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  const TimerEvents t = timer_take(0);
  if (k_format == 2 && score_selects(p.sv)) {  // MXFP8 keys (d_I = 128), prefill chunks
    switch (cdiv(p.H_I, 16)) {
      case 1: return launch_prefill(score_prefill_kernel<1, 4, true, true>, p, stream, t);
      case 2: return launch_prefill(score_prefill_kernel<2, 4, true, true>, p, stream, t);
      case 3: return launch_prefill(score_prefill_kernel<3, 4, true, true>, p, stream, t);
      default: return launch_prefill(score_prefill_kernel<4, 4, true, true>, p, stream, t);
    }
  }
  if (k_format == 2) {  // MXFP8 keys, d_I = 128 (checked by the caller); decode batches
    const int kpw = MX_KPW;
    const dim3 grid(p.sv.num_tokens, cdiv(p.sv.max_ctx_len, kpw));
    switch (cdiv(p.H_I, 16)) {
      case 1: return launch_kernel(score_mx_kernel<1>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
      case 2: return launch_kernel(score_mx_kernel<2>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
      case 3: return launch_kernel(score_mx_kernel<3>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
      default: return launch_kernel(score_mx_kernel<4>, grid, dim3(256), stream, t.start, t.stop, p, kpw);
    }
  }
  return k_fp8 ? launch_dt<true>(p, stream, t) : launch_dt<false>(p, stream, t);
}

}  // namespace idxs
