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
// Work item: (token, group of 16*NW heads, split of the index list).  The
// cache row of every index of the split is resolved once (block table
// included) into LDS.  Selected latent rows are then gathered 32 per tile
// into LDS, and each wave owns 16 heads:
//   S^T[32 keys x 16 heads] = C_tile . Q^T   (MFMA 16x16x32, keys on M)
//   online softmax in fp32 registers (each lane holds 8 keys of one head)
//   O^T[512 x 16 heads]   += V^T . P^T       (MFMA, dv on M)
// The fp32 S^T tile is already laid out as the B operand of the second
// product once the key order inside the contraction is permuted to match;
// the V^T operand comes from the key-major LDS tile through the gfx950
// transposing LDS read (ds_read_b64_tr_b16), so V is stored only once.
//
// bf16 rows go from HBM straight into LDS (global_load_lds_dwordx4, one
// wave instruction per 1 KiB latent row, chunks XOR-swizzled by row so the
// MFMA operand reads are bank-conflict free) through an NBUF-deep ring, so
// NBUF-1 tiles are in flight while one is computed.  FP8 rows (656 bytes)
// are staged through registers and dequantised to bf16 on their way into
// LDS.  Splits (for decode occupancy) are merged by combine_kernel.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TILE = ATTN_TILE;                 // selected rows per tile
constexpr int LAT_STRIDE = 1024 + 32;           // 512 bf16 per row, padded by two 16-byte chunks
constexpr int LAT_TILE_BYTES = TILE * LAT_STRIDE;
constexpr int ROPE_TILE_BYTES = TILE * 128;     // 64 bf16 per row
constexpr int BUF_BYTES = LAT_TILE_BYTES + ROPE_TILE_BYTES;
constexpr float RESCALE_SLACK = 8.0f;           // log2 growth of the running max tolerated before rescaling
constexpr int EAGER_TILES = 1;                  // tiles with exact running-max normalisation
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding; the
// 6-bit vmcnt saturates at 63, and waiting for fewer is always safe).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 *
// lane (lds_addr is wave-uniform).  Written as inline asm so that the
// compiler does not turn later LDS reads of other ring slots into waits for
// every outstanding gather: completion is tracked with wait_vmcnt().
__device__ __forceinline__ void dma16(const uint8_t* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// LDS addresses of 16-byte chunk `ch` of tile row r.  Latent rows are padded
// to 66 chunks (rows 4 apart then share a bank window) and bit 0 of the
// chunk index is flipped on rows with bit 2 set.  Then 8 consecutive rows at
// one chunk (a 128-bit read of 8 lanes) cover all 32 banks, the 4 rows x 2
// chunks of a transposing read of 16 lanes cover all 32 banks, and every
// per-lane address stays affine in the chunk index (immediate offsets),
// because the flip only touches the lane-dependent bit.  The rope part is
// XOR-swizzled.
__device__ __forceinline__ int lat_flip(int r) { return (r >> 2) & 1; }
__device__ __forceinline__ int lat_off(int r, int ch) { return r * LAT_STRIDE + ((ch ^ lat_flip(r)) << 4); }
__device__ __forceinline__ int rope_off(int r, int ch) { return LAT_TILE_BYTES + r * 128 + ((ch ^ (r & 7)) << 4); }

// Per-wave state of the online softmax and the O^T accumulator: the wave
// holds NQ of the 18 k-steps of its Q^T operand (lane: Q[h][32 ks + 8 g .. +8])
// and NT of the 32 dv tiles of O^T (lane: O^T[dv = 16 nt + 4 g + r][head c]).
template <int NQ, int NT>
struct WaveAccT {
  bf16x8 qb[NQ];
  f32x4 o[NT];
  float m_run, l_run;
  int tiles;       // tiles processed so far
};
typedef WaveAccT<18, 32> WaveAcc;

template <int NQ, int NT>
__device__ __forceinline__ void load_q(WaveAccT<NQ, NT>& a, const AttnParams& p, int tok, int h, bool head_ok, int g,
                                       int ks0 = 0) {
  const uint16_t* qrow = p.q + ((int64_t)tok * p.H + (head_ok ? h : 0)) * ROW;
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (head_ok) v = *(const u32x4*)(qrow + (ks0 + kk) * 32 + g * 8);
    a.qb[kk] = as_bf16x8(v);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) a.o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  a.m_run = -INFINITY;
  a.l_run = 0.0f;
  a.tiles = 0;
}

// Per-lane addresses inside a tile buffer.
struct TileAddr {
  int s_lat[2];   // S-phase latent operand of key tiles mt = 0, 1 (chunk 4 ks + g added as offset)
  int s_rope[2][2];
  int v_lo, v_hi; // V^T operand rows 4 g + c / 4 and 16 + 4 g + c / 4
  __device__ __forceinline__ void init(int g, int c) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int r = mt * 16 + c;
      s_lat[mt] = lat_off(r, g);
      s_rope[mt][0] = rope_off(r, g);
      s_rope[mt][1] = rope_off(r, 4 + g);
    }
    const int ra = 4 * g + (c >> 2);
    const int half = (c & 1) * 8;
    v_lo = lat_off(ra, (c & 3) >> 1) + half;
    v_hi = lat_off(ra + 16, (c & 3) >> 1) + half;
  }
  __device__ __forceinline__ int s_off(int ks, int mt) const {
    return ks < 16 ? s_lat[mt] + ks * 64 : s_rope[mt][ks - 16];
  }
};

__device__ __forceinline__ bf16x8 s_operand(const uint8_t* buf, const TileAddr& ad, int ks, int mt) {
  return *(const bf16x8*)(buf + ad.s_off(ks, mt));
}

__device__ __forceinline__ bf16x8 v_operand(const uint8_t* buf, const TileAddr& ad, int nt) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + ad.v_lo + nt * 32));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + ad.v_hi + nt * 32));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Online softmax of one S^T tile (base 2).  valid8 bit j says whether key
// 16 (j / 4) + 4 g + j % 4 of the tile is a real selected row.  Returns the
// P^T operand of the tile and rescales the O^T accumulator when the running
// max moves.
struct PSplit {
  bf16x8 hi, lo;
};

template <int NQ, int NT>
__device__ __forceinline__ PSplit softmax_tile(WaveAccT<NQ, NT>& a, const f32x4 (&sacc)[2], uint32_t valid8,
                                               float scale_log2) {
  float x[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = ((valid8 >> j) & 1u) ? sacc[j >> 2][j & 3] * scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, x[j]);
  }
  tmax = fmaxf(tmax, shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor(tmax, 32));
  // Lazy rescaling: after the first EAGER_TILES tiles keep the running max
  // unless the tile exceeds it by more than RESCALE_SLACK (p values then
  // stay below 2^RESCALE_SLACK; with P split into two bf16 parts their
  // rounding does not depend on the reference).
  const bool first = a.m_run == -INFINITY;
  const float slack = a.tiles < EAGER_TILES ? 0.0f : RESCALE_SLACK;
  a.tiles++;
  const bool grow = tmax > a.m_run + slack;
  const float m_new = grow ? tmax : a.m_run;
  const float alpha = (grow && !first) ? exp2f(a.m_run - m_new) : 1.0f;
  float pv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = m_new == -INFINITY ? 0.0f : exp2f(x[j] - m_new);
  float psum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) psum += pv[j];
  a.l_run = a.l_run * alpha + psum;
  a.m_run = m_new;
  if (__ballot(alpha != 1.0f)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) a.o[nt] *= alpha;
  }
  // P = P_hi + P_lo, both bf16: the PV product runs twice on the same V^T
  // operand, so P carries ~16 mantissa bits instead of 8.
  u32x4 hi, lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const __bf16 h0 = (__bf16)pv[2 * j], h1 = (__bf16)pv[2 * j + 1];
    hi[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lo[j] = pack_bf16x2(pv[2 * j] - (float)h0, pv[2 * j + 1] - (float)h1);
  }
  PSplit r;
  r.hi = as_bf16x8(hi);
  r.lo = as_bf16x8(lo);
  return r;
}

// S^T[32 keys x 16 heads] = C_tile . Q^T over k-steps [ks0, ks0 + NQ).  The
// operands of SB k-steps are read from LDS one batch ahead of the MFMAs
// that use them, and even / odd k-steps accumulate into separate chains, so
// neither LDS latency nor the MFMA dependency latency is exposed per step.
template <int NQ, int NT>
__device__ __forceinline__ void s_phase(const WaveAccT<NQ, NT>& a, const uint8_t* buf, const TileAddr& ad,
                                        f32x4 (&sacc)[2], int ks0 = 0) {
  constexpr int SB = NQ % 6 == 0 ? 6 : (NQ % 3 == 0 ? 3 : 1);
  constexpr int NB = NQ / SB;
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 op[2][SB][2];
#pragma unroll
  for (int kk = 0; kk < SB; ++kk)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) op[0][kk][mt] = s_operand(buf, ad, ks0 + kk, mt);
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi + 1 < NB) {
#pragma unroll
      for (int kk = 0; kk < SB; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) op[(bi + 1) & 1][kk][mt] = s_operand(buf, ad, ks0 + (bi + 1) * SB + kk, mt);
    }
#pragma unroll
    for (int kk = 0; kk < SB; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt][kk & 1] = mfma16(op[bi & 1][kk][mt], a.qb[bi * SB + kk], acc[mt][kk & 1]);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) sacc[mt] = acc[mt][0] + acc[mt][1];
}

// O^T += V^T . P^T over dv tiles [nt0, nt0 + NT); the k-slot j of lane group
// g is key 16 (j / 4) + 4 g + j % 4 (the S^T register layout), which the
// V^T operand rows follow.  Operands of VB tiles are read one batch ahead.
template <int NQ, int NT>
__device__ __forceinline__ void v_phase(WaveAccT<NQ, NT>& a, const uint8_t* buf, const TileAddr& ad, PSplit pb,
                                        int nt0 = 0) {
  constexpr int VB = 4;
  constexpr int NB = NT / VB;
  bf16x8 op[2][VB];
#pragma unroll
  for (int j = 0; j < VB; ++j) op[0][j] = v_operand(buf, ad, nt0 + j);
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi + 1 < NB) {
#pragma unroll
      for (int j = 0; j < VB; ++j) op[(bi + 1) & 1][j] = v_operand(buf, ad, nt0 + (bi + 1) * VB + j);
    }
#pragma unroll
    for (int j = 0; j < VB; ++j) a.o[bi * VB + j] = mfma16(op[bi & 1][j], pb.hi, a.o[bi * VB + j]);
#pragma unroll
    for (int j = 0; j < VB; ++j) a.o[bi * VB + j] = mfma16(op[bi & 1][j], pb.lo, a.o[bi * VB + j]);
  }
}

// One tile, start to finish (used by the FP8 path).
__device__ __forceinline__ void compute_tile(WaveAcc& a, const uint8_t* buf, const TileAddr& ad, uint32_t valid8,
                                             float scale_log2) {
  f32x4 sacc[2];
  s_phase(a, buf, ad, sacc);
  const PSplit pb = softmax_tile(a, sacc, valid8, scale_log2);
  v_phase(a, buf, ad, pb);
}

// Normalise and store the wave's O^T tiles (dv tiles nt0 .. nt0 + NT) and, if
// write_lse, its lse.
template <int NQ, int NT>
__device__ __forceinline__ void write_result(const WaveAccT<NQ, NT>& a, const AttnParams& p, int tok, int split,
                                             int h, bool head_ok, int g, int nt0 = 0, bool write_lse = true) {
  float l_tot = a.l_run;
  l_tot += shfl_xor(l_tot, 16);
  l_tot += shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (a.m_run + log2f(l_tot)) * LN2 : -INFINITY;
  if (!head_ok) return;
  float* orow;
  float* lrow;
  if (p.num_splits == 1) {
    orow = p.out + ((int64_t)tok * p.H + h) * LATENT;
    lrow = p.lse ? p.lse + (int64_t)tok * p.H + h : nullptr;
  } else {
    const int64_t pi = ((int64_t)tok * p.num_splits + split) * p.H + h;
    orow = p.part_o + pi * LATENT;
    lrow = p.part_lse + pi;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) *(f32x4*)(orow + (nt0 + nt) * 16 + g * 4) = a.o[nt] * inv;
  if (write_lse && g == 0 && lrow) *lrow = lse_v;
}

// Work mapping shared by both kernels.  Workgroups are dispatched
// round-robin over the 8 XCDs, so the head groups of one (token, split) pair
// are placed 8 blocks apart and share an XCD (and its L2) for the gathered
// rows.
struct Work {
  int tok, split, hg, b, ctx, e_lo, e_hi, ntiles;
};

template <int NW>
__device__ __forceinline__ bool map_work(const AttnParams& p, Work& w) {
  const int nhg = cdiv(p.H, 16 * NW);
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  w.hg = slot % nhg;
  const int pair = (slot / nhg) * 8 + xcd;
  if (pair >= p.sv.num_tokens * p.num_splits) return false;
  w.tok = pair / p.num_splits;
  w.split = pair % p.num_splits;
  w.b = seq_of_token(p.sv, w.tok);
  w.ctx = p.sv.ctx_len[w.b];
  w.e_lo = w.split * p.split_len;
  w.e_hi = min(p.top_k, w.e_lo + p.split_len);
  w.ntiles = w.e_hi > w.e_lo ? cdiv(w.e_hi - w.e_lo, TILE) : 0;
  return true;
}

// Resolve the cache row of every index entry of the split into LDS:
// rows[i] = row of entry e_lo + i, or ~row0 (negative) when the entry is not
// a valid position (the dummy row0 keeps every gather in bounds).
template <int THREADS>
__device__ __forceinline__ void resolve_rows(const AttnParams& p, const Work& w, int* rows, int tid) {
  const int32_t* idx_row = p.idx + (int64_t)w.tok * p.top_k;
  const int row0 = (int)cache_row(p.sv, w.b, 0);
  const int n = w.ntiles * TILE;
  for (int i = tid; i < n; i += THREADS) {
    const int e = w.e_lo + i;
    const int s = e < w.e_hi ? idx_row[e] : -1;
    rows[i] = (s >= 0 && s < w.ctx) ? (int)cache_row(p.sv, w.b, s) : ~row0;
  }
}

__device__ __forceinline__ uint32_t tile_valid8(const int* rows, int g) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) v |= (rows[(j >> 2) * 16 + g * 4 + (j & 3)] >= 0 ? 1u : 0u) << j;
  return v;
}

// ---------------------------------------------------------------------------
// bf16 rows: direct HBM -> LDS gathers through an NBUF-deep ring.
// ---------------------------------------------------------------------------
template <int NW, int NBUF, int MAXE>
__global__ __launch_bounds__(NW * WAVE, 1) void attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * BUF_BYTES];
  __shared__ int rows_sh[MAXE];
  constexpr int THREADS = NW * WAVE;
  constexpr int LAT_PER_WAVE = TILE / NW;        // latent rows issued per wave per tile
  constexpr int ROPE_INSTR = ROPE_TILE_BYTES / 1024;
  constexpr int LOADS_PER_WAVE = LAT_PER_WAVE + (ROPE_INSTR + NW - 1) / NW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;
  Work w;
  if (!map_work<NW>(p, w)) return;
  const int h = w.hg * 16 * NW + wave * 16 + c;
  const bool head_ok = h < p.H;

  resolve_rows<THREADS>(p, w, rows_sh, tid);
  WaveAcc a;
  load_q(a, p, w.tok, h, head_ok, g);
  wait_vmcnt<0>();  // Q and index loads done: no compiler-inserted waits in the loop
  __syncthreads();

  // issue the gathers of tile k into ring slot k % NBUF
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto issue = [&](int k) {
    const uint32_t buf = smem_base + (k % NBUF) * BUF_BYTES;
    const int* rows = rows_sh + k * TILE;
#pragma unroll
    for (int j = 0; j < LAT_PER_WAVE; ++j) {
      const int r = wave * LAT_PER_WAVE + j;
      int row = rows[r];
      row = row < 0 ? ~row : row;
      dma16(p.kv + (int64_t)row * (ROW * 2) + ((lane ^ lat_flip(r)) << 4), buf + r * LAT_STRIDE);
    }
#pragma unroll
    for (int i = wave; i < ROPE_INSTR; i += NW) {
      const int r = i * 8 + (lane >> 3);
      int row = rows[r];
      row = row < 0 ? ~row : row;
      dma16(p.kv + (int64_t)row * (ROW * 2) + LATENT * 2 + (((lane & 7) ^ (r & 7)) << 4),
            buf + LAT_TILE_BYTES + i * 1024);
    }
  };

  TileAddr ad;
  ad.init(g, c);
#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (k < w.ntiles) issue(k);

  // Iteration k: wait for this wave's gathers of tile k (later tiles stay in
  // flight), one barrier (tile k visible to every wave; ring slot
  // (k - 1) % NBUF is free again), issue tile k + NBUF - 1, compute tile k.
  for (int k = 0; k < w.ntiles; ++k) {
    const int later = min(NBUF - 2, w.ntiles - 1 - k);
    if (later >= 2) wait_vmcnt<2 * LOADS_PER_WAVE>();
    else if (later == 1) wait_vmcnt<LOADS_PER_WAVE>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (k + NBUF - 1 < w.ntiles) issue(k + NBUF - 1);
    compute_tile(a, smem + (k % NBUF) * BUF_BYTES, ad, tile_valid8(rows_sh + k * TILE, g), p.scale_log2);
  }
  write_result(a, p, w.tok, w.split, h, head_ok, g);
}

// ---------------------------------------------------------------------------
// FP8 rows: register staging with dequantisation, double-buffered LDS.
// ---------------------------------------------------------------------------
template <int NW>
struct Fp8Stage {
  static constexpr int THREADS = NW * WAVE;
  // per row: 32 latent code chunks (16 codes each) + 8 rope chunks
  static constexpr int CHUNKS = 40;
  static constexpr int JOBS = (TILE * CHUNKS + THREADS - 1) / THREADS;
  u32x4 raw[JOBS];
  float scale[JOBS];

  __device__ __forceinline__ void load(const AttnParams& p, const int* rows, int tid) {
#pragma unroll
    for (int k = 0; k < JOBS; ++k) {
      const int j = tid + k * THREADS;
      raw[k] = u32x4{0u, 0u, 0u, 0u};
      scale[k] = 0.0f;
      if (j < TILE * CHUNKS) {
        const int r = j / CHUNKS, ch = j % CHUNKS;
        const int row = rows[r];
        if (row >= 0) {
          const uint8_t* base = p.kv + (int64_t)row * FP8_ROW_BYTES;
          if (ch < 32) {
            raw[k] = *(const u32x4*)(base + ch * 16);
            scale[k] = *(const float*)(base + LATENT + (ch >> 3) * 4);
          } else {
            raw[k] = *(const u32x4*)(base + LATENT + 16 + (ch - 32) * 16);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* buf, int tid) {
#pragma unroll
    for (int k = 0; k < JOBS; ++k) {
      const int j = tid + k * THREADS;
      if (j < TILE * CHUNKS) {
        const int r = j / CHUNKS, ch = j % CHUNKS;
        if (ch < 32) {
          const float sc = scale[k];
          u32x2 a0 = e4m3x4_to_bf16(raw[k][0], sc), a1 = e4m3x4_to_bf16(raw[k][1], sc);
          u32x2 a2 = e4m3x4_to_bf16(raw[k][2], sc), a3 = e4m3x4_to_bf16(raw[k][3], sc);
          *(u32x4*)(buf + lat_off(r, 2 * ch)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
          *(u32x4*)(buf + lat_off(r, 2 * ch + 1)) = u32x4{a2[0], a2[1], a3[0], a3[1]};
        } else {
          *(u32x4*)(buf + rope_off(r, ch - 32)) = raw[k];
        }
      }
    }
  }
};

template <int NW, int MAXE>
__global__ __launch_bounds__(NW * WAVE, 1) void attn_fp8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * BUF_BYTES];
  __shared__ int rows_sh[MAXE];
  constexpr int THREADS = NW * WAVE;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;
  Work w;
  if (!map_work<NW>(p, w)) return;
  const int h = w.hg * 16 * NW + wave * 16 + c;
  const bool head_ok = h < p.H;

  resolve_rows<THREADS>(p, w, rows_sh, tid);
  WaveAcc a;
  load_q(a, p, w.tok, h, head_ok, g);
  __syncthreads();

  TileAddr ad;
  ad.init(g, c);
  Fp8Stage<NW> st;
  if (w.ntiles > 0) {
    st.load(p, rows_sh, tid);
    st.store(smem, tid);
  }
  __syncthreads();
  for (int k = 0; k < w.ntiles; ++k) {
    const bool more = k + 1 < w.ntiles;
    if (more) st.load(p, rows_sh + (k + 1) * TILE, tid);
    compute_tile(a, smem + (k & 1) * BUF_BYTES, ad, tile_valid8(rows_sh + k * TILE, g), p.scale_log2);
    if (more) st.store(smem + ((k + 1) & 1) * BUF_BYTES, tid);
    __syncthreads();
  }
  write_result(a, p, w.tok, w.split, h, head_ok, g);
}

// Merge split partials: lse = log sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s.
__global__ __launch_bounds__(128) void combine_kernel(AttnParams p) {
  const int th = blockIdx.x;  // (token, head)
  const int tok = th / p.H, h = th % p.H;
  const int S = p.num_splits;
  const int64_t base = (int64_t)tok * S * p.H + h;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.part_lse[base + (int64_t)s * p.H]);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const int64_t pi = base + (int64_t)s * p.H;
      const float wgt = expf(p.part_lse[pi] - mx);
      if (wgt > 0.0f) {
        wsum += wgt;
        acc += wgt * *(const f32x4*)(p.part_o + pi * LATENT + threadIdx.x * 4);
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  *(f32x4*)(p.out + ((int64_t)tok * p.H + h) * LATENT + threadIdx.x * 4) = acc * inv;
  if (threadIdx.x == 0 && p.lse)
    p.lse[(int64_t)tok * p.H + h] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
}

// nhg16: 16-head groups per block; waves: waves per block
template <typename K>
hipError_t launch_grid(K kernel, const AttnParams& p, int nhg16, int waves, hipStream_t stream) {
  const int nhg = cdiv(p.H, 16 * nhg16);
  const int pairs = p.sv.num_tokens * p.num_splits;
  const int blocks = cdiv(pairs, 8) * 8 * nhg;
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(waves * WAVE), 0, stream, p);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_nw(const AttnParams& p, bool fp8, hipStream_t stream) {
  const int tiles_per_split = cdiv(p.split_len, TILE);
  if (fp8) return launch_grid(attn_fp8_kernel<NW, 2048>, p, NW, NW, stream);
  if (tiles_per_split * TILE <= 1024) return launch_grid(attn_bf16_kernel<NW, 4, 1024>, p, NW, NW, stream);
  return launch_grid(attn_bf16_kernel<NW, 3, 2048>, p, NW, NW, stream);
}

}  // namespace

int attn_num_splits(int num_tokens, int H, int top_k) {
  const int nw = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  const int nhg = cdiv(H, 16 * nw);
  const int items = num_tokens * nhg;
  const int max_splits = std::max(1, cdiv(top_k, 4 * TILE));
  const int s = cdiv(256, std::max(1, items));
  return std::min(std::max(s, 1), max_splits);
}

hipError_t launch_attn(const AttnParams& p, bool kv_fp8, hipStream_t stream) {
  timer_before(2, stream);
  hipError_t e;
  if (p.H <= 16) e = launch_nw<1>(p, kv_fp8, stream);
  else if (p.H <= 32) e = launch_nw<2>(p, kv_fp8, stream);
  else e = launch_nw<4>(p, kv_fp8, stream);
  timer_after(2, stream);
  if (e != hipSuccess || p.num_splits == 1) return e;
  timer_before(3, stream);
  hipLaunchKernelGGL(combine_kernel, dim3(p.sv.num_tokens * p.H), dim3(128), 0, stream, p);
  e = hipGetLastError();
  timer_after(3, stream);
  return e;
}

}  // namespace idxs
