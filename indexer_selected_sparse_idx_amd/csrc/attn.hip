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
// workgroup gathers 32 selected latent rows per tile into LDS (double
// buffered; FP8 rows are dequantised to bf16 on the way), and each wave
// owns 16 heads:
//   S^T[32 keys x 16 heads] = C_tile . Q^T   (MFMA 16x16x32, keys on M)
//   online softmax in fp32 registers (each lane holds 8 keys of one head)
//   O^T[512 x 16 heads]   += V^T . P^T       (MFMA, dv on M)
// The fp32 S^T tile is already laid out as the B operand of the second
// product once the key order inside the contraction is permuted to match;
// the V^T operand comes from the key-major LDS tile through the gfx950
// transposing LDS read (ds_read_b64_tr_b16), so V is stored only once.
// Splits (for decode occupancy) are merged by combine_kernel.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TILE = ATTN_TILE;                 // selected rows per tile
constexpr int LAT_TILE_BYTES = TILE * 1024;     // 512 bf16 per row
constexpr int ROPE_TILE_BYTES = TILE * 128;     // 64 bf16 per row
constexpr int BUF_BYTES = LAT_TILE_BYTES + ROPE_TILE_BYTES;
constexpr float LN2 = 0.69314718055994530942f;

// Swizzled LDS addresses: 16-byte chunk `ch` of row r.
__device__ __forceinline__ int lat_off(int r, int ch) { return r * 1024 + ((ch ^ (r & 15)) << 4); }
__device__ __forceinline__ int rope_off(int r, int ch) { return LAT_TILE_BYTES + r * 128 + ((ch ^ (r & 7)) << 4); }

template <int NW, bool FP8>
struct Stage {
  static constexpr int THREADS = NW * WAVE;
  // bf16 rows: 72 chunks of 16 B (64 latent + 8 rope); fp8 rows: 32 latent
  // code chunks (16 codes each) + 8 rope chunks.
  static constexpr int CHUNKS = FP8 ? 40 : 72;
  static constexpr int JOBS = (TILE * CHUNKS + THREADS - 1) / THREADS;
  u32x4 raw[JOBS];
  float scale[FP8 ? JOBS : 1];

  __device__ __forceinline__ void load(const AttnParams& p, const int32_t* idx_row, int e0, int e_hi,
                                       int b, int ctx, int tid) {
#pragma unroll
    for (int k = 0; k < JOBS; ++k) {
      const int j = tid + k * THREADS;
      raw[k] = u32x4{0u, 0u, 0u, 0u};
      if (FP8) scale[k] = 0.0f;
      if (j < TILE * CHUNKS) {
        const int r = j / CHUNKS, ch = j % CHUNKS;
        const int e = e0 + r;
        const int s = e < e_hi ? idx_row[e] : -1;
        if (s >= 0 && s < ctx) {
          const int64_t row = cache_row(p.sv, b, s);
          if (FP8) {
            const uint8_t* base = p.kv + row * FP8_ROW_BYTES;
            if (ch < 32) {
              raw[k] = *(const u32x4*)(base + ch * 16);
              scale[k] = *(const float*)(base + LATENT + (ch >> 3) * 4);
            } else {
              raw[k] = *(const u32x4*)(base + LATENT + 16 + (ch - 32) * 16);
            }
          } else {
            raw[k] = *(const u32x4*)(p.kv + row * (ROW * 2) + ch * 16);
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
        if (FP8) {
          if (ch < 32) {
            const float sc = scale[k];
            u32x2 a0 = e4m3x4_to_bf16(raw[k][0], sc), a1 = e4m3x4_to_bf16(raw[k][1], sc);
            u32x2 a2 = e4m3x4_to_bf16(raw[k][2], sc), a3 = e4m3x4_to_bf16(raw[k][3], sc);
            *(u32x4*)(buf + lat_off(r, 2 * ch)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
            *(u32x4*)(buf + lat_off(r, 2 * ch + 1)) = u32x4{a2[0], a2[1], a3[0], a3[1]};
          } else {
            *(u32x4*)(buf + rope_off(r, ch - 32)) = raw[k];
          }
        } else {
          if (ch < 64) *(u32x4*)(buf + lat_off(r, ch)) = raw[k];
          else *(u32x4*)(buf + rope_off(r, ch - 64)) = raw[k];
        }
      }
    }
  }
};

template <int NW, bool FP8>
__global__ __launch_bounds__(NW * WAVE, 1) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF_BYTES];
  __shared__ int valid_sh[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;
  const SeqView& sv = p.sv;

  // XCD-aware work mapping: workgroups are dispatched round-robin over the 8
  // XCDs, so the head groups of one (token, split) pair are placed 8 blocks
  // apart and share an XCD (and its L2) for the gathered rows.
  const int nhg = cdiv(p.H, 16 * NW);
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int hg = slot % nhg;
  const int pair = (slot / nhg) * 8 + xcd;
  if (pair >= sv.num_tokens * p.num_splits) return;
  const int tok = pair / p.num_splits;
  const int split = pair % p.num_splits;

  const int b = seq_of_token(sv, tok);
  const int ctx = sv.ctx_len[b];
  const int e_lo = split * p.split_len;
  const int e_hi = min(p.top_k, e_lo + p.split_len);
  const int ntiles = e_hi > e_lo ? cdiv(e_hi - e_lo, TILE) : 0;
  const int32_t* idx_row = p.idx + (int64_t)tok * p.top_k;

  const int h = hg * 16 * NW + wave * 16 + c;  // this lane's head (S, P, O columns)
  const bool head_ok = h < p.H;

  // Q^T operand: lane holds Q[h][32 ks + 8 g .. +8] for the 18 k-steps of 576.
  bf16x8 qb[18];
  {
    const uint16_t* qrow = p.q + ((int64_t)tok * p.H + (head_ok ? h : 0)) * ROW;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok) v = *(const u32x4*)(qrow + ks * 32 + g * 8);
      qb[ks] = as_bf16x8(v);
    }
  }

  f32x4 o[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  Stage<NW, FP8> st;
  if (ntiles > 0) {
    st.load(p, idx_row, e_lo, e_hi, b, ctx, tid);
    st.store(smem, tid);
    if (tid < TILE) {
      const int e = e_lo + tid;
      const int s = e < e_hi ? idx_row[e] : -1;
      valid_sh[0][tid] = (s >= 0 && s < ctx);
    }
  }
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    const uint8_t* buf = smem + cur * BUF_BYTES;
    const bool more = tile + 1 < ntiles;
    const int e_next = e_lo + (tile + 1) * TILE;
    if (more) st.load(p, idx_row, e_next, e_hi, b, ctx, tid);

    // ---- S^T = C . Q^T ---------------------------------------------------
    f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = mt * 16 + c;
        const int off = ks < 16 ? lat_off(r, ks * 4 + g) : rope_off(r, (ks - 16) * 4 + g);
        const bf16x8 a = *(const bf16x8*)(buf + off);
        sacc[mt] = mfma16(a, qb[ks], sacc[mt]);
      }
    }

    // ---- online softmax (base 2) --------------------------------------------
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = (j >> 2) * 16 + g * 4 + (j & 3);
      x[j] = valid_sh[cur][key] ? sacc[j >> 2][j & 3] * p.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[j]);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f;
    float pv[8];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = 0.0f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = exp2f(x[j] - m_new);
    }
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) psum += pv[j];
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pk;
    pk[0] = pack_bf16x2(pv[0], pv[1]);
    pk[1] = pack_bf16x2(pv[2], pv[3]);
    pk[2] = pack_bf16x2(pv[4], pv[5]);
    pk[3] = pack_bf16x2(pv[6], pv[7]);
    const bf16x8 pb = as_bf16x8(pk);

    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) o[nt] *= alpha;
    }

    // ---- O^T += V^T . P^T ------------------------------------------------------
    // k-slot j of lane group g is key 16 (j / 4) + 4 g + j % 4 (the S^T layout).
    const int ra = 4 * g + (c >> 2), rb = ra + 16;
    const int half = (c & 1) * 8;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const int ch = nt * 2 + ((c & 3) >> 1);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + lat_off(ra, ch) + half));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + lat_off(rb, ch) + half));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[nt] = mfma16(a, pb, o[nt]);
    }

    if (more) {
      st.store(smem + (cur ^ 1) * BUF_BYTES, tid);
      if (tid < TILE) {
        const int e = e_next + tid;
        const int s = e < e_hi ? idx_row[e] : -1;
        valid_sh[cur ^ 1][tid] = (s >= 0 && s < ctx);
      }
    }
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
  float l_tot = l_run;
  l_tot += shfl_xor(l_tot, 16);
  l_tot += shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (m_run + log2f(l_tot)) * LN2 : -INFINITY;
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
  for (int nt = 0; nt < 32; ++nt) *(f32x4*)(orow + nt * 16 + g * 4) = o[nt] * inv;
  if (g == 0 && lrow) *lrow = lse_v;
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
      const float w = expf(p.part_lse[pi] - mx);
      if (w > 0.0f) {
        wsum += w;
        acc += w * *(const f32x4*)(p.part_o + pi * LATENT + threadIdx.x * 4);
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  *(f32x4*)(p.out + ((int64_t)tok * p.H + h) * LATENT + threadIdx.x * 4) = acc * inv;
  if (threadIdx.x == 0 && p.lse)
    p.lse[(int64_t)tok * p.H + h] = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
}

template <int NW, bool FP8>
hipError_t launch_nw(const AttnParams& p, hipStream_t stream) {
  const int nhg = cdiv(p.H, 16 * NW);
  const int pairs = p.sv.num_tokens * p.num_splits;
  const int blocks = cdiv(pairs, 8) * 8 * nhg;
  hipLaunchKernelGGL((attn_kernel<NW, FP8>), dim3(blocks), dim3(NW * WAVE), 0, stream, p);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_dt(const AttnParams& p, hipStream_t stream) {
  if (p.H <= 16) return launch_nw<1, FP8>(p, stream);
  if (p.H <= 32) return launch_nw<2, FP8>(p, stream);
  return launch_nw<4, FP8>(p, stream);
}

}  // namespace

int attn_num_splits(int num_tokens, int H, int top_k) {
  const int nw = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  const int nhg = cdiv(H, 16 * nw);
  const int items = num_tokens * nhg;
  const int max_splits = std::max(1, cdiv(top_k, 2 * TILE));
  int s = cdiv(1024, std::max(1, items));
  return std::min(std::max(s, 1), max_splits);
}

hipError_t launch_attn(const AttnParams& p, bool kv_fp8, hipStream_t stream) {
  timer_before(2, stream);
  hipError_t e = kv_fp8 ? launch_dt<true>(p, stream) : launch_dt<false>(p, stream);
  timer_after(2, stream);
  if (e != hipSuccess || p.num_splits == 1) return e;
  timer_before(3, stream);
  hipLaunchKernelGGL(combine_kernel, dim3(p.sv.num_tokens * p.H), dim3(128), 0, stream, p);
  e = hipGetLastError();
  timer_after(3, stream);
  return e;
}

}  // namespace idxs
