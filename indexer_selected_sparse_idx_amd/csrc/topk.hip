// Per-row Top-K selection on gfx950: radix select over order-preserving
// 32-bit keys of the fp32 scores, then an ordered compaction.
//
// Selects, for a query at position t, the m = min(K, t + 1) positions with
// the largest score, ties going to the lower position ("selects the Top-K
// most relevant positions": section "Index-Based Sparse Attention" of Day 0
// Inference Support for New LLM Architectures; the in-place index selection
// of its fused indexer sketch; the tie rule is this library's reading).
//
// One workgroup (16 waves) per row:
// 1. The score kernel has already histogrammed the top 11 bits of every key
//    of the row.  A block-wide suffix scan of that histogram gives the bucket
//    d1 holding the m-th largest key, the count above it and its size.
// 2. One ordered streaming pass over the fp32 score row (4 keys per lane per
//    access): keys in buckets above d1 are emitted directly; keys in d1 are
//    appended, with their positions, to an LDS candidate list, in position
//    order (wavefront prefix sums over per-lane counts, one barrier per 4096
//    keys).
// 3. The candidates (a few thousand at most for smooth score distributions)
//    go through the radix select below; when d1 holds more than the LDS
//    capacity (massive ties) the whole row goes through it instead, read from
//    the score row.
// Radix select over a key list:
// a. Up to four 8-bit digit passes, most significant first, histogram the
//    keys that share the digits chosen so far.  Every wave owns a private
//    LDS histogram (merged after the pass): integer-valued scores put most
//    keys into a few bins, and same-address atomics from different waves
//    would serialise.  A one-wave suffix scan picks the digit whose bucket
//    holds the m-th largest key; when that bucket is taken whole the passes
//    stop early.
// b. Ordered compaction: each wave owns a contiguous segment of the list,
//    counts its keys above / equal to the threshold, and after one exclusive
//    scan over the waves emits them in position order (a wavefront prefix
//    sum over the per-lane counts), so equal keys are taken lowest position
//    first.
// Rows with t + 1 <= K skip the selection: every position is taken.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / WAVE;
constexpr int CAP = 12288;   // LDS candidate capacity (keys + positions)
constexpr int UNROLL = 4;   // 4-key vector accesses in flight per lane

// Key source: the LDS copy of the row, or the fp32 score row itself.
template <bool IN_LDS>
struct Keys {
  const uint32_t* lds;
  const float* row;
  int n;
  // keys i .. i+3 (i % 4 == 0); positions >= n read as 0 (never selected)
  __device__ __forceinline__ u32x4 get4(int i) const {
    u32x4 k;
    if (i + 3 < n) {
      if (IN_LDS) {
        k = *(const u32x4*)(lds + i);
      } else {
        const f32x4 f = *(const f32x4*)(row + i);
        k = u32x4{score_key(f[0]), score_key(f[1]), score_key(f[2]), score_key(f[3])};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k[e] = i + e < n ? (IN_LDS ? lds[i + e] : score_key(row[i + e])) : 0u;
    }
    return k;
  }
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Digit passes of the radix select: FIXED top bits are already known to be
// equal for every key of the list (0, or SCORE_HIST_BITS for the candidates
// of one histogram bucket); the remaining bits go 8 at a time, the last pass
// taking what is left.
template <int FIXED>
struct Digits {
  static constexpr int REST = 32 - FIXED;
  static constexpr int PASSES = (REST + 7) / 8;
  __device__ __forceinline__ static int width(int pass) { return pass + 1 < PASSES ? 8 : REST - 8 * (PASSES - 1); }
  __device__ __forceinline__ static int shift(int pass) {
    int s = REST;
    for (int q = 0; q <= pass; ++q) s -= width(q);
    return s;
  }
};

// Select the m largest of n keys (ties: lowest index first) and write their
// positions (pos[i], or i when pos is null) to out[0 .. m).  Every key's top
// FIXED bits equal prefix0.
template <bool IN_LDS, int FIXED>
__device__ void select_row(const Keys<IN_LDS>& keys, int n, int m, int32_t* out, const int32_t* pos, uint32_t* hist,
                           uint32_t* whist, uint32_t* wcnt, uint32_t prefix0) {
  typedef Digits<FIXED> D;
  __shared__ uint32_t sh_digit, sh_above, sh_whole;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- radix passes ----------------------------------------------------------
  uint32_t prefix = prefix0;  // top bits chosen so far
  uint32_t rem = m;           // positions still to take inside the current bucket
  int cshift = 32 - FIXED;    // keys match the prefix on bits >= cshift
  uint32_t* my_hist = whist + wave * 256;
  const int n4 = (n + 3) / 4 * 4;
  for (int pass = 0; pass < D::PASSES; ++pass) {
    const int shift = D::shift(pass);
    const uint32_t dmask = (1u << D::width(pass)) - 1u;
#pragma unroll
    for (int j = 0; j < 4; ++j) my_hist[lane + 64 * j] = 0;
    for (int i0 = 4 * tid; i0 < n4; i0 += 4 * TOPK_THREADS * UNROLL) {
      u32x4 k[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = i0 + u * 4 * TOPK_THREADS;
        k[u] = i < n4 ? keys.get4(i) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int i = i0 + u * 4 * TOPK_THREADS;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = k[u][e];
          const bool in = i + e < n && (cshift >= 32 || (key >> cshift) == prefix);
          if (in) atomicAdd(&my_hist[(key >> shift) & dmask], 1u);
        }
      }
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t tot = 0;
#pragma unroll
      for (int w = 0; w < TOPK_WAVES; ++w) tot += whist[w * 256 + tid];
      hist[tid] = tot;
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns bins 4L..4L+3; suffix sums from the top bin downwards
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
      const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      uint32_t suf = h0 + h1 + h2 + h3;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      const uint32_t s3 = suf - h0 - h1 - h2;  // keys in bins >= 4L+3
      const uint32_t s2 = s3 + h2, s1 = s2 + h1, s0 = suf;
      const uint32_t a3 = s3 - h3;
      // the chosen digit d has S(d) >= rem > S(d + 1)
      int d = -1;
      uint32_t above = 0, cnt = 0;
      if (s3 >= rem && a3 < rem) { d = 4 * lane + 3; above = a3; cnt = h3; }
      else if (s2 >= rem && s3 < rem) { d = 4 * lane + 2; above = s3; cnt = h2; }
      else if (s1 >= rem && s2 < rem) { d = 4 * lane + 1; above = s2; cnt = h1; }
      else if (s0 >= rem && s1 < rem) { d = 4 * lane; above = s1; cnt = h0; }
      if (d >= 0) {
        sh_digit = d;
        sh_above = above;
        sh_whole = (cnt == rem - above);  // the whole bucket is taken
      }
    }
    __syncthreads();
    prefix = (prefix << D::width(pass)) | sh_digit;
    rem -= sh_above;
    cshift = shift;
    const bool whole = sh_whole;
    __syncthreads();
    if (whole) break;
  }
  // compare keys on their bits >= cshift against `prefix`
  const uint32_t need = rem;       // prefix-equal positions to take
  const uint32_t n_gt = m - need;  // positions above the prefix

  // ---- ordered compaction over per-wave segments (multiples of 256 keys) ------
  const int seg = (n4 + TOPK_WAVES * 256 - 1) / (TOPK_WAVES * 256) * 256;
  const int lo = wave * seg, hi = min(n4, lo + seg);
  uint32_t c_gt = 0, c_eq = 0;
  for (int i0 = lo; i0 < hi; i0 += 256) {
    const int i = i0 + 4 * lane;
    if (i < hi) {
      const u32x4 k = keys.get4(i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t kk = (uint64_t)k[e] >> cshift;
        const bool valid = i + e < n;
        c_gt += (valid && kk > prefix);
        c_eq += (valid && kk == prefix);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    c_gt += __shfl_xor(c_gt, off);
    c_eq += __shfl_xor(c_eq, off);
  }
  if (lane == 0) { wcnt[wave] = c_gt; wcnt[TOPK_WAVES + wave] = c_eq; }
  __syncthreads();
  uint32_t base_gt = 0, base_eq = 0;
  for (int w = 0; w < wave; ++w) { base_gt += wcnt[w]; base_eq += wcnt[TOPK_WAVES + w]; }
  if (base_eq >= need && c_gt == 0) return;
  for (int i0 = lo; i0 < hi; i0 += 256) {
    const int i = i0 + 4 * lane;
    uint32_t fg = 0, fe = 0;  // per-element flags, bit e
    if (i < hi) {
      const u32x4 k = keys.get4(i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t kk = (uint64_t)k[e] >> cshift;
        const bool valid = i + e < n;
        fg |= (uint32_t)(valid && kk > prefix) << e;
        fe |= (uint32_t)(valid && kk == prefix) << e;
      }
    }
    const uint32_t ng = __popc(fg), ne = __popc(fe);
    const uint32_t sg = wave_incl_scan(ng, lane), se = wave_incl_scan(ne, lane);
    uint32_t pg = base_gt + sg - ng, pe = base_eq + se - ne;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((fg >> e) & 1u) {
        if (pg < n_gt) out[pg] = pos ? pos[i + e] : i + e;
        ++pg;
      }
      if ((fe >> e) & 1u) {
        if (pe < need) out[n_gt + pe] = pos ? pos[i + e] : i + e;
        ++pe;
      }
    }
    base_gt += __shfl(sg, 63);
    base_eq += __shfl(se, 63);
  }
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t cand_key[CAP];
  __shared__ __attribute__((aligned(16))) int32_t cand_pos[CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t whist[TOPK_WAVES * 256];
  __shared__ uint32_t wcnt[2 * TOPK_WAVES];
  __shared__ uint32_t wtot[2][TOPK_WAVES][2];
  __shared__ uint32_t sh_d1, sh_above1, sh_cnt1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const SeqView& sv = p.sv;
  const int tok = blockIdx.x;
  const int b = seq_of_token(sv, tok);
  const int ql = q_len(sv, b);
  const int t = sv.ctx_len[b] - ql + (tok - first_token(sv, b));
  const int n = t + 1;
  const int K = p.top_k;
  const int m = min(K, n);
  const float* row = p.scores + (int64_t)tok * p.score_stride;
  int32_t* out = p.out_idx + (int64_t)tok * K;

  for (int i = m + tid; i < K; i += TOPK_THREADS) out[i] = -1;
  if (m == n) {
    for (int i = tid; i < n; i += TOPK_THREADS) out[i] = i;
    return;
  }

  // ---- 1. the bucket of the m-th largest key, from the row histogram ----------
  {
    const uint32_t* gh = p.hist + (int64_t)tok * SCORE_HIST_BINS;
    const uint32_t h0 = gh[2 * tid], h1 = gh[2 * tid + 1];
    uint32_t suf = h0 + h1;  // suffix over this wave's lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suf, off);
      if (lane + off < 64) suf += o;
    }
    if (lane == 0) wcnt[wave] = suf;
    __syncthreads();
    uint32_t above_waves = 0;
    for (int w = wave + 1; w < TOPK_WAVES; ++w) above_waves += wcnt[w];
    const uint32_t s0 = suf + above_waves;  // keys in bins >= 2 tid
    const uint32_t s1 = s0 - h0, s2 = s1 - h1;
    const uint32_t um = (uint32_t)m;
    if (s1 >= um && s2 < um) { sh_d1 = 2 * tid + 1; sh_above1 = s2; sh_cnt1 = h1; }
    else if (s0 >= um && s1 < um) { sh_d1 = 2 * tid; sh_above1 = s1; sh_cnt1 = h0; }
    __syncthreads();
  }
  const uint32_t d1 = sh_d1, above1 = sh_above1, cnt1 = sh_cnt1;
  if (cnt1 > (uint32_t)CAP) {  // massive ties: select over the whole row
    select_row<false, 0>(Keys<false>{nullptr, row, n}, n, m, out, nullptr, hist, whist, wcnt, 0u);
    return;
  }

  // ---- 2. ordered extraction: above d1 -> output, in d1 -> candidates ------------
  const Keys<false> src{nullptr, row, n};
  const int n4 = (n + 3) / 4 * 4;
  uint32_t base_g = 0, base_c = 0;
  int par = 0;
  constexpr int CHUNK = 4 * TOPK_THREADS;
  for (int s0 = 0; s0 < n4; s0 += CHUNK * UNROLL) {
    u32x4 kk[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int i = s0 + u * CHUNK + 4 * tid;
      kk[u] = i < n4 ? src.get4(i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c0 = s0 + u * CHUNK;
      if (c0 >= n4) break;  // uniform
      const int i = c0 + 4 * tid;
      uint32_t fg = 0, fc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t top = kk[u][e] >> (32 - SCORE_HIST_BITS);
        const bool valid = i + e < n;
        fg |= (uint32_t)(valid && top > d1) << e;
        fc |= (uint32_t)(valid && top == d1) << e;
      }
      const uint32_t ng = __popc(fg), nc = __popc(fc);
      const uint32_t sg = wave_incl_scan(ng, lane), sc = wave_incl_scan(nc, lane);
      if (lane == 63) { wtot[par][wave][0] = sg; wtot[par][wave][1] = sc; }
      __syncthreads();
      uint32_t og = base_g + sg - ng, oc = base_c + sc - nc, tg = 0, tc = 0;
#pragma unroll
      for (int w = 0; w < TOPK_WAVES; ++w) {
        const uint32_t a = wtot[par][w][0], c = wtot[par][w][1];
        if (w < wave) { og += a; oc += c; }
        tg += a;
        tc += c;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((fg >> e) & 1u) {
          if (og < above1) out[og] = i + e;
          ++og;
        }
        if ((fc >> e) & 1u) {
          if (oc < (uint32_t)CAP) { cand_key[oc] = kk[u][e]; cand_pos[oc] = i + e; }
          ++oc;
        }
      }
      base_g += tg;
      base_c += tc;
      par ^= 1;
    }
  }
  __syncthreads();

  // ---- 3. the remaining m - above1 positions come from the candidates -------------
  select_row<true, SCORE_HIST_BITS>(Keys<true>{cand_key, nullptr, (int)cnt1}, (int)cnt1, m - (int)above1,
                                    out + above1, cand_pos, hist, whist, wcnt, d1);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  timer_before(1, stream);
  hipLaunchKernelGGL(topk_kernel, dim3(p.sv.num_tokens), dim3(TOPK_THREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  timer_after(1, stream);
  return e;
}

}  // namespace idxs
