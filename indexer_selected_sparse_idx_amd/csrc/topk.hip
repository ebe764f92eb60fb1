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
// 1. Rows of up to 32768 candidates are converted to keys once and kept in
//    LDS; longer rows are re-read from the (L2-resident) score row.
// 2. Up to four 8-bit digit passes, most significant first, histogram the
//    keys that share the digits chosen so far.  Histogram updates are
//    aggregated per wavefront (ballot on the leading lane's bin) because
//    integer-valued scores put most keys into a few bins.  A one-wave suffix
//    scan picks the digit whose bucket holds the m-th largest key; when that
//    bucket is taken whole the passes stop early.
// 3. Ordered compaction: each wave owns a contiguous segment of the row,
//    counts its keys above / equal to the threshold, and after one exclusive
//    scan over the waves emits them with ballot + popcount prefixes, so the
//    equal keys are taken lowest position first.
// Rows with t + 1 <= K skip the selection: every position is taken.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / WAVE;
constexpr int LDS_KEYS = 32768;

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// hist[bin] += 1 for every active lane, one LDS atomic per distinct bin for
// the first few bins, plain atomics for whatever remains.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t bin, int lane) {
  uint64_t act = __ballot(active);
#pragma unroll 1
  for (int it = 0; it < 4 && act; ++it) {
    const int leader = __builtin_ctzll(act);
    const uint32_t lbin = __shfl(bin, leader);
    const uint64_t same = __ballot(active && bin == lbin);
    if (lane == leader) atomicAdd(&hist[lbin], (uint32_t)__popcll(same));
    if (bin == lbin) active = false;
    act &= ~same;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

template <bool IN_LDS>
__device__ __forceinline__ uint32_t key_at(const uint32_t* keys, const float* row, int i) {
  return IN_LDS ? keys[i] : score_key(row[i]);
}

template <bool IN_LDS>
__device__ void select_row(const float* row, int n, int m, int K, int32_t* out, uint32_t* keys, uint32_t* hist,
                           uint32_t* wcnt) {
  __shared__ uint32_t sh_digit, sh_above, sh_whole;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (IN_LDS) {
    for (int i = tid; i < n; i += TOPK_THREADS) keys[i] = score_key(row[i]);
  }
  // ---- radix passes ----------------------------------------------------------
  uint32_t prefix = 0;  // digits chosen so far
  uint32_t rem = m;     // positions still to take inside the current bucket
  int level = 0;        // number of digits fixed
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += TOPK_THREADS) hist[i] = 0;
    __syncthreads();
    const int n_pad = (n + TOPK_THREADS - 1) / TOPK_THREADS * TOPK_THREADS;
    for (int i = tid; i < n_pad; i += TOPK_THREADS) {
      uint32_t key = 0;
      bool in = false;
      if (i < n) {
        key = key_at<IN_LDS>(keys, row, i);
        in = pass == 0 || (key >> (shift + 8)) == prefix;
      }
      hist_add(hist, in, (key >> shift) & 255u, lane);
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
    prefix = (prefix << 8) | sh_digit;
    rem -= sh_above;
    level = pass + 1;
    const bool whole = sh_whole;
    __syncthreads();
    if (whole) break;
  }
  // compare keys on their top 8*level bits against `prefix`
  const int cshift = 32 - 8 * level;
  const uint32_t need = rem;       // prefix-equal positions to take
  const uint32_t n_gt = m - need;  // positions above the prefix

  // ---- ordered compaction over per-wave segments ---------------------------------
  const int seg = (n + TOPK_WAVES - 1) / TOPK_WAVES;
  const int lo = wave * seg, hi = min(n, lo + seg);
  uint32_t c_gt = 0, c_eq = 0;
  for (int i0 = lo; i0 < hi; i0 += 64) {
    const int i = i0 + lane;
    bool gt = false, eq = false;
    if (i < hi) {
      const uint64_t k = (uint64_t)key_at<IN_LDS>(keys, row, i) >> cshift;
      gt = k > prefix;
      eq = k == prefix;
    }
    c_gt += __popcll(__ballot(gt));
    c_eq += __popcll(__ballot(eq));
  }
  if (lane == 0) { wcnt[wave] = c_gt; wcnt[TOPK_WAVES + wave] = c_eq; }
  __syncthreads();
  uint32_t base_gt = 0, base_eq = 0;
  for (int w = 0; w < wave; ++w) { base_gt += wcnt[w]; base_eq += wcnt[TOPK_WAVES + w]; }
  if (base_eq >= need && c_gt == 0) return;
  const uint64_t below = lanes_below(lane);
  for (int i0 = lo; i0 < hi; i0 += 64) {
    const int i = i0 + lane;
    bool gt = false, eq = false;
    if (i < hi) {
      const uint64_t k = (uint64_t)key_at<IN_LDS>(keys, row, i) >> cshift;
      gt = k > prefix;
      eq = k == prefix;
    }
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (gt) {
      const uint32_t slot = base_gt + __popcll(bg & below);
      if (slot < n_gt) out[slot] = i;
    }
    if (eq) {
      const uint32_t slot = base_eq + __popcll(be & below);
      if (slot < need) out[n_gt + slot] = i;
    }
    base_gt += __popcll(bg);
    base_eq += __popcll(be);
  }
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(TopkParams p) {
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wcnt[2 * TOPK_WAVES];

  const int tid = threadIdx.x;
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
  if (n <= LDS_KEYS && p.keys_in_lds) select_row<true>(row, n, m, K, out, dyn, hist, wcnt);
  else select_row<false>(row, n, m, K, out, dyn, hist, wcnt);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p0, hipStream_t stream) {
  TopkParams p = p0;
  // LDS key cache only when some row can use it (dynamic LDS is sized per launch)
  p.keys_in_lds = p.sv.max_ctx_len > p.top_k ? 1 : 0;
  const size_t dyn = p.keys_in_lds ? (size_t)std::min(p.sv.max_ctx_len, LDS_KEYS) * sizeof(uint32_t) : 0;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              LDS_KEYS * (int)sizeof(uint32_t));
    attr_set = true;
  }
  timer_before(1, stream);
  hipLaunchKernelGGL(topk_kernel, dim3(p.sv.num_tokens), dim3(TOPK_THREADS), dyn, stream, p);
  hipError_t e = hipGetLastError();
  timer_after(1, stream);
  return e;
}

}  // namespace idxs
