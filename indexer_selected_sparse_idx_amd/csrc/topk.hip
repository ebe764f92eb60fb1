// Per-row Top-K selection on gfx950: radix select over order-preserving
// 32-bit keys of the fp32 scores, then an ordered compaction.
//
// Selects, for a query at position t, the m = min(K, t + 1) positions with
// the largest score, ties going to the lower position ("selects the Top-K
// most relevant positions": section "Index-Based Sparse Attention" of Day 0
// Inference Support for New LLM Architectures; the in-place index selection
// of its fused indexer sketch; the tie rule is this library's reading).
//
// 1. Four 8-bit digit passes (most significant first) build an LDS histogram
//    of the keys that share the digits chosen so far; a one-wave suffix scan
//    picks the digit whose bucket holds the m-th largest key.  After the last
//    pass the exact threshold key tau and the number `need` of tau-valued
//    positions to take are known.
// 2. One ordered pass over the row: wavefront ballots and popcount prefixes
//    give every key > tau and the first `need` keys == tau (lowest positions
//    first) their output slots.
// Rows with t + 1 <= K skip the selection: every position is taken.
#include "common.h"
#include "kernels.h"

namespace idxs {

namespace {

constexpr int TOPK_THREADS = 512;
constexpr int TOPK_WAVES = TOPK_THREADS / WAVE;

__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_above;
  __shared__ uint32_t wave_gt[TOPK_WAVES], wave_eq[TOPK_WAVES];

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

  // ---- 1. radix passes ----------------------------------------------------
  uint32_t prefix = 0;  // digits chosen so far
  uint32_t rem = m;     // positions still to take inside the current bucket
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += TOPK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += TOPK_THREADS) {
      const uint32_t key = score_key(row[i]);
      if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
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
      // suf = number of keys in bins >= 4L
      const uint32_t s3 = suf - h0 - h1 - h2;  // bins >= 4L+3
      const uint32_t s2 = s3 + h2, s1 = s2 + h1, s0 = suf;
      const uint32_t above3 = s3 - h3;
      // the chosen digit d has S(d) >= rem > S(d + 1)
      if (s3 >= rem && above3 < rem) { sh_digit = 4 * lane + 3; sh_above = above3; }
      else if (s2 >= rem && s3 < rem) { sh_digit = 4 * lane + 2; sh_above = s3; }
      else if (s1 >= rem && s2 < rem) { sh_digit = 4 * lane + 1; sh_above = s2; }
      else if (s0 >= rem && s1 < rem) { sh_digit = 4 * lane; sh_above = s1; }
    }
    __syncthreads();
    prefix = (prefix << 8) | sh_digit;
    rem -= sh_above;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const uint32_t need = rem;          // tau-valued positions to take
  const uint32_t n_gt = m - need;     // positions with key > tau

  // ---- 2. ordered compaction ------------------------------------------------
  uint32_t base_gt = 0, base_eq = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = 0; i0 < n; i0 += TOPK_THREADS) {
    if (base_eq >= need && base_gt >= n_gt) break;
    const int i = i0 + tid;
    uint32_t key = 0;
    if (i < n) key = score_key(row[i]);
    const bool gt = i < n && key > tau;
    const bool eq = i < n && key == tau;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    if (lane == 0) { wave_gt[wave] = __popcll(bgt); wave_eq[wave] = __popcll(beq); }
    __syncthreads();
    uint32_t off_gt = base_gt, off_eq = base_eq, tot_gt = 0, tot_eq = 0;
#pragma unroll
    for (int w = 0; w < TOPK_WAVES; ++w) {
      const uint32_t a = wave_gt[w], e = wave_eq[w];
      if (w < wave) { off_gt += a; off_eq += e; }
      tot_gt += a; tot_eq += e;
    }
    if (gt) {
      const uint32_t slot = off_gt + __popcll(bgt & lt_mask);
      if (slot < n_gt) out[slot] = i;
    }
    if (eq) {
      const uint32_t slot = off_eq + __popcll(beq & lt_mask);
      if (slot < need) out[n_gt + slot] = i;
    }
    base_gt += tot_gt;
    base_eq += tot_eq;
    __syncthreads();
  }
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
