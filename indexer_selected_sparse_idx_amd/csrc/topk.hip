// Per-row Top-K selection on gfx950: radix select over order-preserving
// 32-bit keys of the fp32 scores, then an ordered compaction.
//
// Selects, for a query at position t, the m = min(K, t + 1) positions with
// the largest score, ties going to the lower position ("selects the Top-K
// most relevant positions": section "Index-Based Sparse Attention" of Day 0
// Inference Support for New LLM Architectures; the in-place index selection
// of its fused indexer sketch; the tie rule is this library's reading).
//
// These kernels select for the decode score kernel (and for prefill batches
// whose block tables the prefill kernel cannot stage; the prefill kernel
// otherwise selects on its own).  The score kernel has already histogrammed
// the top 11 bits of every key of the row, so the bucket d1 holding the m-th
// largest key is known before the row is read again.  Two launches then
// select (details below, above the kernels): a compaction pass that many
// workgroups run over chunks of every row (keys above d1 are taken, keys in
// d1 kept as candidates, both in position order), and one workgroup per row
// that gathers them and runs the radix select over the candidates (a few
// thousand at most for smooth score distributions); when d1 holds more than
// the LDS capacity (massive ties) the radix select runs over the whole score
// row.
//
// Radix select over a key list:
// a. Up to four 8-bit digit passes, most significant first, histogram the
//    keys that share the digits chosen so far.  Every wave owns a private
//    LDS histogram (merged after the pass): integer-valued scores put most
//    keys into a few bins, and same-address atomics from different waves
//    would serialise.  A one-wave suffix scan picks the digit whose bucket
//    holds the m-th largest key; when that bucket is taken whole, or when
//    no counted key has a bit set below the digit (the keys of the bucket
//    are then all equal), the passes stop early.
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
constexpr int CAP = 24576;   // LDS candidate capacity (a packed word and a chunk byte each)
constexpr int UNROLL = 4;   // 4-key vector accesses in flight per lane

// Key source: candidate words in LDS (low key bits << 11 | offset in the
// chunk, as the compaction pass packs them; `hi` supplies the key bits above
// them), or the fp32 score row itself.
template <bool IN_LDS>
struct Keys {
  const uint32_t* lds;
  const float* row;
  int n;
  uint32_t hi;
  __device__ __forceinline__ uint32_t from_word(uint32_t w) const { return (w >> 11) | hi; }
  // keys i .. i+3 (i % 4 == 0); positions >= n read as 0 (never selected)
  __device__ __forceinline__ u32x4 get4(int i) const {
    u32x4 k;
    if (i + 3 < n) {
      if (IN_LDS) {
        const u32x4 w = *(const u32x4*)(lds + i);
        k = u32x4{from_word(w[0]), from_word(w[1]), from_word(w[2]), from_word(w[3])};
      } else {
        const f32x4 f = *(const f32x4*)(row + i);
        k = u32x4{score_key(f[0]), score_key(f[1]), score_key(f[2]), score_key(f[3])};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k[e] = i + e < n ? (IN_LDS ? from_word(lds[i + e]) : score_key(row[i + e])) : 0u;
    }
    return k;
  }
};

// Position of list entry i: the entry itself (a whole score row), or, for
// the candidate words, the entry's chunk (one byte per entry, stored beside
// the words) plus the word's offset in it.
struct RowPos {
  __device__ __forceinline__ int operator()(int i) const { return i; }
};
struct CandPos {
  const uint32_t* w;
  const uint8_t* chunk;
  __device__ __forceinline__ int operator()(int i) const {
    return (int)chunk[i] * TOPK_CHUNK + (int)(w[i] & (TOPK_CHUNK - 1));
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
// positions pos(i) to out[0 .. m).  Every key's top FIXED bits equal prefix0.
template <bool IN_LDS, int FIXED, typename Pos>
__device__ void select_row(const Keys<IN_LDS>& keys, int n, int m, int32_t* out, const Pos& pos, uint32_t* hist,
                           uint32_t* whist, uint32_t* wcnt, uint32_t prefix0) {
  typedef Digits<FIXED> D;
  __shared__ uint32_t sh_digit, sh_above, sh_whole, sh_zero;
  __shared__ uint32_t wlow[TOPK_WAVES];  // per wave: OR of the counted keys' bits below the digit
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
    const uint32_t lowmask = (1u << shift) - 1u;
    uint32_t low = 0;
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
          if (in) {
            atomicAdd(&my_hist[(key >> shift) & dmask], 1u);
            low |= key & lowmask;
          }
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) low |= __shfl_xor(low, off);
    if (lane == 0) wlow[wave] = low;
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
      // no counted key has a bit set below this digit (integer-valued
      // scores leave the low mantissa bits empty): the later passes would
      // each pick digit 0 with nothing above it
      const bool zero = __builtin_amdgcn_ballot_w64(lane < TOPK_WAVES && wlow[lane] != 0u) == 0;
      if (d >= 0) {
        sh_digit = d;
        sh_above = above;
        sh_whole = (cnt == rem - above);  // the whole bucket is taken
        sh_zero = zero;
      }
    }
    __syncthreads();
    prefix = (prefix << D::width(pass)) | sh_digit;
    rem -= sh_above;
    cshift = shift;
    const bool whole = sh_whole, zero = sh_zero;
    __syncthreads();
    if (whole) break;
    if (zero) {  // the keys of the chosen bucket are all equal to prefix << shift
      prefix <<= shift;
      cshift = 0;
      break;
    }
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
        if (pg < n_gt) out[pg] = pos(i + e);
        ++pg;
      }
      if ((fe >> e) & 1u) {
        if (pe < need) out[n_gt + pe] = pos(i + e);
        ++pe;
      }
    }
    base_gt += __shfl(sg, 63);
    base_eq += __shfl(se, 63);
  }
}

// ---------------------------------------------------------------------------
// The selection as two launches.
// Both launches start from the row's threshold: the bucket d1 holding the
// m-th largest key, the count above it and its size, which one wave derives
// from the row histogram (every workgroup of a row derives the same).
//   emit    one workgroup per (row, TOPK_CHUNK keys): the chunk's keys above
//           d1 and in d1 are compacted, in position order, into the chunk's
//           own part of the score row (just read, and read by no one else):
//           first the positions above d1, then the d1 keys packed as
//           (low 21 key bits << 11) | (offset in the chunk); the two counts
//           go to a per-chunk table.
//   select  one workgroup per row: the positions above d1 go to the output,
//           chunk after chunk; the packed d1 words go into LDS in position
//           order (4 bytes each, with a byte for the chunk) and the radix
//           select above takes the remaining m - above1 of them.
// Rows with t + 1 <= K take every position.  Rows whose d1 bucket exceeds the
// LDS capacity (massive ties), or with more chunks than the select tracks,
// are left alone by emit and select over the whole score row.
// ---------------------------------------------------------------------------
constexpr int TKE_THREADS = 256;                     // 8 keys per thread
constexpr int TKE_WAVES = TKE_THREADS / WAVE;
constexpr int TK_MAXCH = 256;                        // chunks per row the select tracks (byte chunk ids)
constexpr uint32_t TK_PARTIAL = 0, TK_ALL = 1, TK_WHOLE_ROW = 2;
static_assert(TOPK_CHUNK == 2048 && TOPK_CHUNK == 8 * TKE_THREADS, "11-bit chunk offsets, 8 keys per thread");

// t + 1 for the query token `tok`
__device__ __forceinline__ int row_len(const SeqView& sv, int tok) {
  const int b = seq_of_token(sv, tok);
  return sv.ctx_len[b] - q_len(sv, b) + (tok - first_token(sv, b)) + 1;
}

// The row's threshold record, computed by one wave from the row histogram
// (lane L holds bins 32 L .. 32 L + 31): d1, the bucket holding the m-th
// largest key, above1 = the keys in higher buckets, cnt1 = the keys in d1.
struct TopkRow {
  uint32_t mode, d1, above1, cnt1;
};

__device__ TopkRow row_threshold(const TopkParams& p, int tok, int n, int lane) {
  const uint32_t m = (uint32_t)min(p.top_k, n);
  TopkRow r = {TK_ALL, 0u, 0u, 0u};
  if (m == (uint32_t)n) return r;
  const u32x4* gh = (const u32x4*)(p.hist + (int64_t)tok * SCORE_HIST_BINS + 32 * lane);
  uint32_t h[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 v = gh[j];
    h[4 * j] = v[0]; h[4 * j + 1] = v[1]; h[4 * j + 2] = v[2]; h[4 * j + 3] = v[3];
  }
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) tot += h[j];
  uint32_t suf = tot;  // keys in the bins of lanes >= L
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(suf, off);
    if (lane + off < 64) suf += o;
  }
  uint32_t run = suf - tot;  // keys in the bins above this lane's
  uint32_t d1 = 0, above1 = 0, cnt1 = 0;
  bool found = false;
#pragma unroll
  for (int j = 31; j >= 0; --j) {
    if (run < m && run + h[j] >= m) {
      found = true;
      d1 = 32 * lane + j;
      above1 = run;
      cnt1 = h[j];
    }
    run += h[j];
  }
  const uint64_t fm = __builtin_amdgcn_ballot_w64(found);
  if (fm == 0) {
    r.mode = TK_WHOLE_ROW;  // (a histogram that does not add up to the row: select from the scores)
  } else {
    const int src = __builtin_ctzll(fm);
    r.d1 = __builtin_amdgcn_readlane(d1, src);
    r.above1 = __builtin_amdgcn_readlane(above1, src);
    r.cnt1 = __builtin_amdgcn_readlane(cnt1, src);
    r.mode = (r.cnt1 > (uint32_t)CAP || cdiv(n, TOPK_CHUNK) > TK_MAXCH) ? TK_WHOLE_ROW : TK_PARTIAL;
  }
  return r;
}

__global__ __launch_bounds__(TKE_THREADS) void topk_emit_kernel(TopkParams p) {
  __shared__ uint32_t wt[2][TKE_WAVES];
  __shared__ TopkRow sh_r;
  const int tok = blockIdx.x, chunk = blockIdx.y;
  const int n = row_len(p.sv, tok);
  const int c0 = chunk * TOPK_CHUNK;
  if (c0 >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* row = p.scores + (int64_t)tok * p.score_stride;
  const Keys<false> src{nullptr, row, n, 0u};
  const int i = c0 + 8 * tid;
  const u32x4 k0 = i < n ? src.get4(i) : u32x4{0u, 0u, 0u, 0u};
  const u32x4 k1 = i + 4 < n ? src.get4(i + 4) : u32x4{0u, 0u, 0u, 0u};
  // every workgroup of the row derives the same threshold from the histogram
  if (wave == 0) {
    const TopkRow rr = row_threshold(p, tok, n, lane);
    if (lane == 0) sh_r = rr;
  }
  __syncthreads();
  const TopkRow r = sh_r;
  if (r.mode != TK_PARTIAL) return;
  const uint32_t key[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
  uint32_t fg = 0, fe = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t top = key[e] >> (32 - SCORE_HIST_BITS);
    const bool valid = i + e < n;
    fg |= (uint32_t)(valid && top > r.d1) << e;
    fe |= (uint32_t)(valid && top == r.d1) << e;
  }
  const uint32_t ng = __popc(fg), ne = __popc(fe);
  const uint32_t sg = wave_incl_scan(ng, lane), se = wave_incl_scan(ne, lane);
  if (lane == 63) { wt[0][wave] = sg; wt[1][wave] = se; }
  __syncthreads();  // every key of the chunk has been read: its storage is free
  uint32_t og = sg - ng, oe = se - ne, tg = 0, te = 0;
#pragma unroll
  for (int w = 0; w < TKE_WAVES; ++w) {
    const uint32_t a = wt[0][w], c = wt[1][w];
    if (w < wave) { og += a; oe += c; }
    tg += a;
    te += c;
  }
  uint32_t* seg = (uint32_t*)(row + c0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if ((fg >> e) & 1u) seg[og++] = (uint32_t)(i + e);
    if ((fe >> e) & 1u) seg[tg + oe++] = ((key[e] & ((1u << (32 - SCORE_HIST_BITS)) - 1u)) << 11) | (uint32_t)(i + e - c0);
  }
  if (tid == 0) {
    uint32_t* cc = p.chunk_cnt + ((int64_t)tok * p.nch_stride + chunk) * 2;
    cc[0] = tg;
    cc[1] = te;
  }
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_select_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t cand_w[CAP];
  __shared__ uint8_t cand_c[CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t whist[TOPK_WAVES * 256];
  __shared__ uint32_t wcnt[2 * TOPK_WAVES];
  __shared__ uint32_t choff[2][TK_MAXCH], chcnt[2][TK_MAXCH];
  __shared__ TopkRow sh_r;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tok = blockIdx.x;
  const int n = row_len(p.sv, tok);
  const int K = p.top_k;
  const int m = min(K, n);
  const float* row = p.scores + (int64_t)tok * p.score_stride;
  int32_t* out = p.out_idx + (int64_t)tok * K;
  for (int i = m + tid; i < K; i += TOPK_THREADS) out[i] = -1;
  if (wave == 0) {
    const TopkRow rr = row_threshold(p, tok, n, lane);
    if (lane == 0) sh_r = rr;
  }
  __syncthreads();
  const TopkRow r = sh_r;
  if (r.mode == TK_ALL) {
    for (int i = tid; i < n; i += TOPK_THREADS) out[i] = i;
    return;
  }
  if (r.mode == TK_WHOLE_ROW) {
    select_row<false, 0>(Keys<false>{nullptr, row, n, 0u}, n, m, out, RowPos{}, hist, whist, wcnt, 0u);
    return;
  }

  // chunk offsets: exclusive prefix sums of the per-chunk counts (wave 0,
  // lane L owns chunks 8 L .. 8 L + 7)
  const int nch = cdiv(n, TOPK_CHUNK);
  if (wave == 0) {
    const uint32_t* cc = p.chunk_cnt + (int64_t)tok * p.nch_stride * 2;
    uint32_t g[8], e[8], tg = 0, te = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * lane + j;
      g[j] = c < nch ? cc[2 * c] : 0u;
      e[j] = c < nch ? cc[2 * c + 1] : 0u;
      tg += g[j];
      te += e[j];
    }
    uint32_t og = wave_incl_scan(tg, lane) - tg, oe = wave_incl_scan(te, lane) - te;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * lane + j;
      if (c < nch) {
        choff[0][c] = og; choff[1][c] = oe;
        chcnt[0][c] = g[j]; chcnt[1][c] = e[j];
      }
      og += g[j];
      oe += e[j];
    }
  }
  __syncthreads();
  // positions above d1 to the output; d1 keys to LDS, both in chunk order
  for (int c = wave; c < nch; c += TOPK_WAVES) {
    const uint32_t* seg = (const uint32_t*)(row + (int64_t)c * TOPK_CHUNK);
    const uint32_t ng = chcnt[0][c], ne = chcnt[1][c], og = choff[0][c], oe = choff[1][c];
    for (uint32_t j = lane; j < ng; j += WAVE) out[og + j] = (int32_t)seg[j];
    for (uint32_t j = lane; j < ne; j += WAVE) {
      cand_w[oe + j] = seg[ng + j];
      cand_c[oe + j] = (uint8_t)c;
    }
  }
  __syncthreads();
  select_row<true, SCORE_HIST_BITS>(Keys<true>{cand_w, nullptr, (int)r.cnt1, r.d1 << (32 - SCORE_HIST_BITS)},
                                    (int)r.cnt1, m - (int)r.above1, out + r.above1, CandPos{cand_w, cand_c},
                                    hist, whist, wcnt, r.d1);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  const int T = p.sv.num_tokens;
  const TimerEvents t = timer_take(1);  // start of the compaction, end of the select
  hipError_t e = launch_kernel(topk_emit_kernel, dim3(T, p.nch_stride), dim3(TKE_THREADS), stream, t.start, nullptr, p);
  if (e != hipSuccess) return e;
  return launch_kernel(topk_select_kernel, dim3(T), dim3(TOPK_THREADS), stream, nullptr, t.stop, p);
}

}  // namespace idxs
