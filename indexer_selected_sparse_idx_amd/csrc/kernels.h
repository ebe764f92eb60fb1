// Internal interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxs {

// Device-side view of a batch (see idx_seqs in include/idxsparse.h).
struct SeqView {
  int num_seqs;
  int num_tokens;
  const int32_t* cu_q;         // nullable: one token per sequence
  const int32_t* ctx_len;
  const int32_t* block_table;  // nullable: contiguous cache
  int bt_stride;
  int page_shift;              // log2(page_size)
  int64_t seq_stride;
  int max_q_len;
  int max_ctx_len;
};

__device__ __forceinline__ int64_t cache_row(const SeqView& v, int b, int s) {
  if (v.block_table == nullptr) return (int64_t)b * v.seq_stride + s;
  const int page = v.block_table[(int64_t)b * v.bt_stride + (s >> v.page_shift)];
  return ((int64_t)page << v.page_shift) + (s & ((1 << v.page_shift) - 1));
}

__device__ __forceinline__ int first_token(const SeqView& v, int b) { return v.cu_q ? v.cu_q[b] : b; }
__device__ __forceinline__ int q_len(const SeqView& v, int b) { return v.cu_q ? v.cu_q[b + 1] - v.cu_q[b] : 1; }

// Sequence holding token `tok` (binary search over cu_q).
__device__ __forceinline__ int seq_of_token(const SeqView& v, int tok) {
  if (v.cu_q == nullptr) return tok;
  int lo = 0, hi = v.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (v.cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct ScoreParams {
  SeqView sv;
  const uint16_t* q_idx;   // bf16 [T, H_I, d_I]
  const uint8_t* k_idx;    // rows of d_I bf16 (2 bytes) or e4m3 (1 byte)
  const float* k_scale;    // nullable, per row
  const uint8_t* k_exp;    // MXFP8 keys: 4 E8M0 block exponents per row
  const float* head_w;     // [T, H_I]
  int H_I;
  int d_I;
  float* scores;           // [T, score_stride]
  int64_t score_stride;
  uint32_t* hist;          // [T, SCORE_HIST_BINS] histogram of the top key bits (zeroed by the launcher)
  int top_k;
  int32_t* out_idx;        // [T, top_k]: written by the prefill kernel, which also selects
  // prefill kernel: a fixed set of workgroups takes the token blocks (8
  // query tokens of one sequence) from the counter *pf_counter (zeroed before
  // the launch) until pf_items = num_seqs * max blocks are taken; wave w of
  // workgroup j keeps its candidate list in score row 8 j + w, so the
  // workspace holds 8 rows per workgroup, not one per token
  uint32_t* pf_counter;
  int pf_items;
};

// Workgroups of the prefill indexer: one per token block, at most
// PREFILL_ROW_BUDGET / 8 (the candidate rows of the workspace).
constexpr int PREFILL_ROW_BUDGET = 2048;
constexpr int PREFILL_TOKS = 8;  // query tokens (= waves, = candidate rows) per prefill workgroup
int prefill_workgroups(int num_seqs, int max_q_len);

struct TopkParams {
  SeqView sv;
  float* scores;           // [T, score_stride]; the selection reuses each row's storage
  int64_t score_stride;
  const uint32_t* hist;    // [T, SCORE_HIST_BINS] from the score kernel
  uint32_t* chunk_cnt;     // [T, nch_stride, 2]
  int nch_stride;          // ceil(max_ctx_len / TOPK_CHUNK)
  int top_k;
  int32_t* out_idx;        // [T, top_k]
};

// Keys per workgroup of the selection's compaction pass.
constexpr int TOPK_CHUNK = 2048;

// The score kernel histograms the top SCORE_HIST_BITS bits of every score's
// order-preserving key per row; the selection kernel starts from it.
constexpr int SCORE_HIST_BITS = 11;
constexpr int SCORE_HIST_BINS = 1 << SCORE_HIST_BITS;

struct AttnParams {
  SeqView sv;
  const uint16_t* q;       // bf16 [T, H, 576]
  int H;
  const uint8_t* kv;       // bf16 rows (1152 B) or packed fp8 rows (656 B)
  const int32_t* idx;      // [T, top_k]
  int top_k;
  float scale_log2;        // softmax_scale * log2(e)
  float* out;              // [T, H, 512]
  float* lse;              // [T, H] nullable
  int num_splits;
  int split_len;           // index entries per split (multiple of the tile)
  uint16_t* part_o;        // fp16 [T, num_splits, H, 512] when num_splits > 1: split O / its scale
  float* part_ls;          // [T, num_splits, H, 2]: (lse of the split, power-of-two scale of its stored O)
};

struct KvWriteParams {
  const uint16_t* src;     // bf16 [n, 576] latent rows
  int n;
  const int32_t* dst_row;  // [n] destination cache row (< 0: skipped)
  uint8_t* kv;             // packed FP8 latent rows of 656 bytes
};

struct KeyWriteParams {
  const uint16_t* src;     // bf16 [n, d] index keys
  int n;
  int d;                   // 64 or 128
  const int32_t* dst_row;  // [n] destination cache row (< 0: skipped)
  uint8_t* k;              // e4m3 key rows of d bytes
  float* scale;            // per-row fp32 scale, or null (keys stored with scale 1.0)
};

// Kernel launchers (asynchronous, on `stream`).  Each records the armed
// timing events of its kernel, if any.
// k_format: 0 bf16 keys, 1 e4m3 keys, 2 MXFP8 key rows (decode only)
hipError_t launch_score(const ScoreParams& p, int k_format, hipStream_t stream);
// true when launch_score also runs the Top-K selection (out_idx is then final)
bool score_selects(const SeqView& sv);
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);
hipError_t launch_attn(const AttnParams& p, bool kv_fp8, hipStream_t stream);
hipError_t launch_kv_fp8_write(const KvWriteParams& p, hipStream_t stream);
hipError_t launch_key_fp8_write(const KeyWriteParams& p, hipStream_t stream);

struct KeyMxWriteParams {
  const uint16_t* src;     // bf16 [n, 128] index keys
  int n;
  const int32_t* dst_row;  // [n] destination cache row (< 0: skipped)
  uint8_t* k;              // E4M3FN codes, rows of 128 bytes
  uint8_t* k_exp;          // E8M0 block exponents, rows of 4 bytes
};

hipError_t launch_key_mxfp8_write(const KeyMxWriteParams& p, hipStream_t stream);

// Timing hook (api.cpp): the events armed for the next launch of `kernel`
// (null when none), disarmed by the call.
struct TimerEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
TimerEvents timer_take(int kernel);

// A kernel launch that, given events, has the dispatch itself record them
// (hipExtLaunchKernelGGL: the start and end timestamps of the kernel, with
// no separate event packets between kernels on the stream).
template <typename K, typename... A>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                         A... args) {
  if (start || stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

// Attention split heuristic shared by the workspace query and the launcher.
int attn_num_splits(int num_tokens, int H, int top_k);
constexpr int ATTN_TILE = 32;

}  // namespace idxs
