// C ABI of libidxsparse.so (declared in include/idxsparse.h): host-side
// argument checks, workspace layout and kernel dispatch.  Nothing here
// touches device memory contents or synchronises the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "idxsparse.h"
#include "kernels.h"

// Scratch memory of idx_sparse_attn_decode_static, the entry point that
// allocates nothing: a file-scope device array of IDX_STATIC_SCRATCH_BYTES
// that every GPU the library runs on holds until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address on each GPU comes from hipGetSymbolAddress (static_scratch below),
// and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[IDX_STATIC_SCRATCH_BYTES];

namespace idxs {

namespace {

// Measurement hook state.  g_armed has bit k set while kernel k holds an
// armed event pair in g_timers[k]; an unarmed launch only loads g_armed (an
// atomic), so calls that nobody measures share no mutable state and may run
// from several host threads at once.  Arming and the launch it measures are
// a single-threaded measurement aid.
struct Timer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
Timer g_timers[IDX_KERNEL_COUNT];
std::atomic<uint32_t> g_armed{0};

constexpr size_t WS_ALIGN = 256;
size_t align_up(size_t v) { return (v + WS_ALIGN - 1) & ~(WS_ALIGN - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int v) { int s = 0; while ((1 << s) < v) ++s; return s; }


int check_seqs(const idx_seqs* s) {
  if (!s) return IDX_ERR_INVALID_ARG;
  if (s->num_seqs < 1 || s->num_seqs > 65535) return IDX_ERR_INVALID_ARG;
  if (s->num_tokens < 0) return IDX_ERR_INVALID_ARG;
  if (!s->ctx_len || !aligned4(s->ctx_len)) return IDX_ERR_INVALID_ARG;
  if (s->max_q_len < 1 || s->max_ctx_len < 1 || s->max_q_len > s->max_ctx_len) return IDX_ERR_INVALID_ARG;
  if (s->cu_q == nullptr) {
    if (s->num_tokens != s->num_seqs || s->max_q_len != 1) return IDX_ERR_INVALID_ARG;
  } else if (!aligned4(s->cu_q)) {
    return IDX_ERR_INVALID_ARG;
  }
  if (s->block_table) {
    if (!aligned4(s->block_table) || s->bt_stride < 1) return IDX_ERR_INVALID_ARG;
    if (!pow2(s->page_size) || s->page_size > 65536) return IDX_ERR_INVALID_ARG;
    if ((int64_t)s->bt_stride * s->page_size < s->max_ctx_len) return IDX_ERR_INVALID_ARG;
  } else if (s->seq_stride < s->max_ctx_len) {
    return IDX_ERR_INVALID_ARG;
  }
  return IDX_OK;
}

SeqView make_view(const idx_seqs* s) {
  SeqView v;
  v.num_seqs = s->num_seqs;
  v.num_tokens = s->num_tokens;
  v.cu_q = s->cu_q;
  v.ctx_len = s->ctx_len;
  v.block_table = s->block_table;
  v.bt_stride = s->bt_stride;
  v.page_shift = s->block_table ? log2i(s->page_size) : 0;
  v.seq_stride = s->seq_stride;
  v.max_q_len = s->max_q_len;
  v.max_ctx_len = s->max_ctx_len;
  return v;
}

int check_indexer(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx, int k_dtype,
                  const void* k_scale, const float* head_w, int H_I, int d_I, int top_k) {
  int rc = check_seqs(seqs);
  if (rc) return rc;
  if (!q_idx || !k_idx || !head_w) return IDX_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned4(head_w)) return IDX_ERR_INVALID_ARG;
  if (!aligned16(k_idx)) return IDX_ERR_INVALID_ARG;
  if (k_scale && !aligned4(k_scale)) return IDX_ERR_INVALID_ARG;
  if (H_I < 1 || top_k < 1) return IDX_ERR_INVALID_ARG;
  if (q_dtype != IDX_BF16) return IDX_ERR_UNSUPPORTED;
  if (k_dtype != IDX_BF16 && k_dtype != IDX_E4M3 && k_dtype != IDX_MXFP8) return IDX_ERR_UNSUPPORTED;
  if (H_I > 64 || (d_I != 64 && d_I != 128) || top_k > 2048) return IDX_ERR_UNSUPPORTED;
  if (k_dtype == IDX_MXFP8) {
    // the block exponents are required
    if (!k_scale) return IDX_ERR_INVALID_ARG;
    if (d_I != 128) return IDX_ERR_UNSUPPORTED;
  }
  return IDX_OK;
}

int check_attn(const idx_seqs* seqs, const void* q, int H, const void* kv, int kv_dtype, int top_k,
               float softmax_scale, const float* out, const float* lse) {
  int rc = check_seqs(seqs);
  if (rc) return rc;
  if (!q || !kv || !out) return IDX_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return IDX_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return IDX_ERR_INVALID_ARG;
  if (H < 1 || top_k < 1) return IDX_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 3.0e38f) return IDX_ERR_INVALID_ARG;
  if (kv_dtype != IDX_BF16 && kv_dtype != IDX_KV_FP8_656) return IDX_ERR_UNSUPPORTED;
  if (H > 128 || top_k > 2048) return IDX_ERR_UNSUPPORTED;
  return IDX_OK;
}

// Pitch of a score-workspace row in 4-byte words: one fp32 score per
// position (positions padded to a multiple of 64) for the decode-style
// kernels; for the prefill kernel two words (a (key, position) candidate
// pair) per position plus one spare pair (its 16-byte list loads read pairs
// two at a time), padded the same way.
int64_t score_stride(const idx_seqs* s) {
  if (score_selects(make_view(s))) return 2 * (((int64_t)s->max_ctx_len + 1 + 63) / 64 * 64);
  return ((int64_t)s->max_ctx_len + 63) / 64 * 64;
}

// score workspace: score rows (one per token; for the prefill kernel one
// per wave of its workgroups, see prefill_workgroups), then the per-row key
// histograms (prefill: its work counter)
size_t score_rows_bytes(const idx_seqs* s) {
  const size_t rows = score_selects(make_view(s)) ? (size_t)prefill_workgroups(s->num_seqs, s->max_q_len) * PREFILL_TOKS
                                                  : (size_t)std::max(s->num_tokens, 0);
  return align_up(rows * (size_t)score_stride(s) * sizeof(float));
}
// (the prefill kernel keeps its histograms in LDS and selects itself: no
// global histograms or selection counts)
size_t score_hist_bytes(const idx_seqs* s) {
  if (score_selects(make_view(s))) return 0;
  return align_up((size_t)std::max(s->num_tokens, 0) * SCORE_HIST_BINS * sizeof(uint32_t));
}
int topk_nch(const idx_seqs* s) { return std::max(1, (s->max_ctx_len + TOPK_CHUNK - 1) / TOPK_CHUNK); }
size_t score_ws_bytes(const idx_seqs* s) {
  if (score_selects(make_view(s))) return score_rows_bytes(s) + align_up(16);
  return score_rows_bytes(s) + score_hist_bytes(s) +
         align_up((size_t)std::max(s->num_tokens, 0) * topk_nch(s) * 2 * sizeof(uint32_t));
}

size_t attn_ws_bytes(const idx_seqs* s, int H, int top_k) {
  const int S = attn_num_splits(s->num_tokens, H, top_k);
  if (S <= 1) return 0;
  const size_t parts = (size_t)std::max(s->num_tokens, 0) * S * H;
  return align_up(parts * 512 * sizeof(uint16_t)) + align_up(parts * 2 * sizeof(float));
}

size_t idx_buf_bytes(const idx_seqs* s, int top_k) {
  return align_up((size_t)std::max(s->num_tokens, 0) * top_k * sizeof(int32_t));
}

int run_indexer(const idx_seqs* seqs, const void* q_idx, const void* k_idx, int k_dtype, const void* k_scale,
                const float* head_w, int H_I, int d_I, int top_k, int32_t* out_idx, void* ws,
                hipStream_t stream) {
  ScoreParams sp;
  sp.sv = make_view(seqs);
  sp.q_idx = static_cast<const uint16_t*>(q_idx);
  sp.k_idx = static_cast<const uint8_t*>(k_idx);
  sp.k_scale = k_dtype == IDX_MXFP8 ? nullptr : static_cast<const float*>(k_scale);
  sp.k_exp = k_dtype == IDX_MXFP8 ? static_cast<const uint8_t*>(k_scale) : nullptr;
  sp.head_w = head_w;
  sp.H_I = H_I;
  sp.d_I = d_I;
  sp.scores = static_cast<float*>(ws);
  sp.score_stride = score_stride(seqs);
  uint8_t* const base = static_cast<uint8_t*>(ws);
  const size_t hist_off = score_rows_bytes(seqs);
  const size_t cnt_off = hist_off + score_hist_bytes(seqs);
  sp.hist = reinterpret_cast<uint32_t*>(base + hist_off);
  sp.top_k = top_k;
  sp.out_idx = out_idx;
  sp.pf_counter = reinterpret_cast<uint32_t*>(base + score_rows_bytes(seqs));  // (prefill kernel only)
  sp.pf_items = seqs->num_seqs * ((seqs->max_q_len + PREFILL_TOKS - 1) / PREFILL_TOKS);
  const int k_format = k_dtype == IDX_E4M3 ? 1 : k_dtype == IDX_MXFP8 ? 2 : 0;
  if (launch_score(sp, k_format, stream) != hipSuccess) return IDX_ERR_HIP;
  if (score_selects(sp.sv)) {
    // the score kernel has selected: an armed Top-K timer measures nothing
    const TimerEvents t = timer_take(IDX_KERNEL_TOPK);
    if (t.start) (void)hipEventRecord(t.start, stream);
    if (t.stop) (void)hipEventRecord(t.stop, stream);
    return IDX_OK;
  }
  TopkParams tp;
  tp.sv = sp.sv;
  tp.scores = sp.scores;
  tp.score_stride = sp.score_stride;
  tp.hist = sp.hist;
  tp.chunk_cnt = reinterpret_cast<uint32_t*>(base + cnt_off);
  tp.nch_stride = topk_nch(seqs);
  tp.top_k = top_k;
  tp.out_idx = out_idx;
  if (launch_topk(tp, stream) != hipSuccess) return IDX_ERR_HIP;
  return IDX_OK;
}

int run_attn(const idx_seqs* seqs, const void* q, int H, const void* kv, int kv_dtype, const int32_t* idx,
             int top_k, float softmax_scale, float* out, float* lse, void* ws, hipStream_t stream) {
  AttnParams ap;
  ap.sv = make_view(seqs);
  ap.q = static_cast<const uint16_t*>(q);
  ap.H = H;
  ap.kv = static_cast<const uint8_t*>(kv);
  ap.idx = idx;
  ap.top_k = top_k;
  ap.scale_log2 = softmax_scale * 1.4426950408889634f;
  ap.out = out;
  ap.lse = lse;
  ap.num_splits = attn_num_splits(seqs->num_tokens, H, top_k);
  ap.split_len = (top_k + ap.num_splits - 1) / ap.num_splits;
  ap.split_len = (ap.split_len + ATTN_TILE - 1) / ATTN_TILE * ATTN_TILE;
  ap.part_o = nullptr;
  ap.part_ls = nullptr;
  if (ap.num_splits > 1) {
    const size_t parts = (size_t)seqs->num_tokens * ap.num_splits * H;
    ap.part_o = static_cast<uint16_t*>(ws);
    ap.part_ls = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up(parts * 512 * sizeof(uint16_t)));
  }
  if (launch_attn(ap, kv_dtype == IDX_KV_FP8_656, stream) != hipSuccess) return IDX_ERR_HIP;
  return IDX_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept; null when
// the lookup fails.
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;

void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next call
    return nullptr;
  }
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

TimerEvents timer_take(int kernel) {
  TimerEvents e;
  const uint32_t bit = 1u << kernel;
  if ((g_armed.load(std::memory_order_acquire) & bit) == 0) return e;  // the common case: nothing armed
  e.start = g_timers[kernel].start;
  e.stop = g_timers[kernel].stop;
  g_timers[kernel] = Timer{};
  g_armed.fetch_and(~bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace idxs

using namespace idxs;

extern "C" {

const char* idx_status_string(int status) {
  switch (status) {
    case IDX_OK: return "IDX_OK";
    case IDX_ERR_INVALID_ARG: return "IDX_ERR_INVALID_ARG: null or misaligned pointer, or a size/bound out of range";
    case IDX_ERR_UNSUPPORTED: return "IDX_ERR_UNSUPPORTED: dtype or dimension outside the supported set";
    case IDX_ERR_WORKSPACE: return "IDX_ERR_WORKSPACE: workspace missing or smaller than required";
    case IDX_ERR_HIP: return "IDX_ERR_HIP: a HIP kernel launch failed";
    case IDX_ERR_TOO_LARGE:
      return "IDX_ERR_TOO_LARGE: the call needs more scratch than the library's static buffer holds "
             "(IDX_STATIC_SCRATCH_BYTES); use the entry point that takes a workspace";
    default: return "unknown idx_status";
  }
}

size_t idx_score_topk_workspace(const idx_seqs* seqs, int H_I, int d_I, int top_k) {
  (void)H_I; (void)d_I; (void)top_k;
  if (check_seqs(seqs)) return 0;
  return score_ws_bytes(seqs);
}

size_t sparse_mla_attn_workspace(const idx_seqs* seqs, int H, int top_k) {
  if (check_seqs(seqs) || H < 1 || top_k < 1) return 0;
  return attn_ws_bytes(seqs, H, top_k);
}

size_t idx_sparse_attn_workspace(const idx_seqs* seqs, int H_I, int d_I, int H, int top_k) {
  if (check_seqs(seqs) || H < 1 || top_k < 1) return 0;
  (void)H_I; (void)d_I;
  return std::max(score_ws_bytes(seqs), attn_ws_bytes(seqs, H, top_k)) + idx_buf_bytes(seqs, top_k);
}

int idx_score_topk(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx, int k_dtype,
                   const void* k_scale, const float* head_w, int H_I, int d_I, int top_k, int32_t* out_idx,
                   void* ws, size_t ws_bytes, void* stream) {
  int rc = check_indexer(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k);
  if (rc) return rc;
  if (!out_idx || !aligned4(out_idx)) return IDX_ERR_INVALID_ARG;
  if (seqs->num_tokens == 0) return IDX_OK;
  if (!ws || !aligned16(ws) || ws_bytes < score_ws_bytes(seqs)) return IDX_ERR_WORKSPACE;
  return run_indexer(seqs, q_idx, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k, out_idx, ws,
                     static_cast<hipStream_t>(stream));
}

int sparse_mla_attn(const idx_seqs* seqs, const void* q, int H, const void* kv, int kv_dtype, const int32_t* idx,
                    int top_k, float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_attn(seqs, q, H, kv, kv_dtype, top_k, softmax_scale, out, lse);
  if (rc) return rc;
  if (!idx || !aligned4(idx)) return IDX_ERR_INVALID_ARG;
  if (seqs->num_tokens == 0) return IDX_OK;
  const size_t need = attn_ws_bytes(seqs, H, top_k);
  if (need && (!ws || !aligned16(ws) || ws_bytes < need)) return IDX_ERR_WORKSPACE;
  return run_attn(seqs, q, H, kv, kv_dtype, idx, top_k, softmax_scale, out, lse, ws,
                  static_cast<hipStream_t>(stream));
}

static int fused(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx, int k_dtype,
                 const void* k_scale, const float* head_w, int H_I, int d_I, int top_k, const void* q, int H,
                 const void* kv, int kv_dtype, float softmax_scale, float* out, float* lse, int32_t* out_idx,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_indexer(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k);
  if (rc) return rc;
  rc = check_attn(seqs, q, H, kv, kv_dtype, top_k, softmax_scale, out, lse);
  if (rc) return rc;
  if (out_idx && !aligned4(out_idx)) return IDX_ERR_INVALID_ARG;
  if (seqs->num_tokens == 0) return IDX_OK;
  const size_t need = idx_sparse_attn_workspace(seqs, H_I, d_I, H, top_k);
  if (!ws || !aligned16(ws) || ws_bytes < need) return IDX_ERR_WORKSPACE;
  // workspace: [scratch shared by the score rows and the attention partials][indices]
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t scratch = std::max(score_ws_bytes(seqs), attn_ws_bytes(seqs, H, top_k));
  int32_t* idx = out_idx ? out_idx : reinterpret_cast<int32_t*>(base + scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_indexer(seqs, q_idx, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k, idx, base, st);
  if (rc) return rc;
  return run_attn(seqs, q, H, kv, kv_dtype, idx, top_k, softmax_scale, out, lse, base, st);
}

int idx_sparse_attn_prefill(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx, int k_dtype,
                            const void* k_scale, const float* head_w, int H_I, int d_I, int top_k, const void* q,
                            int H, const void* kv, int kv_dtype, float softmax_scale, float* out, float* lse,
                            int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  return fused(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k, q, H, kv, kv_dtype,
               softmax_scale, out, lse, out_idx, ws, ws_bytes, stream);
}

int idx_sparse_attn_decode(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx, int k_dtype,
                           const void* k_scale, const float* head_w, int H_I, int d_I, int top_k, const void* q,
                           int H, const void* kv, int kv_dtype, float softmax_scale, float* out, float* lse,
                           int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  if (seqs && seqs->cu_q != nullptr) return IDX_ERR_INVALID_ARG;
  return fused(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k, q, H, kv, kv_dtype,
               softmax_scale, out, lse, out_idx, ws, ws_bytes, stream);
}

int idx_sparse_attn_decode_static(const idx_seqs* seqs, const void* q_idx, int q_dtype, const void* k_idx,
                                  int k_dtype, const void* k_scale, const float* head_w, int H_I, int d_I, int top_k,
                                  const void* q, int H, const void* kv, int kv_dtype, float softmax_scale, float* out,
                                  float* lse, int32_t* out_idx, void* stream) {
  if (seqs && seqs->cu_q != nullptr) return IDX_ERR_INVALID_ARG;
  int rc = check_indexer(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k);
  if (rc) return rc;
  rc = check_attn(seqs, q, H, kv, kv_dtype, top_k, softmax_scale, out, lse);
  if (rc) return rc;
  if (seqs->num_tokens == 0) return IDX_OK;
  const size_t need = idx_sparse_attn_workspace(seqs, H_I, d_I, H, top_k);
  if (need > IDX_STATIC_SCRATCH_BYTES) return IDX_ERR_TOO_LARGE;
  void* ws = static_scratch();
  if (!ws) return IDX_ERR_HIP;
  return fused(seqs, q_idx, q_dtype, k_idx, k_dtype, k_scale, head_w, H_I, d_I, top_k, q, H, kv, kv_dtype,
               softmax_scale, out, lse, out_idx, ws, IDX_STATIC_SCRATCH_BYTES, stream);
}

int idx_kv_fp8_write(const void* src, int n, const int32_t* dst_row, void* kv, void* stream) {
  if (n < 0) return IDX_ERR_INVALID_ARG;
  if (n == 0) return IDX_OK;
  if (!src || !dst_row || !kv) return IDX_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(kv) || !aligned4(dst_row)) return IDX_ERR_INVALID_ARG;
  KvWriteParams p;
  p.src = static_cast<const uint16_t*>(src);
  p.n = n;
  p.dst_row = dst_row;
  p.kv = static_cast<uint8_t*>(kv);
  return launch_kv_fp8_write(p, static_cast<hipStream_t>(stream)) == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}

int idx_key_fp8_write(const void* src, int n, int d_I, const int32_t* dst_row, void* k_cache, float* k_scale,
                      void* stream) {
  if (n < 0 || (d_I != 64 && d_I != 128)) return IDX_ERR_INVALID_ARG;
  if (n == 0) return IDX_OK;
  if (!src || !dst_row || !k_cache) return IDX_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(k_cache) || !aligned4(dst_row)) return IDX_ERR_INVALID_ARG;
  if (k_scale && !aligned4(k_scale)) return IDX_ERR_INVALID_ARG;
  KeyWriteParams p;
  p.src = static_cast<const uint16_t*>(src);
  p.n = n;
  p.d = d_I;
  p.dst_row = dst_row;
  p.k = static_cast<uint8_t*>(k_cache);
  p.scale = k_scale;
  return launch_key_fp8_write(p, static_cast<hipStream_t>(stream)) == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}

int idx_key_mxfp8_write(const void* src, int n, const int32_t* dst_row, void* k_cache, void* k_exp, void* stream) {
  if (n < 0) return IDX_ERR_INVALID_ARG;
  if (n == 0) return IDX_OK;
  if (!src || !dst_row || !k_cache || !k_exp) return IDX_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(k_cache) || !aligned4(dst_row) || !aligned4(k_exp)) return IDX_ERR_INVALID_ARG;
  KeyMxWriteParams p;
  p.src = static_cast<const uint16_t*>(src);
  p.n = n;
  p.dst_row = dst_row;
  p.k = static_cast<uint8_t*>(k_cache);
  p.k_exp = static_cast<uint8_t*>(k_exp);
  return launch_key_mxfp8_write(p, static_cast<hipStream_t>(stream)) == hipSuccess ? IDX_OK : IDX_ERR_HIP;
}

int idx_timer_arm(int kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= IDX_KERNEL_COUNT || !start_event || !stop_event) return IDX_ERR_INVALID_ARG;
  g_timers[kernel].start = static_cast<hipEvent_t>(start_event);
  g_timers[kernel].stop = static_cast<hipEvent_t>(stop_event);
  g_armed.fetch_or(1u << kernel, std::memory_order_release);
  return IDX_OK;
}

}  // extern "C"
