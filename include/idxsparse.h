/*
 * idxsparse.h -- C ABI of libidxsparse.so: index-selected sparse latent
 * attention on AMD Instinct MI355X (gfx950).
 *
 * The operation is the index-based sparse attention branch described in
 * "Day 0 Inference Support for New LLM Architectures: Optimization Practices"
 * (section "Index-Based Sparse Attention": a lightweight indexer scores the
 * history, weights the heads and selects the Top-K positions; a sparse core
 * reads the KV entries at those positions and attends over them) and in
 * "Day 0 Inference Adaptation and Performance Optimization for New Models"
 * (section 3: an indexing stage, then a sparse attention stage that reads
 * the main KV at the selected indices; section 1: the selection sits on top
 * of Multi-head Latent Attention, one latent cache shared by all heads).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers inside `idx_seqs` and every tensor argument are DEVICE
 *   pointers; `idx_seqs` itself is a host struct.  The caller owns all
 *   memory.  The library never allocates, never synchronises the device and
 *   keeps no state between calls (the measurement hook at the end excepted).
 * - Thread safety: every entry point is re-entrant and may be called from
 *   several host threads at once (on the same or different streams; calls
 *   that share output or workspace memory race on it, like any two kernels).
 *   A call that no armed timer measures reads one atomic word of the
 *   library and writes none.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   A call returns after enqueueing; results are ready when the stream is.
 * - Return value: IDX_OK, or a negative idx_status from host-side argument
 *   checks made BEFORE anything is enqueued (nothing is launched then), or
 *   IDX_ERR_HIP if a launch failed.  idx_status_string() names a status.
 * - Device-side contents are not validated: ctx_len[b] >= q_len(b) >= 1,
 *   valid page ids in the block table and in-range cache rows are
 *   preconditions; violating them is undefined behaviour.
 * - Tensor pointers must be 16-byte aligned.
 *
 * Batches
 * -------
 * A call covers B sequences.  Sequence b holds ctx_len[b] cached positions
 * (its new tokens included).  Its q_len(b) query tokens are the LAST q_len(b)
 * positions: query i of sequence b sits at position
 *     t = ctx_len[b] - q_len(b) + i,
 * and the causal history of that query is every position s <= t.  Tokens are
 * numbered 0..T-1 across the batch in sequence order (cu_q offsets).
 *
 * Cache rows.  Contiguous cache: position s of sequence b is row
 *     b * seq_stride + s.
 * Paged cache (block_table != NULL): it is row
 *     block_table[b * bt_stride + s / page_size] * page_size + s % page_size.
 * The index-key cache and the latent cache use the same row numbering and
 * the same block table.
 */
#ifndef IDXSPARSE_H
#define IDXSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IDX_OK = 0,
  IDX_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or bound  */
  IDX_ERR_UNSUPPORTED = -2,   /* well-formed but outside the supported set    */
  IDX_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than required      */
  IDX_ERR_HIP = -4,           /* a HIP launch reported an error               */
  IDX_ERR_TOO_LARGE = -5      /* idx_sparse_attn_decode_static: the call needs
                                 more scratch than IDX_STATIC_SCRATCH_BYTES   */
} idx_status;

typedef enum {
  IDX_BF16 = 1,        /* bfloat16                                               */
  IDX_E4M3 = 2,        /* OCP FP8 E4M3FN codes, one byte per value               */
  IDX_KV_FP8_656 = 3,  /* packed FP8 latent row of 656 bytes: 512 e4m3 latent
                          codes, 4 little-endian fp32 scales (one per
                          128-value tile; value j = code[j] * scale[j / 128]),
                          64 bf16 rope values.  The per-token tile of 128 with
                          its own scale follows "Hierarchical Quantization"
                          (Day 0 Inference Support..., KV cache bullet) and
                          section 4 of Day 0 Inference Adaptation and
                          Performance Optimization for New Models.           */
  IDX_MXFP8 = 4        /* MXFP8 index keys (d_I = 128): rows of 128 E4M3FN
                          codes in k_idx, and in k_scale 4 E8M0 bytes per row,
                          one per block of 32 codes (value j = code[j] *
                          2^(byte[j / 32] - 127)).  The index quantised in
                          blocks of 32 ("Hierarchical Quantization",
                          index-cache bullet, Day 0 Inference Support...).
                          Any batch (in prefill calls each query token streams
                          its own causal key range); the query is quantised on
                          the fly per head and block of 32 (shared exponent
                          floor(log2 amax) - 8, codes E4M3(clamp(q / 2^e,
                          +-448))).                                            */
} idx_dtype;

typedef struct idx_seqs {
  int32_t num_seqs;            /* B >= 1                                           */
  int32_t num_tokens;          /* T = total query tokens (== B when cu_q is NULL)  */
  const int32_t *cu_q;         /* device int32 [B + 1] token offsets, cu_q[0] = 0;
                                  NULL => one query token per sequence (decode)    */
  const int32_t *ctx_len;      /* device int32 [B]                                 */
  int32_t max_q_len;           /* host upper bound of q_len(b) (1 for decode)      */
  int32_t max_ctx_len;         /* host upper bound of ctx_len[b]                   */
  const int32_t *block_table;  /* device int32 [B, bt_stride] page ids, or NULL    */
  int32_t bt_stride;           /* entries per block-table row                      */
  int32_t page_size;           /* power of two, 1..65536 (paged caches only)       */
  int64_t seq_stride;          /* rows per sequence, contiguous caches only;
                                  must be >= max_ctx_len                           */
} idx_seqs;

/* ------------------------------------------------------------------------ *
 * Indexer: score every causal position, then select the Top-K.
 *
 * For each query token at position t of sequence b and each s <= t:
 *     S[s] = sum_h head_w[tok, h] * ReLU(k_scale[row(s)] * dot(q_idx[tok, h, :], k_idx[row(s), :]))
 * (relevance scoring, head-weight weighting, then Top-K: the fused indexer of
 * "Internal Fusion of the Indexer", Day 0 Inference Support...; section 3
 * of Day 0 Inference Acceleration for New LLM Architectures.  The per-head
 * ReLU, the absence of a 1/sqrt(d) factor and the tie rule are this
 * library's reading where the pages are silent.)
 * out_idx[tok, :] receives the min(top_k, t + 1) positions with the largest
 * S, ties going to the lower position, as logical positions s (not rows), in
 * no particular order, followed by -1 up to top_k.  Scores are accumulated in
 * fp32 from bf16 (or e4m3) products.
 *
 *   q_idx    [T, H_I, d_I], dtype q_dtype (IDX_BF16)
 *   k_idx    cache rows of d_I values, dtype k_dtype (IDX_BF16, IDX_E4M3, or
 *            IDX_MXFP8: E4M3 codes, d_I = 128); 16-byte aligned
 *   k_scale  bf16 / e4m3 keys: fp32 per cache row, or NULL for 1.0.  A
 *            quantisation scale, so it must be >= 0: ReLU(k * x) = k * ReLU(x)
 *            then holds, and prefill calls apply it to the head-weighted sum
 *            (one multiply per key).
 *            IDX_MXFP8: required, uint8 [rows, 4] E8M0 block exponents (row r
 *            at byte 4 r), 4-byte aligned
 *   head_w   fp32 [T, H_I]
 *   H_I      1..64 indexer heads;  d_I in {64, 128};  top_k 1..2048
 *   out_idx  int32 [T, top_k]
 *   ws       device workspace of >= idx_score_topk_workspace(...) bytes
 * ------------------------------------------------------------------------ */
size_t idx_score_topk_workspace(const idx_seqs *seqs, int H_I, int d_I, int top_k);
int idx_score_topk(const idx_seqs *seqs,
                   const void *q_idx, int q_dtype,
                   const void *k_idx, int k_dtype,
                   const void *k_scale,
                   const float *head_w,
                   int H_I, int d_I, int top_k,
                   int32_t *out_idx,
                   void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * Sparse latent attention over given indices.
 *
 * For each token and head h, over the entries s of idx[tok, :] with
 * 0 <= s < ctx_len[b] (other entries, e.g. -1 padding, are skipped):
 *     l_s = softmax_scale * dot(q[tok, h, :], c[row(s), 0:576])
 *     out[tok, h, :] = sum_s softmax(l)_s * c[row(s), 0:512]
 *     lse[tok, h] = log(sum_s exp(l_s))
 * where c is the latent row (576 = 512 latent + 64 rope, shared by all
 * heads).  A token with no valid entry gets out = 0, lse = -inf.  (Reading
 * the KV entries at the selected indices and attending in blocks: "Index-
 * Based Sparse Attention", Day 0 Inference Support...; section 3 of Day 0
 * Inference Acceleration...; MLA latent cache: section 1 of Day 0 Inference
 * Adaptation and Performance Optimization for New Models.)
 * Products are bf16 x bf16 with fp32 accumulation; FP8 rows are dequantised
 * to bf16 before use; the softmax is computed online in fp32.
 *
 *   q        [T, H, 576] bf16;  H in 1..128
 *   kv       cache rows, dtype kv_dtype (IDX_BF16: 576 bf16 = 1152 bytes;
 *            IDX_KV_FP8_656: 656-byte packed rows)
 *   idx      int32 [T, top_k] logical positions;  top_k 1..2048
 *   softmax_scale  finite and > 0 (a softmax temperature; 1/sqrt(576) in
 *            the pages' models), else IDX_ERR_INVALID_ARG
 *   out      fp32 [T, H, 512];  lse fp32 [T, H] or NULL
 * ------------------------------------------------------------------------ */
size_t sparse_mla_attn_workspace(const idx_seqs *seqs, int H, int top_k);
int sparse_mla_attn(const idx_seqs *seqs,
                    const void *q, int H,
                    const void *kv, int kv_dtype,
                    const int32_t *idx, int top_k,
                    float softmax_scale,
                    float *out, float *lse,
                    void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * Fused entry points: the indexer, then sparse attention on its indices, on
 * one stream with the selected indices as the only hand-over (the pages'
 * single synchronisation point where the Top-K results are ready: section 3
 * of Day 0 Inference Adaptation and Performance Optimization for New
 * Models).  Arguments are those of idx_score_topk followed by those of
 * sparse_mla_attn.  out_idx may be NULL: the indices then live in the
 * workspace only.  idx_sparse_attn_decode requires seqs->cu_q == NULL (one
 * token per sequence); idx_sparse_attn_prefill accepts any batch.
 * ------------------------------------------------------------------------ */
size_t idx_sparse_attn_workspace(const idx_seqs *seqs, int H_I, int d_I, int H, int top_k);
int idx_sparse_attn_prefill(const idx_seqs *seqs,
                            const void *q_idx, int q_dtype,
                            const void *k_idx, int k_dtype,
                            const void *k_scale, const float *head_w,
                            int H_I, int d_I, int top_k,
                            const void *q, int H,
                            const void *kv, int kv_dtype,
                            float softmax_scale,
                            float *out, float *lse, int32_t *out_idx,
                            void *ws, size_t ws_bytes, void *stream);
int idx_sparse_attn_decode(const idx_seqs *seqs,
                           const void *q_idx, int q_dtype,
                           const void *k_idx, int k_dtype,
                           const void *k_scale, const float *head_w,
                           int H_I, int d_I, int top_k,
                           const void *q, int H,
                           const void *kv, int kv_dtype,
                           float softmax_scale,
                           float *out, float *lse, int32_t *out_idx,
                           void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * Allocation-free fused decode, for callers that cannot allocate device
 * memory (work under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc).  Same arguments, checks and results as
 * idx_sparse_attn_decode, without the workspace: the call uses a static
 * device buffer of IDX_STATIC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (looked up once per device on the
 * first call there; the calling thread's current device must be the
 * stream's).  It allocates nothing and calls no allocating routine.
 * Returns IDX_ERR_TOO_LARGE, before anything is enqueued, when
 * idx_sparse_attn_workspace(seqs, H_I, d_I, H, top_k) exceeds that size (64
 * requests x 32768 positions with Top-K 2048 and 128 heads need about 34
 * MiB).  Every call on one GPU shares that GPU's buffer, which keeps the
 * last call's contents (nothing in it has to start at zero: the call clears
 * what it accumulates): two calls that can overlap on one GPU (different
 * streams, or host threads) race and give undefined results; calls in order
 * on one stream are safe.
 * ------------------------------------------------------------------------ */
#define IDX_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int idx_sparse_attn_decode_static(const idx_seqs *seqs,
                                  const void *q_idx, int q_dtype,
                                  const void *k_idx, int k_dtype,
                                  const void *k_scale, const float *head_w,
                                  int H_I, int d_I, int top_k,
                                  const void *q, int H,
                                  const void *kv, int kv_dtype,
                                  float softmax_scale,
                                  float *out, float *lse, int32_t *out_idx,
                                  void *stream);

/* ------------------------------------------------------------------------ *
 * FP8 latent-cache writer: quantise latent rows into the packed 656-byte
 * rows of an IDX_KV_FP8_656 cache (the producer side of that cache).
 *
 * Each latent row keeps per-token tiles of 128 values, each with its own
 * scale computed online from the row ("Hierarchical Quantization", KV cache
 * bullet, in Day 0 Inference Support...; section 4 of Day 0 Inference
 * Adaptation and Performance Optimization for New Models).  Tile j of a row
 * gets scale_j = amax_j / 448 (fp32; amax_j the largest |value| of the tile)
 * and codes E4M3FN(clamp(value / scale_j, -448, 448)) (fp32 division,
 * rounded to the nearest E4M3FN value, ties to even, the sign kept); an
 * all-zero tile gets scale 0 and codes 0.  The 64 rope values are copied.
 * (The scale rule and the rounding are this library's reading; the pages
 * give the tile size.)
 *
 *   src      bf16 [n, 576] latent rows (512 latent values, then 64 rope)
 *   n        rows, >= 0 (0: nothing is launched)
 *   dst_row  device int32 [n]: the cache row each source row is written
 *            to; entries < 0 are skipped.  Two entries naming the same row
 *            race (undefined which is kept).
 *   kv       the cache: rows of 656 bytes, 16-byte aligned; only the named
 *            rows are written.
 * ------------------------------------------------------------------------ */
int idx_kv_fp8_write(const void *src, int n, const int32_t *dst_row, void *kv, void *stream);

/* ------------------------------------------------------------------------ *
 * FP8 index-key writer: store bf16 index keys as E4M3FN codes in an
 * IDX_E4M3 key cache (rows of d_I bytes), with one fp32 scale per row or
 * with scale 1.0.  The indexer keys join the FP8 quantisation of "Hierarchical
 * Quantization" (Day 0 Inference Support..., index-cache bullet); the
 * per-row scale granularity is this library's reading (the pages quantise
 * the index in groups of 32, which is not built here).
 *
 *   src      bf16 [n, d_I] keys;  d_I in {64, 128};  n >= 0
 *   dst_row  device int32 [n]: destination cache row (entries < 0 skipped)
 *   k_cache  E4M3FN key rows of d_I bytes, 16-byte aligned
 *   k_scale  fp32 per cache row, or NULL.  Non-NULL: row scale = amax / 448
 *            (fp32), codes E4M3FN(clamp(k / scale, -448, 448)) (an all-zero
 *            row gets scale 0 and codes 0), and the scale is written to
 *            k_scale[dst_row[i]] -- the per-row key scale the indexer reads.
 *            NULL: codes E4M3FN(clamp(k, -448, 448)), scale 1.0.
 * Rounding: to the nearest E4M3FN value, ties to even, the sign kept.
 * ------------------------------------------------------------------------ */
int idx_key_fp8_write(const void *src, int n, int d_I, const int32_t *dst_row, void *k_cache, float *k_scale,
                      void *stream);

/* ------------------------------------------------------------------------ *
 * MXFP8 index-key writer: quantises n new bf16 keys of d_I = 128 into the
 * MXFP8 index cache that idx_score_topk reads with k_dtype IDX_MXFP8 --
 * blocks of 32 values sharing a power-of-two scale ("Hierarchical
 * Quantization", index-cache bullet, in Day 0 Inference Support for New LLM
 * Architectures; section 4 of Day 0 Inference Adaptation and Performance
 * Optimization for New Models).  Per block the OCP MX rule for E4M3
 * elements: e = floor(log2(amax)) - 8, clamped to [-127, 127]; E8M0 byte
 * e + 127; codes E4M3FN(clamp(k / 2^e, -448, 448)), rounded to the nearest
 * value, ties to even, the sign kept; an all-zero block gets byte 0 and
 * codes 0.
 *
 *   src      bf16 [n, 128] keys;  n >= 0 (n == 0: nothing is launched)
 *   dst_row  device int32 [n]: destination cache row (entries < 0 skipped)
 *   k_cache  E4M3FN codes, rows of 128 bytes, 16-byte aligned
 *   k_exp    E8M0 block exponents, rows of 4 bytes (block j of row r at
 *            k_exp[4 r + j]), 4-byte aligned
 * Rows not named by dst_row are left untouched.  Errors: IDX_ERR_INVALID_ARG
 * for n < 0, a NULL or misaligned pointer; IDX_ERR_HIP for a launch failure.
 * ------------------------------------------------------------------------ */
int idx_key_mxfp8_write(const void *src, int n, const int32_t *dst_row, void *k_cache, void *k_exp, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *idx_status_string(int status);

/* ------------------------------------------------------------------------ *
 * Measurement hook.  idx_timer_arm(kernel, start, stop) makes the NEXT
 * launch of `kernel` by any entry point record the hipEvent_t `start` at the
 * start of its (first) dispatch and `stop` at the end of its (last), on the
 * stream it is launched on, and then disarms.  The dispatches record the
 * events themselves (hipExtLaunchKernelGGL), so an armed launch runs back to
 * back with its neighbours like an unarmed one.  One arm per kernel at a
 * time.  Arming, and the launch it measures, are not thread-safe against
 * other arming or measured launches of the same kernel (a measurement aid,
 * not part of the compute path); unmeasured calls are unaffected.
 * Returns IDX_OK or IDX_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
typedef enum {
  IDX_KERNEL_SCORE = 0,     /* indexer score                                  */
  IDX_KERNEL_TOPK = 1,      /* Top-K selection of the decode indexer (the
                               prefill indexer selects inside its score
                               kernel)                                       */
  IDX_KERNEL_ATTN = 2,      /* sparse latent attention                        */
  IDX_KERNEL_COMBINE = 3,   /* split merge of the attention partials (only
                               launched when a call splits the index lists) */
  IDX_KERNEL_KV_WRITE = 4,  /* FP8 latent-cache writer                      */
  IDX_KERNEL_COUNT = 5
} idx_kernel;
int idx_timer_arm(int kernel, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* IDXSPARSE_H */
