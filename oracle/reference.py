"""CPU oracle for index-selected sparse latent attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
CPU-baseline leg may import this module.  It is plain, single-threaded
float64 NumPy written from the definitions, with no blocking, fusion or
reordering, so that it can be checked against the pages by eye.  It shares no
code with the HIP path.

What is computed, and where the pages define it:

* Lightweight indexer score -- "Day 0 Inference Support for New LLM
  Architectures" (page 1), section "Index-Based Sparse Attention" (the
  indexer scores history positions, weights the heads, selects Top-K) and
  "Internal Fusion of the Indexer" (the fused_indexer sketch: batched dot of
  the index query with the paged K cache, weighted sum over heads, Top-K);
  page 3 section 2 (relevance scoring, head weight summation, Top-K
  selection).  The pages leave the per-head non-linearity, the scaling and
  the key sharing open; the reading taken is
      S[t, s] = sum_h w[t, h] * ReLU(k_scale[s] * (q_I[t, h, :] . k_I[s, :]))
  over every causal position s <= t, with one key row per position shared by
  all indexer heads and no 1/sqrt(d) factor.
* Top-K -- the same passages: the min(K, t + 1) positions of largest score,
  ties going to the lower position (the pages are silent on ties; this is the
  reading taken).  Valid indices first, then -1 padding up to K.
* Sparse attention core -- page 1 "Index-Based Sparse Attention" (read the KV
  entries at the selected indices and attend over them), page 3 section 3,
  page 4 section 3; latent cache shared by all heads per page 1 (low-rank
  latent cache) and page 4 section 1 (MLA).  Each selected position s
  contributes its 576-wide latent row c[s] as key and its first 512 values as
  value:
      l_s = scale * (q[t, h, :] . c[s, :]),  O[t, h, :] = sum_s softmax(l)_s c[s, :512]
      lse[t, h] = log sum_s exp(l_s)
  An empty selection gives O = 0 and lse = -inf.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import formats

LATENT = formats.LATENT
ROW = formats.ROW


# --------------------------------------------------------------------------
# Single-row definitions
# --------------------------------------------------------------------------

def indexer_scores(q_heads, keys, w, k_scale=None):
    """Scores of one query over n candidate keys.

    q_heads: float64 [H_I, d_I]; keys: float64 [n, d_I]; w: float64 [H_I];
    k_scale: float64 [n] or None (all ones).  Returns float64 [n]:
    S[s] = sum_h w[h] * max(0, k_scale[s] * (q_heads[h] . keys[s])).
    Signed zero is canonicalised to +0 so that equal scores compare equal
    bit for bit.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dots = keys @ q_heads.T                       # [n, H_I]: q_h . k_s
    if k_scale is not None:
        dots = dots * np.asarray(k_scale, dtype=np.float64)[:, None]
    relu = np.maximum(dots, 0.0)
    scores = relu @ w                             # head-weighted sum
    return scores + 0.0


def topk_select(scores, top_k):
    """Top-K of one score row with lower-position tie breaking.

    m = min(top_k, n) entries are selected: every position whose score is
    strictly above the m-th largest score tau, then the lowest positions whose
    score equals tau until m are taken.  Returns int32 [top_k]: the selected
    positions in ascending order followed by -1 padding.
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    m = min(int(top_k), n)
    out = np.full(int(top_k), -1, dtype=np.int32)
    if m == 0:
        return out
    tau = np.partition(scores, n - m)[n - m]      # m-th largest value
    above = np.flatnonzero(scores > tau)
    ties = np.flatnonzero(scores == tau)[: m - above.size]
    chosen = np.sort(np.concatenate([above, ties]))
    out[:m] = chosen
    return out


def sparse_attention(q_heads, rows, scale):
    """Softmax attention of H query heads over m selected latent rows.

    q_heads: float64 [H, 576]; rows: float64 [m, 576].  Returns
    (O float64 [H, 512], lse float64 [H]).  m == 0 gives O = 0, lse = -inf.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H = q_heads.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, LATENT)), np.full(H, -np.inf)
    logits = scale * (q_heads @ rows.T)           # [H, m]
    mu = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mu)
    z = p.sum(axis=1, keepdims=True)
    out = (p @ rows[:, :LATENT]) / z
    lse = mu[:, 0] + np.log(z[:, 0])
    return out, lse


# --------------------------------------------------------------------------
# Batches of sequences (contiguous or paged caches)
# --------------------------------------------------------------------------

@dataclass
class Seqs:
    """Host description of a batch.

    ctx_len[b]: cached positions of sequence b, the new tokens included.
    cu_q: query-token offsets [B + 1], or None for one query per sequence.
    Query i of sequence b sits at position ctx_len[b] - q_len[b] + i.
    block_table: [B, n_pages] page ids, or None for a contiguous cache in
    which sequence b's row s is physical row b * seq_stride + s.  In a paged
    cache it is row block_table[b, s // page_size] * page_size + s % page_size.
    """
    ctx_len: np.ndarray
    cu_q: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    page_size: int = 64
    seq_stride: int = 0

    @property
    def num_seqs(self):
        return int(len(self.ctx_len))

    def q_len(self, b):
        if self.cu_q is None:
            return 1
        return int(self.cu_q[b + 1] - self.cu_q[b])

    def first_token(self, b):
        return b if self.cu_q is None else int(self.cu_q[b])

    @property
    def num_tokens(self):
        return self.num_seqs if self.cu_q is None else int(self.cu_q[-1])

    def token_positions(self):
        """[(b, t)] for every query token in order."""
        out = []
        for b in range(self.num_seqs):
            ql = self.q_len(b)
            for i in range(ql):
                out.append((b, int(self.ctx_len[b]) - ql + i))
        return out

    def physical_rows(self, b, positions):
        positions = np.asarray(positions, dtype=np.int64)
        if self.block_table is None:
            return b * int(self.seq_stride) + positions
        pages = np.asarray(self.block_table[b], dtype=np.int64)[positions // self.page_size]
        return pages * self.page_size + positions % self.page_size


def decode_rows(raw, dtype, rows):
    """Stored rows -> float64.  dtype: 'bf16' (uint16 bits), 'e4m3'
    (uint8 codes) or 'fp8_656' (packed FP8 latent rows)."""
    sel = np.asarray(raw)[rows]
    if dtype == "bf16":
        return formats.bf16_bits_to_f64(sel)
    if dtype == "e4m3":
        return formats.e4m3_bytes_to_f64(sel)
    if dtype == "fp8_656":
        return formats.fp8_rows_to_f64(sel)
    raise ValueError(dtype)


def score_topk(seqs, q_idx, k_idx, k_dtype, head_w, top_k, k_scale=None, tokens=None):
    """Indexer + Top-K for the listed tokens (default: all).

    q_idx: uint16 [T, H_I, d_I] bf16 bits; k_idx: [rows, d_I] raw (uint16
    bf16 bits or uint8 e4m3); head_w: float32 [T, H_I]; k_scale: float32
    [rows] or None.  Returns int32 [len(tokens), top_k].
    """
    pos = seqs.token_positions()
    if tokens is None:
        tokens = range(len(pos))
    tokens = list(tokens)
    out = np.empty((len(tokens), int(top_k)), dtype=np.int32)
    cache_b, cache_keys, cache_scale = None, None, None
    for r, tok in enumerate(tokens):
        b, t = pos[tok]
        if b != cache_b:
            phys = seqs.physical_rows(b, np.arange(int(seqs.ctx_len[b])))
            cache_keys = decode_rows(k_idx, k_dtype, phys)
            cache_scale = None if k_scale is None else np.asarray(k_scale, np.float64)[phys]
            cache_b = b
        q = formats.bf16_bits_to_f64(q_idx[tok])
        w = np.asarray(head_w[tok], dtype=np.float64)
        s = indexer_scores(q, cache_keys[: t + 1], w,
                           None if cache_scale is None else cache_scale[: t + 1])
        out[r] = topk_select(s, top_k)
    return out


def attention(seqs, q, kv, kv_dtype, idx, scale, tokens=None):
    """Sparse attention for the listed tokens (default: all).

    q: uint16 [T, H, 576] bf16 bits; kv: raw latent rows ('bf16' uint16
    [rows, 576] or 'fp8_656' uint8 [rows, 656]); idx: int32 [n_tokens, K]
    holding the index row of each listed token.  Entries < 0 or >= ctx_len
    of the token's sequence are skipped.  Returns (O [n, H, 512], lse [n, H]).
    """
    pos = seqs.token_positions()
    if tokens is None:
        tokens = range(len(pos))
    tokens = list(tokens)
    H = q.shape[1]
    out = np.empty((len(tokens), H, LATENT), dtype=np.float64)
    lse = np.empty((len(tokens), H), dtype=np.float64)
    for r, tok in enumerate(tokens):
        b, _t = pos[tok]
        sel = np.asarray(idx[r], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < int(seqs.ctx_len[b]))]
        rows = decode_rows(kv, kv_dtype, seqs.physical_rows(b, sel))
        qh = formats.bf16_bits_to_f64(q[tok])
        out[r], lse[r] = sparse_attention(qh, rows, scale)
    return out, lse
