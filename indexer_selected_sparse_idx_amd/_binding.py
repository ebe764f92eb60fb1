"""ctypes marshalling for libidxsparse.so.

Each Python function has the name of the C entry point it calls and passes
tensor data pointers, sizes and the current HIP stream straight through.
Outputs and workspaces are allocated with torch when the caller does not
pass them (device-memory plumbing only).
"""
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# IDXSPARSE_LIB selects another build of the same library (e.g. a tuning
# variant); by default the in-tree build is used.
lib_path = os.environ.get("IDXSPARSE_LIB") or os.path.join(_HERE, "libidxsparse.so")

IDX_OK = 0
IDX_BF16, IDX_E4M3, IDX_KV_FP8_656, IDX_MXFP8 = 1, 2, 3, 4
IDX_KERNEL_SCORE, IDX_KERNEL_TOPK, IDX_KERNEL_ATTN, IDX_KERNEL_COMBINE, IDX_KERNEL_KV_WRITE = 0, 1, 2, 3, 4
FP8_ROW_BYTES = 656


class IdxError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, idx_status_string(status)))


class _IdxSeqs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("cu_q", ctypes.c_void_p),
        ("ctx_len", ctypes.c_void_p),
        ("max_q_len", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("seq_stride", ctypes.c_int64),
    ]


_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_SEQ = ctypes.POINTER(_IdxSeqs)

_SIGNATURES = {
    "idx_status_string": (ctypes.c_char_p, [_I]),
    "idx_score_topk_workspace": (_SZ, [_SEQ, _I, _I, _I]),
    "sparse_mla_attn_workspace": (_SZ, [_SEQ, _I, _I]),
    "idx_sparse_attn_workspace": (_SZ, [_SEQ, _I, _I, _I, _I]),
    "idx_score_topk": (_I, [_SEQ, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P, _P, _SZ, _P]),
    "sparse_mla_attn": (_I, [_SEQ, _P, _I, _P, _I, _P, _I, _F, _P, _P, _P, _SZ, _P]),
    "idx_sparse_attn_prefill": (_I, [_SEQ, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P, _I, _P, _I, _F,
                                     _P, _P, _P, _P, _SZ, _P]),
    "idx_sparse_attn_decode": (_I, [_SEQ, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P, _I, _P, _I, _F,
                                    _P, _P, _P, _P, _SZ, _P]),
    "idx_sparse_attn_decode_static": (_I, [_SEQ, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P, _I, _P, _I, _F,
                                           _P, _P, _P, _P]),
    "idx_kv_fp8_write": (_I, [_P, _I, _P, _P, _P]),
    "idx_key_fp8_write": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "idx_key_mxfp8_write": (_I, [_P, _I, _P, _P, _P, _P]),
    "idx_timer_arm": (_I, [_I, _P, _P]),
}


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise RuntimeError("libidxsparse.so is not built (%s); run "
                               "`python -m indexer_selected_sparse_idx_amd.build`" % lib_path)
        L = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def idx_status_string(status):
    return lib().idx_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Seqs:
    """A batch description (mirrors idx_seqs).

    ctx_len: int32 device tensor [B]; cu_q: int32 device tensor [B + 1] or
    None (one token per sequence); block_table: int32 device tensor
    [B, bt_stride] or None (contiguous cache with `seq_stride` rows per
    sequence).  max_q_len / max_ctx_len are host-side bounds.
    """

    def __init__(self, ctx_len, cu_q=None, *, max_q_len, max_ctx_len, num_tokens=None,
                 block_table=None, page_size=64, seq_stride=0):
        self.ctx_len = ctx_len
        self.cu_q = cu_q
        self.block_table = block_table
        B = int(ctx_len.shape[0])
        if num_tokens is None:
            if cu_q is not None:
                raise ValueError("num_tokens is required when cu_q is given")
            num_tokens = B
        self._c = _IdxSeqs(
            num_seqs=B, num_tokens=int(num_tokens), cu_q=_ptr(cu_q).value if cu_q is not None else None,
            ctx_len=ctx_len.data_ptr(), max_q_len=int(max_q_len), max_ctx_len=int(max_ctx_len),
            block_table=block_table.data_ptr() if block_table is not None else None,
            bt_stride=int(block_table.shape[1]) if block_table is not None else 0,
            page_size=int(page_size), seq_stride=int(seq_stride))

    @property
    def num_tokens(self):
        return self._c.num_tokens

    @property
    def ref(self):
        return ctypes.byref(self._c)


def _kdtype(t, k_scale=None):
    """Key format: bf16, E4M3 (uint8 / float8_e4m3fn codes), or MXFP8 when the
    scale argument holds uint8 E8M0 block exponents [rows, 4]."""
    if t.dtype == torch.bfloat16:
        return IDX_BF16
    if k_scale is not None and k_scale.dtype == torch.uint8:
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("MXFP8 keys must be E4M3 codes")
        return IDX_MXFP8
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return IDX_E4M3
    raise ValueError("unsupported index-key dtype %s" % t.dtype)


def _kvdtype(t):
    if t.dtype == torch.bfloat16:
        return IDX_BF16
    if t.dtype == torch.uint8 and t.shape[-1] == FP8_ROW_BYTES:
        return IDX_KV_FP8_656
    raise ValueError("unsupported latent-cache dtype %s / shape %s" % (t.dtype, tuple(t.shape)))


def _check(rc, where):
    if rc != IDX_OK:
        raise IdxError(rc, where)


def _workspace(nbytes, device, ws):
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    if nbytes == 0:
        return None, 0
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, nbytes


def idx_score_topk_workspace(seqs, H_I, d_I, top_k):
    return int(lib().idx_score_topk_workspace(seqs.ref, H_I, d_I, top_k))


def sparse_mla_attn_workspace(seqs, H, top_k):
    return int(lib().sparse_mla_attn_workspace(seqs.ref, H, top_k))


def idx_sparse_attn_workspace(seqs, H_I, d_I, H, top_k):
    return int(lib().idx_sparse_attn_workspace(seqs.ref, H_I, d_I, H, top_k))


def idx_score_topk(seqs, q_idx, k_idx, head_w, top_k, k_scale=None, out_idx=None, ws=None):
    """Indexer scores + Top-K.  Returns int32 [T, top_k] (valid first, -1 after)."""
    T, H_I, d_I = q_idx.shape
    if out_idx is None:
        out_idx = torch.empty((T, top_k), dtype=torch.int32, device=q_idx.device)
    ws, nbytes = _workspace(idx_score_topk_workspace(seqs, H_I, d_I, top_k), q_idx.device, ws)
    rc = lib().idx_score_topk(seqs.ref, _ptr(q_idx), IDX_BF16 if q_idx.dtype == torch.bfloat16 else -1,
                              _ptr(k_idx), _kdtype(k_idx, k_scale), _ptr(k_scale), _ptr(head_w),
                              H_I, d_I, top_k, _ptr(out_idx), _ptr(ws), nbytes, _stream())
    _check(rc, "idx_score_topk")
    return out_idx


def sparse_mla_attn(seqs, q, kv, idx, softmax_scale, out=None, lse=None, want_lse=True, ws=None):
    """Sparse latent attention over given indices.  Returns (out, lse)."""
    T, H, _ = q.shape
    top_k = idx.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(sparse_mla_attn_workspace(seqs, H, top_k), q.device, ws)
    rc = lib().sparse_mla_attn(seqs.ref, _ptr(q), H, _ptr(kv), _kvdtype(kv), _ptr(idx), top_k,
                               float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream())
    _check(rc, "sparse_mla_attn")
    return out, lse


def _fused(name, seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale, k_scale, out, lse,
           out_idx, want_lse, ws):
    T, H_I, d_I = q_idx.shape
    H = q.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(idx_sparse_attn_workspace(seqs, H_I, d_I, H, top_k), q.device, ws)
    rc = getattr(lib(), name)(seqs.ref, _ptr(q_idx), IDX_BF16 if q_idx.dtype == torch.bfloat16 else -1,
                              _ptr(k_idx), _kdtype(k_idx, k_scale), _ptr(k_scale), _ptr(head_w), H_I, d_I, top_k,
                              _ptr(q), H, _ptr(kv), _kvdtype(kv), float(softmax_scale),
                              _ptr(out), _ptr(lse), _ptr(out_idx), _ptr(ws), nbytes, _stream())
    _check(rc, name)
    return out, lse, out_idx


def idx_sparse_attn_prefill(seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale, k_scale=None,
                            out=None, lse=None, out_idx=None, want_lse=True, ws=None):
    """Fused indexer + sparse attention for any batch.  Returns (out, lse, out_idx)."""
    return _fused("idx_sparse_attn_prefill", seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale,
                  k_scale, out, lse, out_idx, want_lse, ws)


def idx_sparse_attn_decode(seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale, k_scale=None,
                           out=None, lse=None, out_idx=None, want_lse=True, ws=None):
    """Fused indexer + sparse attention, one token per sequence."""
    return _fused("idx_sparse_attn_decode", seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale,
                  k_scale, out, lse, out_idx, want_lse, ws)


IDX_STATIC_SCRATCH_BYTES = 64 << 20


def idx_sparse_attn_decode_static(seqs, q_idx, k_idx, head_w, top_k, q, kv, softmax_scale, k_scale=None,
                                  out=None, lse=None, out_idx=None, want_lse=True):
    """Fused decode through the entry point that allocates nothing (its
    scratch is the library's static device buffer).  Outputs not passed are
    allocated here, by the caller's side of the boundary."""
    T, H_I, d_I = q_idx.shape
    H = q.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    rc = lib().idx_sparse_attn_decode_static(
        seqs.ref, _ptr(q_idx), IDX_BF16 if q_idx.dtype == torch.bfloat16 else -1, _ptr(k_idx),
        _kdtype(k_idx, k_scale), _ptr(k_scale), _ptr(head_w), H_I, d_I, top_k, _ptr(q), H, _ptr(kv), _kvdtype(kv),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(out_idx), _stream())
    _check(rc, "idx_sparse_attn_decode_static")
    return out, lse, out_idx


def idx_kv_fp8_write(src, dst_row, kv):
    """Quantise bf16 latent rows src [n, 576] into the packed 656-byte FP8
    rows dst_row[i] of kv (uint8 [rows, 656]); entries of dst_row < 0 are
    skipped.  Returns kv."""
    n = int(src.shape[0])
    rc = lib().idx_kv_fp8_write(_ptr(src), n, _ptr(dst_row), _ptr(kv), _stream())
    _check(rc, "idx_kv_fp8_write")
    return kv


def idx_key_fp8_write(src, dst_row, k_cache, k_scale=None):
    """Store bf16 index keys src [n, d_I] as E4M3FN codes in rows dst_row[i]
    of k_cache (uint8 [rows, d_I]); with k_scale (fp32 [rows]) each row gets
    an amax/448 scale written to k_scale, without it the scale is 1.0.
    Returns k_cache."""
    n, d = int(src.shape[0]), int(src.shape[1])
    rc = lib().idx_key_fp8_write(_ptr(src), n, d, _ptr(dst_row), _ptr(k_cache), _ptr(k_scale), _stream())
    _check(rc, "idx_key_fp8_write")
    return k_cache


def idx_key_mxfp8_write(src, dst_row, k_cache, k_exp):
    """Store bf16 index keys src [n, 128] as MXFP8 in rows dst_row[i]: E4M3FN
    codes in k_cache (uint8 [rows, 128]) and E8M0 block exponents in k_exp
    (uint8 [rows, 4]).  Returns (k_cache, k_exp)."""
    n = int(src.shape[0])
    if n and int(src.shape[1]) != 128:
        raise ValueError("idx_key_mxfp8_write: keys must have 128 values")
    rc = lib().idx_key_mxfp8_write(_ptr(src), n, _ptr(dst_row), _ptr(k_cache), _ptr(k_exp), _stream())
    _check(rc, "idx_key_mxfp8_write")
    return k_cache, k_exp


def idx_timer_arm(kernel, start_event, stop_event):
    """Record torch.cuda.Event pair around the next launch of `kernel`."""
    rc = lib().idx_timer_arm(int(kernel), ctypes.c_void_p(start_event.cuda_event),
                             ctypes.c_void_p(stop_event.cuda_event))
    _check(rc, "idx_timer_arm")
