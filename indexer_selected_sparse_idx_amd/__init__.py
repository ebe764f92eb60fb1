"""Python binding of libidxsparse.so (index-selected sparse latent attention
for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/idxsparse.h.  PyTorch provides
device memory and the current stream.  There is no fallback: if the shared
library is missing, importing the binding's entry points raises.
"""
from ._binding import (IDX_BF16, IDX_E4M3, IDX_KERNEL_ATTN, IDX_KERNEL_COMBINE,
                       IDX_KERNEL_KV_WRITE, IDX_KERNEL_SCORE, IDX_KERNEL_TOPK, IDX_KV_FP8_656, IDX_MXFP8,
                       IDX_STATIC_SCRATCH_BYTES, IdxError, Seqs, idx_key_fp8_write, idx_key_mxfp8_write, idx_kv_fp8_write, idx_score_topk, idx_score_topk_workspace,
                       idx_sparse_attn_decode, idx_sparse_attn_decode_static, idx_sparse_attn_prefill,
                       idx_sparse_attn_workspace, idx_status_string,
                       idx_timer_arm, lib, lib_path, sparse_mla_attn,
                       sparse_mla_attn_workspace)

__all__ = [
    "IDX_BF16", "IDX_E4M3", "IDX_KV_FP8_656", "IDX_MXFP8", "IDX_KERNEL_SCORE", "IDX_KERNEL_TOPK",
    "IDX_KERNEL_ATTN", "IDX_KERNEL_COMBINE", "IDX_KERNEL_KV_WRITE", "IDX_STATIC_SCRATCH_BYTES", "IdxError", "Seqs",
    "idx_key_fp8_write", "idx_key_mxfp8_write", "idx_kv_fp8_write", "idx_score_topk",
    "idx_score_topk_workspace", "idx_sparse_attn_decode", "idx_sparse_attn_decode_static",
    "idx_sparse_attn_prefill",
    "idx_sparse_attn_workspace", "idx_status_string", "idx_timer_arm", "lib", "lib_path",
    "sparse_mla_attn", "sparse_mla_attn_workspace",
]
