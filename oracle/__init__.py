"""CPU oracle (test infrastructure only).

Plain float64 NumPy implementation of the indexer score, Top-K selection and
sparse latent attention, and of the FP8 latent-row writer (in the fp32 steps
its definition fixes), written from the pages' definitions.  It is used by
tests/, the smoke check and the bench's CPU-baseline leg only, and it shares
no code with the HIP library.
"""
from .formats import (E4M3_TABLE, FP8_ROW_BYTES, bf16_bits_to_f64,
                      e4m3_bytes_to_f64, e4m3_value, fp8_rows_to_f64)
from .reference import (Seqs, attention, decode_rows, indexer_scores,
                        score_topk, sparse_attention, topk_select)
from .writer import e4m3_encode, e4m3_keys_from_bf16, fp8_rows_from_bf16

__all__ = [
    "E4M3_TABLE", "FP8_ROW_BYTES", "bf16_bits_to_f64", "e4m3_bytes_to_f64",
    "e4m3_value", "fp8_rows_to_f64", "Seqs", "attention", "decode_rows",
    "indexer_scores", "score_topk", "sparse_attention", "topk_select",
    "e4m3_encode", "e4m3_keys_from_bf16", "fp8_rows_from_bf16",
]
