"""FP8 latent-row writer, written from its definition (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only tests/, the smoke check and the bench's CPU-baseline leg do.

The FP8 KV cache keeps every latent row as per-token tiles of 128 values,
each with its own scale computed online from the row ("Hierarchical
Quantization", KV cache bullet, in Day 0 Inference Support for New LLM
Architectures; section 4 of Day 0 Inference Adaptation and Performance
Optimization for New Models).  The pages give the tile size but not the
scale rule or the rounding; the reading taken here:

* scale_j = amax_j / 448 in fp32 (amax_j: the largest |value| of tile j, so
  the largest value maps to the largest finite E4M3FN value, 448);
* code = E4M3(clamp(value / scale_j, -448, 448)), the division in fp32 and
  the E4M3 rounding to the nearest value, ties to the even code (last
  mantissa bit 0), the sign kept (a negative value that rounds to zero gives
  -0); an all-zero tile has scale 0 and codes 0;
* the 64 rope values are stored unchanged as bf16.

The packed row is the 656-byte layout decoded by formats.fp8_rows_to_f64.
Index keys (e4m3_keys_from_bf16) follow the same rule with one scale per
key row, or are stored with scale 1.0.
"""
import numpy as np

from .formats import E4M3_TABLE, FP8_ROW_BYTES, FP8_TILE, LATENT, ROPE, ROW

E4M3_MAX = 448.0
# finite non-negative codes 0x00 .. 0x7E in increasing value order
_POS_CODES = np.arange(0x7F)
_POS_VALUES = E4M3_TABLE[_POS_CODES]


def e4m3_encode(x):
    """Nearest E4M3FN code of a value with |x| <= 448, ties to the even
    code, sign kept.  x: float (any float type; its exact value is used)."""
    x = float(x)
    if not (abs(x) <= E4M3_MAX):
        raise ValueError("e4m3_encode: |x| must be <= 448 (clamp first): %r" % x)
    neg = np.signbit(x)
    a = abs(x)
    # largest code whose value is <= a, and the next one up
    lo = int(np.searchsorted(_POS_VALUES, a, side="right")) - 1
    if _POS_VALUES[lo] == a or lo == len(_POS_VALUES) - 1:
        code = lo
    else:
        hi = lo + 1
        d_lo, d_hi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
        if d_lo < d_hi:
            code = lo
        elif d_hi < d_lo:
            code = hi
        else:
            code = lo if lo % 2 == 0 else hi
    return (0x80 | code) if neg else code


def fp8_rows_from_bf16(bits):
    """bf16 latent rows (uint16 bit patterns [n, 576]) -> packed FP8 rows
    (uint8 [n, 656])."""
    bits = np.asarray(bits, dtype=np.uint16)
    if bits.ndim != 2 or bits.shape[1] != ROW:
        raise ValueError("rows must be [n, 576]")
    n = bits.shape[0]
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    out = np.zeros((n, FP8_ROW_BYTES), dtype=np.uint8)
    for r in range(n):
        scales = np.zeros(LATENT // FP8_TILE, dtype=np.float32)
        for j in range(LATENT // FP8_TILE):
            tile = f32[r, j * FP8_TILE:(j + 1) * FP8_TILE]
            amax = np.float32(np.max(np.abs(tile)))
            scale = np.float32(amax / np.float32(E4M3_MAX))
            scales[j] = scale
            for i, v in enumerate(tile):
                if scale > 0:
                    q = np.float32(v / scale)
                    q = np.float32(min(max(float(q), -E4M3_MAX), E4M3_MAX))
                else:
                    q = np.float32(0.0)
                out[r, j * FP8_TILE + i] = e4m3_encode(q)
        out[r, LATENT:LATENT + 16] = scales.view(np.uint8)
        out[r, LATENT + 16:] = bits[r, LATENT:].view(np.uint8)
    return out


def e4m3_keys_from_bf16(bits, scaled):
    """bf16 index-key rows (uint16 bit patterns [n, d]) -> (e4m3 codes uint8
    [n, d], per-row fp32 scales [n] or None).

    scaled=False: code = E4M3(clamp(k, -448, 448)) (keys stored with scale
    1.0, as the FP8-key workloads hold them).  scaled=True: per row, scale =
    amax / 448 in fp32 and code = E4M3(clamp(k / scale, -448, 448)) (fp32
    division), an all-zero row getting scale 0 and codes 0; the indexer then
    reads the scale as its per-row key scale."""
    bits = np.asarray(bits, dtype=np.uint16)
    if bits.ndim != 2:
        raise ValueError("keys must be [n, d]")
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    n, d = f32.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros(n, dtype=np.float32) if scaled else None
    for r in range(n):
        if scaled:
            amax = np.float32(np.max(np.abs(f32[r])))
            scale = np.float32(amax / np.float32(E4M3_MAX))
            scales[r] = scale
        for i in range(d):
            v = f32[r, i]
            if scaled:
                q = np.float32(v / scale) if scale > 0 else np.float32(0.0)
            else:
                q = v
            q = np.float32(min(max(float(q), -E4M3_MAX), E4M3_MAX))
            codes[r, i] = e4m3_encode(q)
    return codes, scales


def mx_block_quantize(values):
    """One MXFP8 block, from the OCP MX definition for E4M3 elements: shared
    exponent e = floor(log2(amax)) - 8 (8: the exponent of E4M3's largest
    normal), clamped to [-127, 127], and e = -127 (byte 0) for an all-zero
    block; codes E4M3(clamp(v / 2^e, -448, 448)).  values: exact floats
    (32 of them).  Returns (codes uint8 [32], E8M0 byte = e + 127)."""
    v = np.asarray(values, dtype=np.float64)
    amax = float(np.max(np.abs(v)))
    if amax == 0.0:
        return np.zeros(v.shape, dtype=np.uint8), 0
    e = int(np.frexp(amax)[1]) - 1 - 8   # frexp: amax = m 2^E, m in [0.5, 1), so floor(log2) = E - 1
    e = min(max(e, -127), 127)
    q = np.clip(v / 2.0 ** e, -E4M3_MAX, E4M3_MAX)   # exact: division by a power of two
    return np.array([e4m3_encode(x) for x in q], dtype=np.uint8), e + 127


def mxfp8_from_values(values):
    """float rows [n, 128] -> MXFP8 keys: codes uint8 [n, 128] and E8M0
    block exponents uint8 [n, 4]."""
    from .formats import MX_BLOCK, MX_D
    v = np.asarray(values, dtype=np.float64)
    codes = np.zeros((v.shape[0], MX_D), dtype=np.uint8)
    exps = np.zeros((v.shape[0], MX_D // MX_BLOCK), dtype=np.uint8)
    for r in range(v.shape[0]):
        for b in range(MX_D // MX_BLOCK):
            c, e8 = mx_block_quantize(v[r, b * MX_BLOCK:(b + 1) * MX_BLOCK])
            codes[r, b * MX_BLOCK:(b + 1) * MX_BLOCK] = c
            exps[r, b] = e8
    return codes, exps
