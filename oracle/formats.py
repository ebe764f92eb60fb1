"""Exact decoding of the stored number formats into float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only tests/, the smoke check and the bench's CPU-baseline leg do.

The oracle reads the same bytes the GPU reads and turns them into float64
values with no rounding:

* bf16: the upper half of an IEEE-754 binary32; widening is a 16-bit shift.
* e4m3 ("FP8 E4M3FN", the OCP 8-bit float): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals when the exponent field is 0, the two
  codes S.1111.111 are NaN and there is no infinity.  Page 1 of the pages
  ("Hierarchical Quantization", the layered-strategy list) and page 4 (section
  4) call for an FP8 KV cache; the pages do not name the FP8 variant, and the
  OCP E4M3FN reading is the one taken here.
* The packed FP8 latent row (656 bytes): 512 e4m3 latent values, then 4
  little-endian fp32 scales (one per 128-element tile of the latent part,
  the per-token tile of 128 named on page 1 "Hierarchical Quantization" and
  page 4 section 4), then 64 bf16 rope values.  Latent value j decodes to
  e4m3[j] * scale[j // 128]; the rope part is bf16 as stored.
"""
import numpy as np

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE
FP8_ROW_BYTES = LATENT + 4 * 4 + ROPE * 2  # 656
FP8_TILE = 128


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_value(code):
    """Value of one OCP E4M3FN code (0..255), written out from the definition."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1 - bias)
        return sign * (man_field / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_bytes_to_f64(codes):
    """e4m3 codes (uint8 array) -> float64 through the 256-entry table."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp8_rows_to_f64(rows):
    """Packed 656-byte latent rows (uint8 [n, 656]) -> float64 [n, 576]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    assert rows.ndim == 2 and rows.shape[1] == FP8_ROW_BYTES
    n = rows.shape[0]
    lat = e4m3_bytes_to_f64(rows[:, :LATENT])
    scales = rows[:, LATENT:LATENT + 16].copy().view("<f4").astype(np.float64)  # [n, 4]
    rope_bits = rows[:, LATENT + 16:].copy().view("<u2")                        # [n, 64]
    out = np.empty((n, ROW), dtype=np.float64)
    for tile in range(LATENT // FP8_TILE):
        sl = slice(tile * FP8_TILE, (tile + 1) * FP8_TILE)
        out[:, sl] = lat[:, sl] * scales[:, tile:tile + 1]
    out[:, LATENT:] = bf16_bits_to_f64(rope_bits)
    return out


# MXFP8 index keys: rows of 128 e4m3 codes, and per row 4 E8M0 scale bytes
# (one per block of 32 values; the scale of a block is 2^(byte - 127)), kept
# in an array of their own.  The pages quantise the index to MXFP8 with
# groups of 32 ("Hierarchical Quantization", index-cache bullet, in Day 0
# Inference Support for New LLM Architectures; section 4 of Day 0 Inference
# Adaptation and Performance Optimization for New Models); the storage
# layout is this library's.
MX_BLOCK = 32
MX_D = 128


def mxfp8_to_f64(codes, exps):
    """MXFP8 keys (codes uint8 [n, 128], E8M0 bytes uint8 [n, 4]) -> float64
    [n, 128], exactly."""
    codes = E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    e = np.asarray(exps, dtype=np.uint8).astype(np.int64) - 127
    return codes * np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=1)
