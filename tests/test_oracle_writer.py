"""Pins of the oracle's FP8 latent-row writer (CPU).

The writer (oracle/writer.py) is pinned against what the definition fixes:
every E4M3FN code round-trips, values halfway between two codes go to the
even one and values just off halfway to the nearer one (the definition of
round-to-nearest-even, checked at every pair of neighbouring codes), torch's
own float8_e4m3fn conversion (a library routine) agrees on random values, a
hand-built row with exactly representable tiles gives the codes written out
by hand, and decoding any written row stays within half a code step of the
input.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import writer as W


def _finite_codes():
    return [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_encode_round_trips_every_code():
    for c in _finite_codes():
        assert W.e4m3_encode(F.E4M3_TABLE[c]) == c, hex(c)


def test_e4m3_encode_halfway_goes_to_even_code():
    for c in range(0x7E):
        lo, hi = F.E4M3_TABLE[c], F.E4M3_TABLE[c + 1]
        mid = (lo + hi) / 2.0                           # exact in float64
        even = c if c % 2 == 0 else c + 1
        assert W.e4m3_encode(mid) == even, (hex(c), mid)
        assert W.e4m3_encode(-mid) == 0x80 | even
        assert W.e4m3_encode(np.nextafter(mid, np.inf)) == c + 1
        assert W.e4m3_encode(np.nextafter(mid, -np.inf)) == c


def test_e4m3_encode_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 3000), rng.normal(0, 1, 3000), rng.normal(0, 1e-2, 2000)])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([W.e4m3_encode(x) for x in v], dtype=np.uint8)
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(got, ref)


def _bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_writer_hand_built_row():
    row = np.zeros(576, dtype=np.float32)
    # tile 0: amax 56 -> scale 56 / 448 = 0.125 exactly; value v -> v / 0.125
    row[0], row[1], row[2], row[3] = 56.0, 1.5, -0.125, 0.0625
    # tile 1: all zero -> scale 0, codes 0
    # tile 2: amax 448 -> scale 1; a negative zero keeps its sign
    row[256], row[257] = -448.0, -0.0
    # tile 3: amax 2**-3 -> scale 2**-3 / 448 (not a power of two)
    row[384] = 0.125
    row[512:] = np.arange(64, dtype=np.float32) * 0.5 - 8.0   # rope
    out = W.fp8_rows_from_bf16(_bits(row)[None, :])[0]
    codes = out[:512]
    scales = out[512:528].view(np.float32)
    # 56 / 0.125 = 448 -> 0x7E; 1.5 / 0.125 = 12 = 1.5 * 2^3 -> 0 1010 100 = 0x54;
    # -0.125 / 0.125 = -1 -> 1 0111 000 = 0xB8; 0.0625 / 0.125 = 0.5 -> 0 0110 000 = 0x30
    assert list(codes[:4]) == [0x7E, 0x54, 0xB8, 0x30]
    assert np.all(codes[4:128] == 0)
    assert scales[0] == np.float32(0.125)
    assert scales[1] == 0.0 and np.all(codes[128:256] == 0)
    assert scales[2] == np.float32(1.0)
    assert codes[256] == 0xFE and codes[257] == 0x80         # -448; -0 keeps its sign
    assert scales[3] == np.float32(np.float32(0.125) / np.float32(448.0))
    assert codes[384] == 0x7E                                # amax maps to 448
    assert np.array_equal(out[528:].view(np.uint16), _bits(row[512:]))


def test_writer_decodes_within_half_a_code_step():
    rng = np.random.default_rng(11)
    rows = np.concatenate([rng.normal(0, 1, (6, 576)), rng.normal(0, 1, (2, 576)) * 1e-3]).astype(np.float32)
    rows[7, :128] = 0.0
    bits = _bits(rows)
    x = F.bf16_bits_to_f64(bits)
    packed = W.fp8_rows_from_bf16(bits)
    back = F.fp8_rows_to_f64(packed)
    assert np.array_equal(back[:, 512:], x[:, 512:])         # rope unchanged
    scales = packed[:, 512:528].view(np.float32).astype(np.float64)
    for r in range(rows.shape[0]):
        for j in range(4):
            t = x[r, 128 * j:128 * (j + 1)]
            d = back[r, 128 * j:128 * (j + 1)]
            s = scales[r, j]
            assert s == pytest.approx(np.max(np.abs(t)) / 448.0, rel=1e-7, abs=0)
            # half a step: 2^-4 relative for normal codes, 2^-10 absolute
            # (in units of the scale) for subnormal ones, plus the fp32
            # division's own rounding
            bound = np.maximum(np.abs(t) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20)
            assert np.all(np.abs(d - t) <= bound)


def test_key_writer_unscaled_integers_are_exact():
    # integer keys in [-16, 16] are exact E4M3 values: scale 1.0 keeps them
    k = np.arange(-16, 17, dtype=np.float32)
    k = np.concatenate([k, np.zeros(128 - k.size, np.float32)])[None, :]
    codes, scales = W.e4m3_keys_from_bf16(_bits(k), scaled=False)
    assert scales is None
    assert np.array_equal(F.e4m3_bytes_to_f64(codes), k.astype(np.float64))
    # 500 clamps to 448; 17 lies halfway between 16 and 18 and goes to the even code (16)
    c2, _ = W.e4m3_keys_from_bf16(_bits(np.array([[500.0, -500.0, 17.0, 19.0]], np.float32)), scaled=False)
    assert list(F.e4m3_bytes_to_f64(c2[0])) == [448.0, -448.0, 16.0, 20.0]


def test_key_writer_scaled_rows():
    rng = np.random.default_rng(13)
    k = rng.integers(-8, 9, (5, 64)).astype(np.float32)
    k[2] = 0.0
    k[3, 7] = 8.0
    codes, scales = W.e4m3_keys_from_bf16(_bits(k), scaled=True)
    for r in range(5):
        amax = np.max(np.abs(k[r]))
        assert scales[r] == np.float32(np.float32(amax) / np.float32(448.0))
        if amax == 0:
            assert np.all(codes[r] == 0)
            continue
        back = F.e4m3_bytes_to_f64(codes[r]) * scales[r]
        # the largest key maps to the largest code; every key within half a code step
        assert np.max(np.abs(F.e4m3_bytes_to_f64(codes[r]))) == 448.0
        bound = np.maximum(np.abs(k[r]) * 2.0 ** -4, scales[r] * 2.0 ** -10) * (1 + 2.0 ** -20)
        assert np.all(np.abs(back - k[r]) <= bound)


def test_mx_block_follows_the_shared_exponent_rule():
    # amax 4 -> e = floor(log2 4) - 8 = -6: 4 -> 256 (0x78), -3 -> -192 (0xF4), 1 -> 64 (0x68)
    codes, e8 = W.mx_block_quantize([4.0, -3.0, 1.0, 0.0] + [0.0] * 28)
    assert e8 == 127 - 6 and list(codes[:4]) == [0x78, 0xF4, 0x68, 0x00]
    # the largest element lands in [256, 448] (or saturates to 448 above it)
    rng = np.random.default_rng(3)
    for _ in range(200):
        v = rng.normal(0, 10.0 ** rng.uniform(-6, 6), 32)
        c, e8 = W.mx_block_quantize(v)
        top = np.max(np.abs(F.E4M3_TABLE[c]))
        assert 256.0 <= top <= 448.0
        back = F.E4M3_TABLE[c] * 2.0 ** (e8 - 127)
        # within half a code step, or saturated at 448 (|v| / 2^e in (448, 512))
        step = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** (e8 - 127 - 9))
        ok = (np.abs(back - v) <= step) | (np.abs(v) / 2.0 ** (e8 - 127) > 448.0)
        assert np.all(ok)
    z, e8 = W.mx_block_quantize(np.zeros(32))
    assert e8 == 0 and np.all(z == 0)


def test_mxfp8_round_trip_integer_keys():
    rng = np.random.default_rng(5)
    k = rng.integers(-8, 9, (6, 128)).astype(np.float64)
    k[2, :32] = 0.0
    codes, exps = W.mxfp8_from_values(k)
    assert codes.shape == (6, 128) and exps.shape == (6, 4)
    assert np.array_equal(F.mxfp8_to_f64(codes, exps), k)
    assert exps[2, 0] == 0                                   # all-zero block: exponent byte 0
