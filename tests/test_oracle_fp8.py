"""Pins of the FP8 (E4M3) oracle: values the format definition fixes, a brute-force
encoder that scans every code, and the scale-exponent rule by search."""
import math

import numpy as np
import pytest

from oracle import fp8
from bruteforce import bf_e4m3_encode, bf_e4m3_value, bf_fp8_exponent


def test_decode_fixed_values():
    # values the format definition fixes: zeros, the subnormal and normal extremes, 1, 2,
    # the largest finite value and the NaN codes
    d = fp8.e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x40, 0x7E, 0xFE, 0x7F, 0xFF],
                                 dtype=np.uint8))
    assert d[0] == 0.0 and not np.signbit(d[0]) and d[1] == 0.0 and np.signbit(d[1])
    assert d[2] == 2.0 ** -9 and d[3] == 7 * 2.0 ** -9 and d[4] == 2.0 ** -6
    assert d[5] == 1.0 and d[6] == 1.875 and d[7] == 2.0 and d[8] == 448.0 and d[9] == -448.0
    assert np.isnan(d[10]) and np.isnan(d[11])


def test_decode_matches_field_definition_and_order():
    codes = np.arange(256, dtype=np.uint8)
    d = fp8.e4m3_decode(codes)
    for c in range(256):
        v = bf_e4m3_value(c)
        assert (v is None and np.isnan(d[c])) or d[c] == v
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # strictly increasing magnitudes
    assert np.array_equal(d[0x80:0xFF], -pos)             # sign symmetry


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_matches_bruteforce():
    rng = np.random.default_rng(5)
    vals = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                      # exact ties
    xs = np.concatenate([
        rng.normal(0, 1, 300), rng.normal(0, 100, 200), rng.uniform(-2.0 ** -6, 2.0 ** -6, 200),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, -0.0, 447.9, 448.0, 460.0, 464.0, 1e6, -1e6, 2.0 ** -11, -2.0 ** -10],
    ])
    got = fp8.e4m3_encode(xs)
    exp = np.array([bf_e4m3_encode(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, exp)
    assert fp8.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_exponent_rule_matches_search():
    rng = np.random.default_rng(6)
    xs = list(rng.lognormal(0, 4, 300)) + [448.0, 224.0, 896.0, 1.0, 2.0 ** -20, 3.5, 1e30]
    xs += [float(np.nextafter(np.float64(v), np.inf)) for v in (448.0, 224.0, 0.875)]
    xs += [float(np.nextafter(np.float64(v), 0.0)) for v in (448.0, 224.0, 0.875)]
    for a in xs:
        assert fp8.fp8_exponent(a) == max(-127, bf_fp8_exponent(a)), a
    assert fp8.fp8_exponent(1e-40) == -127 and fp8.fp8_exponent(448.0 * 2.0 ** -127) == -127
    assert fp8.fp8_exponent(0.0) == 0
    assert fp8.fp8_exponent(448.0) == 0 and fp8.fp8_exponent(449.0) == 1 and fp8.fp8_exponent(224.0) == -1


def test_quantize_error_bound_and_range():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, (2, 33, 3, 16)) * np.array([1.0, 1e-3, 50.0])[None, None, :, None]
    codes, e = fp8.quantize_fp8(x)
    assert codes.dtype == np.uint8 and e.shape == (2, 3)
    deq = fp8.dequantize_fp8(codes, e)
    for b in range(2):
        for h in range(3):
            sl = x[b, :, h, :]
            assert e[b, h] == bf_fp8_exponent(float(np.max(np.abs(sl))))
            y = sl * 2.0 ** -int(e[b, h])
            assert np.max(np.abs(y)) <= 448.0
            r = deq[b, :, h, :] * 2.0 ** -int(e[b, h])
            # half a unit in the last place: 2^-4 relative (normal), 2^-10 absolute (subnormal)
            assert np.all(np.abs(y - r) <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10) + 1e-300)
    # the largest magnitude of each slice lands in the top binade (no wasted range)
    top = np.max(np.abs(fp8.e4m3_decode(codes)), axis=(1, 3))
    assert np.all(top > 224.0 - 1e-9)


# ---- block scaling (one E8M0 scale per 32-element run of head_dim)

def test_blocks_golden():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_blocks_small.json")))
    x = np.zeros(g["shape"])
    for r, c, v in g["nonzero_inputs"]:
        x[r, c] = v
    codes, scales = fp8.quantize_fp8_blocks(x)
    assert scales.dtype == np.uint8 and scales.tolist() == g["expected_scales"]
    want = np.zeros(g["shape"], dtype=np.uint8)
    for r, c, v in g["expected_nonzero_codes"]:
        want[r, c] = v
    assert np.array_equal(codes, want)


def _graded(rng, shape, span=6):
    """N(0,1) values with each 32-element run scaled by its own power of two in
    2^-span..2^span, so that neighbouring blocks get different exponents."""
    x = rng.normal(0, 1, shape)
    runs = x.reshape(shape[:-1] + (shape[-1] // 32, 32))
    runs *= np.exp2(rng.integers(-span, span + 1, runs.shape[:-1]))[..., None]
    return runs.reshape(shape)


def test_blocks_reduce_to_per_slice_quantization():
    # a block is quantized as quantize_fp8 quantizes a slice holding only that block
    rng = np.random.default_rng(11)
    x = _graded(rng, (2, 5, 3, 64))
    x[1, 2, 0, 32:] = 0.0                                   # an all-zero block
    codes, scales = fp8.quantize_fp8_blocks(x)
    assert codes.shape == x.shape and scales.shape == (2, 5, 3, 2)
    for idx in np.ndindex(2, 5, 3, 2):
        b, s, h, k = idx
        run = x[b, s, h, 32 * k:32 * k + 32].reshape(1, 1, 1, 32)
        c1, e1 = fp8.quantize_fp8(run)
        assert np.array_equal(codes[b, s, h, 32 * k:32 * k + 32], c1.reshape(32))
        assert int(scales[idx]) == int(e1[0, 0]) + 127
    assert scales[1, 2, 0, 1] == 127 and not codes[1, 2, 0, 32:].any()


def test_blocks_exponents_minimal_and_error_bound():
    rng = np.random.default_rng(12)
    x = _graded(rng, (3, 7, 2, 128))
    x[0, 0, 0, :32] *= 2.0 ** -140                          # below the E8M0 range: e held at -127
    codes, scales = fp8.quantize_fp8_blocks(x)
    e = scales.astype(np.int64) - 127
    runs = x.reshape(3, 7, 2, 4, 32)
    amax = np.max(np.abs(runs), axis=-1)
    assert np.all(amax <= 448.0 * np.exp2(e.astype(float)))
    assert np.all((e == -127) | (amax > 448.0 * np.exp2(e - 1.0)))
    assert e[0, 0, 0, 0] == -127
    for i, a in enumerate(amax.ravel()[:50]):
        assert e.ravel()[i] == max(-127, bf_fp8_exponent(float(a)))
    y = runs * np.exp2(-e.astype(float))[..., None]
    r = fp8.e4m3_decode(codes).reshape(y.shape)
    assert np.all(np.abs(y - r) <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10) + 1e-300)
    deq = fp8.dequantize_fp8_blocks(codes, scales)
    assert np.array_equal(deq.reshape(y.shape), r * np.exp2(e.astype(float))[..., None])
    # values already on the grid come back unchanged (a block whose maximum rounded down to
    # 224 * 2^e may take e - 1, with doubled codes of the same values)
    c2, s2 = fp8.quantize_fp8_blocks(deq)
    assert np.array_equal(fp8.dequantize_fp8_blocks(c2, s2), deq)


def test_blocks_finer_than_per_slice():
    # E4M3 keeps its relative precision over its normal range (2^-6 .. 448, about 2^15), so
    # a scale per block gains where the runs of one slice span more than that: there the
    # small runs of a per-slice scale fall into the subnormals or to zero
    rng = np.random.default_rng(13)
    x = _graded(rng, (1, 64, 1, 128), span=14)
    cs, es = fp8.quantize_fp8(x)
    cb, sb = fp8.quantize_fp8_blocks(x)
    def rel(deq):   # mean over blocks of the block's largest error relative to its largest value
        d = np.abs(deq - x).reshape(-1, 32).max(axis=1)
        return float(np.mean(d / np.abs(x).reshape(-1, 32).max(axis=1)))
    r_slice, r_block = rel(fp8.dequantize_fp8(cs, es)), rel(fp8.dequantize_fp8_blocks(cb, sb))
    assert r_block <= 2.0 ** -4 and r_block < 0.25 * r_slice
