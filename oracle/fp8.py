"""FP8 (OCP E4M3) encoding and the quantization of q and k for the fp8 score GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name fp8 variants of the DiT (NeoPP page, "Run the replay examples": the
``*_fp8`` launchers) but give no recipe. The reading fixed here: q and k are stored as
OCP FP8 E4M3 codes with one power-of-two scale per (branch, head); the score GEMM
multiplies the decoded codes times their scales; everything after the scores (softmax,
P.V with bf16 V) is the bf16 path. Decoding is exact, so the attention of the fp8 path is
the attention of the dequantized q and k, which ``reference.attention`` evaluates. A
second, finer reading (``quantize_fp8_blocks``) gives each run of 32 head_dim elements
its own power-of-two scale.

E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities): exponent field
e > 0 encodes (1 + m/8) * 2^(e-7), e = 0 encodes (m/8) * 2^-6; the code S.1111.111 is NaN,
so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes (uint8 array); NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def _finite_table() -> Tuple[np.ndarray, np.ndarray]:
    """Non-negative finite codes 0x00..0x7E and their values, increasing."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, e4m3_decode(codes)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the code with an even mantissa, i.e. the
    even code number); magnitudes beyond 448 saturate to +-448; NaN -> 0x7F. The sign of
    a value that rounds to zero is kept (-0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _finite_table()
    a = np.abs(x)
    # index of the largest table value <= a (a >= 0)
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 1)
    hi = np.clip(lo + 1, 0, len(vals) - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0) & (hi != lo))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.int64)
    mag = np.where(a >= E4M3_MAX, 0x7E, mag)
    out = np.where(np.signbit(x), mag | 0x80, mag)
    out = np.where(np.isnan(x), 0x7F, out)
    return out.astype(np.uint8)


def fp8_exponent(amax: float) -> int:
    """The scale exponent of a slice with largest magnitude amax: the smallest integer e
    with amax <= 448 * 2^e (so every scaled value fits the finite range); 0 for amax = 0.
    The scale 2^e is consumed as an E8M0 value (2^(v - 127), v in 0..254), so e is held at
    -127 or above (a slice below 448 * 2^-127 keeps e = -127 and still fits)."""
    a = float(amax)
    if a == 0.0:
        return 0
    m, E = math.frexp(a)            # a = m * 2^E, 0.5 <= m < 1; 448 = 0.875 * 2^9
    return max(-127, E - 9 + (1 if m > 0.875 else 0))


def quantize_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize x [B, S, H, D] per (branch, head): e[b, h] = fp8_exponent(max |x[b, :, h, :]|),
    codes = e4m3_encode(x * 2^-e). Returns (codes uint8 [B, S, H, D], e int8 [B, H])."""
    x = np.asarray(x, dtype=np.float64)
    B, S, H, D = x.shape
    e = np.zeros((B, H), dtype=np.int64)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            e[b, h] = fp8_exponent(np.max(np.abs(x[b, :, h, :])) if S > 0 else 0.0)
            codes[b, :, h, :] = e4m3_encode(x[b, :, h, :] * 2.0 ** (-int(e[b, h])))
    return codes, e.astype(np.int8)


def dequantize_fp8(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """codes [B, S, H, D] and exponents [B, H] -> values (float64)."""
    v = e4m3_decode(codes)
    return v * np.exp2(np.asarray(e, dtype=np.float64))[:, None, :, None]


# ---- block scaling -------------------------------------------------------------------------
# A second reading of the recipe, finer than one scale per (branch, head): the scale is
# shared by each run of BLOCK = 32 consecutive elements of the head_dim axis of one
# (branch, token, head) row, the block size and the E8M0 scale format of the OCP
# Microscaling (MX) formats specification. The rule inside a block is the per-slice rule
# above, so a block is quantized exactly as quantize_fp8 would quantize a slice holding
# only that block's values. The scale of a block is stored as its E8M0 code e + 127
# (value 2^(code - 127)), the operand format of the matrix core's scaled fp8 products.

BLOCK = 32


def quantize_fp8_blocks(x: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize x [..., D] (D a multiple of block) per run of `block` consecutive elements
    of the last axis: e = fp8_exponent(max |run|), codes = e4m3_encode(run * 2^-e).
    Returns (codes uint8 [..., D], scales uint8 [..., D / block]) with each scale held as
    its E8M0 code e + 127."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % block != 0:
        raise ValueError(f"last axis {D} is not a multiple of {block}")
    runs = x.reshape(x.shape[:-1] + (D // block, block))
    amax = np.max(np.abs(runs), axis=-1) if runs.size else np.zeros(runs.shape[:-1])
    e = np.array([fp8_exponent(a) for a in amax.ravel()], dtype=np.int64).reshape(amax.shape)
    codes = e4m3_encode(runs * np.exp2(-e.astype(np.float64))[..., None])
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)


def dequantize_fp8_blocks(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """codes [..., D] and E8M0 scale codes [..., D / block] -> values (float64)."""
    v = e4m3_decode(codes)
    runs = v.reshape(v.shape[:-1] + (v.shape[-1] // block, block))
    s = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return (runs * s[..., None]).reshape(v.shape)
