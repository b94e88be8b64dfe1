"""Pure-Python brute force used to pin the oracle on tiny inputs.

Written independently of ``oracle/`` (plain lists, ``math`` and ``math.fsum``; no
numpy): the RoPE angle of each pair, the rotation, the score of every key, the
softmax and the weighted sum are spelled out element by element.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence


def bf_position(i: int, grid: Sequence[int], offset: Sequence[int]) -> List[int]:
    # coordinates of token i in a row-major grid, axis 0 slowest
    n = len(grid)
    strides = [1] * n
    for a in range(n - 2, -1, -1):
        strides[a] = strides[a + 1] * grid[a + 1]
    return [(i // strides[a]) % grid[a] + offset[a] for a in range(n)]


def bf_rope_token(x: List[float], pos: List[int], pairs: Sequence[int], theta: float,
                  interleaved: bool, global_freq: bool = False) -> List[float]:
    D = len(x)
    half = D // 2
    out = list(x)
    j = 0
    for axis, npairs in enumerate(pairs):
        for u in range(npairs):
            if global_freq:
                # one ladder over every pair of the head; the section picks the axis
                freq = math.pow(theta, -(2.0 * j) / D)
            else:
                freq = math.pow(theta, -(2.0 * u) / (2.0 * npairs))
            phi = pos[axis] * freq
            ia, ib = (2 * j, 2 * j + 1) if interleaved else (j, j + half)
            a, b = x[ia], x[ib]
            out[ia] = a * math.cos(phi) - b * math.sin(phi)
            out[ib] = a * math.sin(phi) + b * math.cos(phi)
            j += 1
    return out


def bf_rope(x, grid, pairs, offset, theta=10000.0, interleaved=False, global_freq=False):
    """x: nested lists [S][H][D] -> rotated nested lists."""
    return [[bf_rope_token(list(map(float, x[i][h])), bf_position(i, grid, offset), pairs, theta, interleaved,
                           global_freq)
             for h in range(len(x[i]))] for i in range(len(x))]


def bf_attention(q, k, v, pk=None, pv=None, scale: Optional[float] = None):
    """q [Sq][Hq][D], k/v [S][Hkv][D], pk/pv [P][Hkv][D] or None -> o [Sq][Hq][D]."""
    Sq, Hq, D = len(q), len(q[0]), len(q[0][0])
    keys = (list(pk) if pk is not None else []) + list(k)
    vals = (list(pv) if pv is not None else []) + list(v)
    Hkv = len(keys[0])
    group = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    out = []
    for i in range(Sq):
        row = []
        for h in range(Hq):
            g = h // group
            s = [sc * math.fsum(float(q[i][h][d]) * float(keys[j][g][d]) for d in range(D))
                 for j in range(len(keys))]
            m = max(s)
            w = [math.exp(t - m) for t in s]
            z = math.fsum(w)
            row.append([math.fsum(w[j] * float(vals[j][g][d]) for j in range(len(keys))) / z
                        for d in range(len(vals[0][g]))])
        out.append(row)
    return out


def bf_lse(q, k, pk=None, scale: Optional[float] = None):
    """q [Sq][Hq][D], k [S][Hkv][D], pk [P][Hkv][D] or None -> [Hq][Sq] of log sum_j exp(s_j)."""
    Sq, Hq, D = len(q), len(q[0]), len(q[0][0])
    keys = (list(pk) if pk is not None else []) + list(k)
    group = Hq // len(keys[0])
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    out = [[0.0] * Sq for _ in range(Hq)]
    for h in range(Hq):
        g = h // group
        for i in range(Sq):
            s = [sc * math.fsum(float(q[i][h][d]) * float(keys[j][g][d]) for d in range(D))
                 for j in range(len(keys))]
            m = max(s)
            out[h][i] = m + math.log(math.fsum(math.exp(t - m) for t in s))
    return out


def bf_e4m3_value(code: int) -> float:
    """Value of one E4M3 code by its field definition (None for NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)


def bf_e4m3_encode(x: float) -> int:
    """Nearest finite E4M3 code by scanning every code (ties: even code); beyond the
    largest finite value, the largest; NaN -> 0x7F."""
    if x != x:
        return 0x7F
    best, bd = None, None
    for c in range(0x7F):
        v = bf_e4m3_value(c)
        d = abs(abs(x) - v)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    if math.copysign(1.0, x) < 0:
        best |= 0x80
    return best


def bf_fp8_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, by search (0 for amax = 0)."""
    if amax == 0.0:
        return 0
    for e in range(-160, 160):
        if amax <= math.ldexp(448.0, e):
            return e
    raise ValueError(amax)
