"""Plain float64 definitions of every step of the attention hot path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
leg call this module; the HIP product path never does.

Sources (pages as titled; sections named):
* "NeoPP: LightLLM integration and KV replay", section "KV file layout": the online
  KV tensor is [layers, 2, seq, kv_heads, head_dim]; the replay files hold
  [layers, 2, kv_heads, seq, head_dim]; loading swaps dimensions 2 and 3 and saving
  applies transpose(2, 3). Position offsets are passed explicitly, never inferred
  from tensor sizes. Intro: the KV cache plus position offsets condition the DiT,
  two KV branches (cond / uncond) when CFG is on.
* KLiteInfer README, section "架构" (architecture): bidirectional attention is two
  strided-batched GEMMs with a softmax between them; RoPE / 2-D RoPE / MRoPE
  operators; intro bullets: SigLIP ViT with 2-D RoPE and bidirectional attention,
  GQA in the decoder.
* "LingBot-Video" recipe, "Key Parameters": guidance_scale, CFG active above 1.0.

Readings where the pages are silent (the same choices are fixed for the HIP path):
rotary pairs are half-split (x[j], x[j + D/2]) unless ``interleaved`` (x[2j], x[2j+1]);
each axis of a multi-axis RoPE is an ordinary 1-D RoPE over its own contiguous
section of pairs with d_k = 2*pairs_k; theta = 10000; the offset is added to every
axis; prefix keys are used as stored (already rotated by the encoder that wrote the
cache); GQA groups are contiguous (q head h reads kv head h // (Hq/Hkv)); index 0 of
the size-2 KV dimension is K; own tokens are ordered row-major over the grid; the
CFG combination is uncond + s*(cond - uncond).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------------
# KV relayout ("KV file layout": replay [L,2,H,S,D] <-> online [L,2,S,H,D])
# ---------------------------------------------------------------------------------
def relayout(src: np.ndarray, direction: int = 0) -> np.ndarray:
    """Swap dimensions 2 and 3 of a [L, 2, A, B, D] tensor, as a new contiguous array.

    direction 0 maps replay [L,2,H,S,D] to online [L,2,S,H,D]; direction 1 maps online
    to replay. Both are the same axis swap; the values are copied bit for bit (the
    input's dtype is kept).
    """
    if src.ndim != 5 or src.shape[1] != 2:
        raise ValueError("relayout expects [L, 2, A, B, D]")
    if direction not in (0, 1):
        raise ValueError("direction must be 0 or 1")
    return np.ascontiguousarray(np.swapaxes(src, 2, 3))


# ---------------------------------------------------------------------------------
# Positions of own tokens (row-major over the grid, plus the per-axis offset)
# ---------------------------------------------------------------------------------
def positions(grid: Sequence[int], offset: Sequence[int]) -> np.ndarray:
    """Integer positions [S, n_axes] of own tokens i = 0..S-1.

    Token i is unravelled row-major over ``grid`` (axis 0 slowest) and each axis
    coordinate is shifted by that axis's offset.
    """
    grid = [int(g) for g in grid]
    S = int(np.prod(grid))
    out = np.zeros((S, len(grid)), dtype=np.int64)
    for i in range(S):
        rem = i
        for ax in range(len(grid) - 1, -1, -1):
            out[i, ax] = rem % grid[ax] + int(offset[ax])
            rem //= grid[ax]
    return out


# ---------------------------------------------------------------------------------
# RoPE (KLiteInfer "架构": RoPE, 2-D RoPE, MRoPE operators)
# ---------------------------------------------------------------------------------
def rope_angles(pos: np.ndarray, pairs: Sequence[int], theta: float = 10000.0,
                global_freq: bool = False) -> np.ndarray:
    """Rotation angle [S, D/2] of every (token, rotary pair).

    Pairs are split into contiguous sections, one per axis in axis order. By default
    each section has its own frequency ladder: pair j of axis k with local index u
    rotates by pos[:, k] * theta ** (-2u / d_k), where d_k = 2 * pairs[k]. With
    ``global_freq`` there is one ladder over all D/2 pairs, as in the MRoPE of the
    KLiteInfer page's ERNIE decoder (section "架构"): pair j rotates by
    pos[:, k] * theta ** (-2j / D) and the sections only choose the axis k.
    """
    S = pos.shape[0]
    half = int(sum(pairs))
    ang = np.zeros((S, half), dtype=np.float64)
    j = 0
    for k, pk in enumerate(pairs):
        d_k = 2 * int(pk)
        for u in range(int(pk)):
            if global_freq:
                inv_freq = float(theta) ** (-2.0 * j / (2 * half))
            else:
                inv_freq = float(theta) ** (-2.0 * u / d_k)
            ang[:, j] = pos[:, k].astype(np.float64) * inv_freq
            j += 1
    return ang


def rope(x: np.ndarray, grid: Sequence[int], pairs: Sequence[int], offset: Sequence[int],
         theta: float = 10000.0, interleaved: bool = False, rows: Optional[np.ndarray] = None,
         global_freq: bool = False) -> np.ndarray:
    """Rotate x [S, H, D] (one branch) by the positions of its tokens; returns float64.

    Half-split pairs (a, b) = (j, j + D/2), or interleaved (2j, 2j+1):
    a' = a cos(phi) - b sin(phi), b' = a sin(phi) + b cos(phi).
    With ``rows``, x holds only those tokens ([len(rows), H, D]) of the grid.
    """
    x = _f64(x)
    S, H, D = x.shape
    if 2 * int(sum(pairs)) != D:
        raise ValueError("sum of pairs must be head_dim / 2")
    pos = positions(grid, offset)
    if rows is not None:
        pos = pos[np.asarray(rows)]
    if pos.shape[0] != S:
        raise ValueError("x has a different number of tokens than the grid (or rows)")
    phi = rope_angles(pos, pairs, theta, global_freq)                  # [S, D/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    if interleaved:
        ia = np.arange(0, D, 2)
        ib = ia + 1
    else:
        ia = np.arange(0, D // 2)
        ib = ia + D // 2
    a = x[:, :, ia]
    b = x[:, :, ib]
    out = np.empty_like(x)
    out[:, :, ia] = a * c - b * s
    out[:, :, ib] = a * s + b * c
    return out


# ---------------------------------------------------------------------------------
# Attention over [prefix ++ own] (KLiteInfer "架构": GEMM, softmax, GEMM; non-causal)
# ---------------------------------------------------------------------------------
def _keys_values(k: np.ndarray, v: np.ndarray, prefix_k: Optional[np.ndarray],
                 prefix_v: Optional[np.ndarray]):
    k = _f64(k)
    v = _f64(v)
    if prefix_k is None or prefix_k.shape[0] == 0:
        return k, v
    return np.concatenate([_f64(prefix_k), k], 0), np.concatenate([_f64(prefix_v), v], 0)


def attention_weights(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      prefix_k: Optional[np.ndarray] = None, prefix_v: Optional[np.ndarray] = None,
                      scale: Optional[float] = None, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Softmax weights [R, Hq, P+S] of one branch (keys = prefix rows then own rows)."""
    q = _f64(q)
    Sq, Hq, D = q.shape
    K, _ = _keys_values(k, v, prefix_k, prefix_v)
    Hkv = K.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    r = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.zeros((len(r), Hq, K.shape[0]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = sc * (q[r, h, :] @ K[:, g, :].T)                        # [R, Skv]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = w / w.sum(axis=1, keepdims=True)
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              prefix_k: Optional[np.ndarray] = None, prefix_v: Optional[np.ndarray] = None,
              scale: Optional[float] = None, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Non-causal attention output [R, Hq, D] of one branch, in float64.

    q [Sq,Hq,D] (already rotated), k/v [Sq,Hkv,D] own tokens (k already rotated),
    prefix_k/prefix_v [P,Hkv,D] or None. For q head h the kv head is h // (Hq/Hkv);
    keys are the prefix rows followed by the own rows; every query sees every key.
    s_j = scale * <q, K_j>, m = max_j s_j, w_j = exp(s_j - m), o = sum_j w_j V_j / sum_j w_j.
    ``rows`` selects a subset of query rows (rows are independent).
    """
    q = _f64(q)
    Sq, Hq, D = q.shape
    K, V = _keys_values(k, v, prefix_k, prefix_v)
    Hkv = K.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    r = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.zeros((len(r), Hq, V.shape[2]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = sc * (q[r, h, :] @ K[:, g, :].T)                        # [R, Skv]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        z = w.sum(axis=1, keepdims=True)
        out[:, h, :] = (w @ V[:, g, :]) / z
    return out


def attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  prefix_k: Optional[np.ndarray] = None, prefix_v: Optional[np.ndarray] = None,
                  scale: Optional[float] = None, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Log-sum-exp of the scaled scores, [Hq, R] (natural log), of one branch.

    lse_i = log sum_j exp(s_ij) over the same keys as ``attention`` (prefix rows then own
    rows), with s_ij = scale * <q_i, K_j>; evaluated as m + log sum_j exp(s_ij - m),
    m = max_j s_ij. It is the softmax normaliser of the KLiteInfer "架构" attention: the
    weights are exp(s_ij - lse_i).
    """
    q = _f64(q)
    Sq, Hq, D = q.shape
    K, _ = _keys_values(k, v, prefix_k, prefix_v)
    Hkv = K.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    r = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.zeros((Hq, len(r)), dtype=np.float64)
    for h in range(Hq):
        s = sc * (q[r, h, :] @ K[:, h // G, :].T)                   # [R, Skv]
        m = s.max(axis=1)
        out[h, :] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def merge_partials(parts_o: Sequence[np.ndarray], parts_lse: Sequence[np.ndarray]):
    """Combine attention results over disjoint key sets into the result over their union.

    parts_o[p] [R, Hq, D] is the attention output over key set p alone and parts_lse[p]
    [Hq, R] its log-sum-exp (-inf for an empty set, whose output values are then ignored). Softmax over the union has the
    normaliser exp(lse) = sum_p exp(lse_p), and each part's normalised output enters with
    weight exp(lse_p - lse), so
        lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) * o_p.
    This is the rescaling step of the online softmax (the softmax between the two GEMMs of
    the KLiteInfer "架构" attention) applied to whole key blocks; it is what a key range
    split across workgroups, or across devices (the NeoPP replay's sequence-parallel
    degree), needs. Returns (o [R, Hq, D], lse [Hq, R]).
    """
    if len(parts_o) == 0 or len(parts_o) != len(parts_lse):
        raise ValueError("need one lse per part and at least one part")
    L = np.stack([_f64(x) for x in parts_lse])                       # [n, Hq, R]
    m = L.max(axis=0)                                                 # [Hq, R]
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one non-empty part")
    e = np.exp(L - m[None])                                           # exp(-inf) = 0
    lse = m + np.log(e.sum(axis=0))
    wts = np.exp(L - lse[None])                                       # [n, Hq, R]
    o = np.zeros(_f64(parts_o[0]).shape, dtype=np.float64)
    for p, op in enumerate(parts_o):
        # an empty key set has no output (0/0): its term is absent from the sum
        term = wts[p].T[:, :, None] * _f64(op)
        o += np.where(np.isneginf(L[p]).T[:, :, None], 0.0, term)
    return o, lse


# ---------------------------------------------------------------------------------
# Classifier-free guidance ("Key Parameters": guidance_scale, active above 1.0)
# ---------------------------------------------------------------------------------
def cfg_combine(cond: np.ndarray, uncond: np.ndarray, guidance: float) -> np.ndarray:
    """uncond + guidance * (cond - uncond), in float64."""
    c = _f64(cond)
    u = _f64(uncond)
    return u + float(guidance) * (c - u)
