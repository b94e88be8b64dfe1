"""Pins of the CPU oracle against things other than itself (CPU only).

* brute force: pure-Python evaluation of every element on tiny inputs;
* library special cases: torch's float64 math SDPA (with and without grouped heads),
  complex multiplication for RoPE, torch.transpose for the relayout;
* hand-derived fixtures under tests/golden/;
* invariants the mathematics fixes (row sums, Skv = 1, constant V, q = 0, key
  permutation, GQA = repeated MHA, RoPE identity / norm / relative shift / offset
  continuation / axis reduction / pairing permutation, CFG closed forms).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from bruteforce import bf_attention, bf_lse, bf_position, bf_rope

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape, seed=None):
    r = np.random.default_rng(seed) if seed is not None else RNG
    return r.standard_normal(shape)


def _maxrel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def _evalexpr(e):
    if isinstance(e, str):
        return eval(e, {"__builtins__": {}}, {"cos": math.cos, "sin": math.sin, "sqrt": math.sqrt,
                                               "log": math.log})
    return float(e)


# ------------------------------------------------------------------ brute force
ROPE_CASES = [
    # grid, pairs, offset, D, interleaved
    ((10,), (4,), (3,), 8, False),
    ((10,), (4,), (3,), 8, True),
    ((3, 4), (2, 2), (5, 7), 8, False),
    ((3, 4), (3, 5), (0, 2), 16, True),
    ((2, 2, 3), (3, 3, 2), (1, 2, 3), 16, False),
    ((2, 2, 3), (2, 3, 3), (0, 0, 0), 16, True),
]


@pytest.mark.parametrize("grid,pairs,offset,D,inter", ROPE_CASES)
def test_rope_matches_bruteforce(grid, pairs, offset, D, inter):
    S = int(np.prod(grid))
    x = _rand(S, 3, D)
    got = oracle.rope(x, grid, pairs, offset, 10000.0, inter)
    exp = np.array(bf_rope(x.tolist(), grid, pairs, offset, 10000.0, inter))
    assert _maxrel(got, exp) <= 1e-13


@pytest.mark.parametrize("grid,pairs,offset,D,inter", ROPE_CASES[2:])
def test_rope_global_freq_matches_bruteforce(grid, pairs, offset, D, inter):
    S = int(np.prod(grid))
    x = _rand(S, 3, D)
    got = oracle.rope(x, grid, pairs, offset, 10000.0, inter, global_freq=True)
    exp = np.array(bf_rope(x.tolist(), grid, pairs, offset, 10000.0, inter, global_freq=True))
    assert _maxrel(got, exp) <= 1e-13


def test_rope_global_freq_reductions():
    # one axis: the global ladder and the per-axis ladder are the same ladder
    x = _rand(10, 2, 16)
    assert np.array_equal(oracle.rope(x, (10,), (8,), (3,), global_freq=True), oracle.rope(x, (10,), (8,), (3,)))
    # every axis at the same position p: plain 1-D RoPE over the head at position p
    # (the text-token case of an MRoPE decoder)
    y = _rand(1, 2, 16)
    for p in (0, 5, 77):
        got = oracle.rope(y, (1, 1, 1), (2, 3, 3), (p, p, p), global_freq=True)
        exp = oracle.rope(y, (1,), (8,), (p,))
        assert np.max(np.abs(got - exp)) <= 1e-15
    # the two ladders differ for a multi-axis split (the mode is not a no-op)
    z = _rand(6, 1, 16)
    assert not np.allclose(oracle.rope(z, (2, 3), (4, 4), (1, 2), global_freq=True), oracle.rope(z, (2, 3), (4, 4), (1, 2)))


ATTN_CASES = [
    # Sq, P, Hq, Hkv, D
    (5, 0, 2, 2, 8),
    (7, 3, 2, 1, 8),
    (6, 8, 4, 2, 16),
    (9, 4, 4, 1, 16),
    (1, 0, 1, 1, 8),
    (12, 5, 8, 2, 8),
]


@pytest.mark.parametrize("Sq,P,Hq,Hkv,D", ATTN_CASES)
def test_attention_matches_bruteforce(Sq, P, Hq, Hkv, D):
    q = _rand(Sq, Hq, D)
    k = _rand(Sq, Hkv, D)
    v = _rand(Sq, Hkv, D)
    pk = _rand(P, Hkv, D) if P else None
    pv = _rand(P, Hkv, D) if P else None
    got = oracle.attention(q, k, v, pk, pv)
    exp = np.array(bf_attention(q.tolist(), k.tolist(), v.tolist(),
                                pk.tolist() if P else None, pv.tolist() if P else None))
    assert _maxrel(got, exp) <= 1e-13


@pytest.mark.parametrize("Sq,P,Hq,Hkv,D", ATTN_CASES)
def test_lse_matches_bruteforce(Sq, P, Hq, Hkv, D):
    q = _rand(Sq, Hq, D)
    k = _rand(Sq, Hkv, D)
    pk = _rand(P, Hkv, D) if P else None
    got = oracle.attention_lse(q, k, k, pk, pk)
    exp = np.array(bf_lse(q.tolist(), k.tolist(), pk.tolist() if P else None))
    assert got.shape == (Hq, Sq)
    assert np.max(np.abs(got - exp)) <= 1e-12


def test_lse_closed_forms():
    D = 8
    q = _rand(3, 2, D)
    k1 = _rand(1, 1, D)
    # one key: the log-sum-exp is that key's scaled score
    s = (q[:, :, :] @ k1[0, 0]) / math.sqrt(D)                        # [3, 2]
    assert np.max(np.abs(oracle.attention_lse(q, k1, k1) - s.T)) <= 1e-14
    # q = 0: every score is 0, so lse = log(number of keys) (prefix and own both count)
    z = np.zeros((4, 2, D))
    assert np.max(np.abs(oracle.attention_lse(z, _rand(4, 1, D), _rand(4, 1, D), _rand(5, 1, D), _rand(5, 1, D))
                      - math.log(9))) <= 1e-14
    # n copies of one key: lse = s + log n
    k5 = np.repeat(k1, 5, axis=0)
    assert np.max(np.abs(oracle.attention_lse(q, k5, k5) - (s.T + math.log(5)))) <= 1e-13
    # the softmax weights are exp(s - lse)
    q2, k2 = _rand(6, 4, D), _rand(6, 2, D)
    pk2 = _rand(3, 2, D)
    wts = oracle.attention_weights(q2, k2, k2, pk2, pk2)               # [R, Hq, Skv]
    keys = np.concatenate([pk2, k2], 0)
    for h in range(4):
        sc = q2[:, h, :] @ keys[:, h // 2, :].T / math.sqrt(D)
        lse = oracle.attention_lse(q2, k2, k2, pk2, pk2)[h]
        assert np.max(np.abs(np.exp(sc - lse[:, None]) - wts[:, h, :])) <= 1e-14


@pytest.mark.parametrize("cuts", [(4,), (3, 9), (1, 6, 10), (5, 6, 7, 8)])
def test_merge_of_key_splits_matches_bruteforce(cuts):
    # disjoint contiguous ranges of [prefix ++ own], one of them straddling the prefix end
    Sq, P, Hq, Hkv, D = 5, 6, 4, 2, 8
    q, k, v = _rand(Sq, Hq, D), _rand(Sq, Hkv, D), _rand(Sq, Hkv, D)
    pk, pv = _rand(P, Hkv, D), _rand(P, Hkv, D)
    K, V = np.concatenate([pk, k], 0), np.concatenate([pv, v], 0)
    bounds = (0,) + cuts + (P + Sq,)
    po, pl = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        po.append(oracle.attention(q, K[a:b], V[a:b]))
        pl.append(oracle.attention_lse(q, K[a:b], V[a:b]))
    o, lse = oracle.merge_partials(po, pl)
    exp_o = np.array(bf_attention(q.tolist(), k.tolist(), v.tolist(), pk.tolist(), pv.tolist()))
    exp_l = np.array(bf_lse(q.tolist(), k.tolist(), pk.tolist()))
    assert _maxrel(o, exp_o) <= 1e-13
    assert np.max(np.abs(lse - exp_l)) <= 1e-12
    # the parts may come in any order
    o2, lse2 = oracle.merge_partials(po[::-1], pl[::-1])
    assert _maxrel(o2, o) <= 1e-14 and np.max(np.abs(lse2 - lse)) <= 1e-14


def test_merge_special_cases():
    q, k, v = _rand(4, 2, 8), _rand(7, 1, 8), _rand(7, 1, 8)
    o, l = oracle.attention(q, k, v), oracle.attention_lse(q, k, v)
    # one part is returned unchanged
    o1, l1 = oracle.merge_partials([o], [l])
    assert _maxrel(o1, o) <= 1e-15 and np.max(np.abs(l1 - l)) <= 1e-15
    # an empty part (lse = -inf, output 0) changes nothing
    o2, l2 = oracle.merge_partials([np.zeros_like(o), o], [np.full_like(l, -np.inf), l])
    assert _maxrel(o2, o) <= 1e-15 and np.max(np.abs(l2 - l)) <= 1e-15
    # ... whatever its output holds (an empty set's output is 0/0)
    o3, _ = oracle.merge_partials([np.full_like(o, np.nan), o], [np.full_like(l, -np.inf), l])
    assert _maxrel(o3, o) <= 1e-15
    # two halves with equal lse: plain average, lse + log 2
    oa, ob = _rand(4, 2, 8), _rand(4, 2, 8)
    om, lm = oracle.merge_partials([oa, ob], [l, l])
    assert _maxrel(om, 0.5 * (oa + ob)) <= 1e-15 and np.max(np.abs(lm - (l + math.log(2)))) <= 1e-14
    # a part far below the other carries (almost) no weight
    om, lm = oracle.merge_partials([oa, ob], [l, l - 800.0])
    assert _maxrel(om, oa) <= 1e-15
    with pytest.raises(ValueError):
        oracle.merge_partials([oa], [np.full_like(l, -np.inf)])


def test_rope_then_attention_matches_bruteforce():
    grid, pairs, off = (3, 4), (2, 2), (6, 6)
    S, P, Hq, Hkv, D = 12, 6, 4, 2, 8
    q, k, v = _rand(S, Hq, D), _rand(S, Hkv, D), _rand(S, Hkv, D)
    pk, pv = _rand(P, Hkv, D), _rand(P, Hkv, D)
    got = oracle.attention(oracle.rope(q, grid, pairs, off), oracle.rope(k, grid, pairs, off), v, pk, pv)
    qb = bf_rope(q.tolist(), grid, pairs, off)
    kb = bf_rope(k.tolist(), grid, pairs, off)
    exp = np.array(bf_attention(qb, kb, v.tolist(), pk.tolist(), pv.tolist()))
    assert _maxrel(got, exp) <= 1e-13


def test_positions_bruteforce():
    for grid, off in [((64,), (32,)), ((60, 65), (0, 0)), ((21, 30, 52), (3, 5, 7)), ((2, 3, 4), (1, 0, 2))]:
        pos = oracle.positions(grid, off)
        S = int(np.prod(grid))
        for i in list(range(0, S, max(1, S // 97))) + [S - 1]:
            assert list(pos[i]) == bf_position(i, grid, off)
    # a hand-checked 3-D case: 17 = 1*12 + 1*4 + 1 on a 2x3x4 grid
    assert list(oracle.positions((2, 3, 4), (10, 20, 30))[17]) == [11, 21, 31]


# ------------------------------------------------------------------ library special cases
@pytest.mark.parametrize("Sq,P,Hq,Hkv,D", [(33, 0, 4, 4, 16), (40, 0, 8, 2, 32), (17, 9, 4, 1, 8)])
def test_attention_matches_torch_math_sdpa(Sq, P, Hq, Hkv, D):
    q, k, v = _rand(Sq, Hq, D), _rand(Sq, Hkv, D), _rand(Sq, Hkv, D)
    pk = _rand(P, Hkv, D) if P else None
    pv = _rand(P, Hkv, D) if P else None
    got = oracle.attention(q, k, v, pk, pv)
    K = np.concatenate([pk, k], 0) if P else k
    V = np.concatenate([pv, v], 0) if P else v
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1, Hq, Sq, D]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()
    tv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=False, enable_gqa=(Hq != Hkv))
    ref = ref[0].permute(1, 0, 2).numpy()
    assert _maxrel(got, ref) <= 1e-12


def test_rope_matches_complex_rotation():
    # each pair (a, b) as the complex number a + ib multiplied by exp(i*phi)
    grid, pairs, off, D = (5, 6), (3, 5), (2, 9), 16
    S = 30
    x = _rand(S, 2, D)
    got = oracle.rope(x, grid, pairs, off)
    z = x[:, :, : D // 2] + 1j * x[:, :, D // 2:]
    freqs = [10000.0 ** (-u / 3.0) for u in range(3)] + [10000.0 ** (-u / 5.0) for u in range(5)]
    rows = np.array([(i // 6 + 2, i % 6 + 9) for i in range(S)], dtype=np.float64)
    phi = np.concatenate([rows[:, :1] * np.array(freqs[:3]), rows[:, 1:] * np.array(freqs[3:])], 1)
    zr = z * np.exp(1j * phi)[:, None, :]
    exp = np.concatenate([zr.real, zr.imag], 2)
    assert _maxrel(got, exp) <= 1e-13


def test_relayout_matches_torch_transpose():
    src = torch.randn(3, 2, 4, 5, 6).to(torch.bfloat16)
    got = oracle.relayout(src.view(torch.int16).numpy(), 0)
    exp = src.transpose(2, 3).contiguous().view(torch.int16).numpy()
    assert got.shape == exp.shape and np.array_equal(got, exp)
    back = oracle.relayout(got, 1)
    assert np.array_equal(back, src.view(torch.int16).numpy())


# ------------------------------------------------------------------ hand-derived fixtures
def test_golden_relayout():
    g = json.load(open(os.path.join(GOLDEN, "relayout_small.json")))
    src = np.array(g["replay"], dtype=np.int32)
    assert list(src.shape) == g["replay_shape"]
    got = oracle.relayout(src, 0)
    assert np.array_equal(got, np.array(g["online"], dtype=np.int32))
    assert np.array_equal(oracle.relayout(got, 1), src)


def test_golden_rope():
    g = json.load(open(os.path.join(GOLDEN, "rope_d4.json")))
    S = g["grid"][0]
    x = np.zeros((S, 1, 4))
    x[g["token"], 0] = g["x"]
    got = oracle.rope(x, g["grid"], g["pairs"], g["offset"], g["theta"], False)[g["token"], 0]
    exp = [_evalexpr(e) for e in g["expected"]]
    assert np.max(np.abs(got - exp)) <= 1e-14
    x[g["token"], 0] = g["interleaved_x"]
    got = oracle.rope(x, g["grid"], g["pairs"], g["offset"], g["theta"], True)[g["token"], 0]
    exp = [_evalexpr(e) for e in g["interleaved_expected"]]
    assert np.max(np.abs(got - exp)) <= 1e-14


def test_golden_attention():
    g = json.load(open(os.path.join(GOLDEN, "attention_2key.json")))
    q = np.array(g["q"], dtype=np.float64)
    k = np.array([[[_evalexpr(e) for e in h] for h in row] for row in g["k"]])
    v = np.array(g["v"], dtype=np.float64)
    # own tokens: the single query token plus a second key token; query row 0 only
    got = oracle.attention(np.concatenate([q, q], 0), k, v, rows=np.array([0]))
    assert np.max(np.abs(got - np.array(g["expected"]))) <= 1e-14


def test_golden_cfg():
    g = json.load(open(os.path.join(GOLDEN, "cfg_small.json")))
    got = oracle.cfg_combine(g["cond"], g["uncond"], g["guidance"])
    assert np.array_equal(got, np.array(g["expected"]))


# ------------------------------------------------------------------ invariants
def test_weights_rows_sum_to_one():
    q, k, v = _rand(11, 4, 16), _rand(11, 2, 16), _rand(11, 2, 16)
    w = oracle.attention_weights(q, k, v, _rand(5, 2, 16), _rand(5, 2, 16))
    assert w.shape == (11, 4, 16)
    assert np.max(np.abs(w.sum(-1) - 1.0)) <= 1e-14
    assert np.all(w > 0)


def test_single_key_returns_v():
    q, k, v = _rand(1, 2, 8), _rand(1, 2, 8), _rand(1, 2, 8)
    assert np.array_equal(oracle.attention(q, k, v), v)


def test_constant_v_returns_that_row():
    S, H, D = 9, 2, 8
    row = _rand(D)
    v = np.broadcast_to(row, (S, H, D)).copy()
    o = oracle.attention(_rand(S, H, D), _rand(S, H, D), v)
    assert np.max(np.abs(o - row)) <= 1e-14


def test_zero_query_gives_mean_of_values():
    S, P, H, D = 7, 3, 2, 8
    k, v, pk, pv = _rand(S, H, D), _rand(S, H, D), _rand(P, H, D), _rand(P, H, D)
    o = oracle.attention(np.zeros((S, H, D)), k, v, pk, pv)
    mean = np.concatenate([pv, v], 0).mean(0)
    assert np.max(np.abs(o - mean[None])) <= 1e-14


def test_key_permutation_invariance_across_prefix_boundary():
    S, P, Hq, Hkv, D = 8, 5, 4, 2, 8
    q, k, v, pk, pv = _rand(S, Hq, D), _rand(S, Hkv, D), _rand(S, Hkv, D), _rand(P, Hkv, D), _rand(P, Hkv, D)
    base = oracle.attention(q, k, v, pk, pv)
    K = np.concatenate([pk, k], 0)
    V = np.concatenate([pv, v], 0)
    perm = np.random.default_rng(7).permutation(S + P)
    K2, V2 = K[perm], V[perm]
    o2 = oracle.attention(q, K2[P:], V2[P:], K2[:P], V2[:P])
    assert _maxrel(o2, base) <= 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    S, P, Hq, Hkv, D = 6, 4, 8, 2, 8
    q, k, v, pk, pv = _rand(S, Hq, D), _rand(S, Hkv, D), _rand(S, Hkv, D), _rand(P, Hkv, D), _rand(P, Hkv, D)
    G = Hq // Hkv
    rep = lambda t: np.repeat(t, G, axis=1)  # noqa: E731  kv head g serves q heads g*G .. g*G+G-1
    a = oracle.attention(q, k, v, pk, pv)
    b = oracle.attention(q, rep(k), rep(v), rep(pk), rep(pv))
    assert np.array_equal(a, b)


def test_row_subset_equals_full():
    q, k, v = _rand(10, 2, 8), _rand(10, 2, 8), _rand(10, 2, 8)
    full = oracle.attention(q, k, v)
    rows = np.array([9, 0, 4])
    assert np.max(np.abs(oracle.attention(q, k, v, rows=rows) - full[rows])) <= 1e-15


def test_rope_position_zero_is_identity_and_norm_preserved():
    x = _rand(12, 3, 16)
    y = oracle.rope(x, (3, 4), (4, 4), (0, 0))
    assert np.array_equal(y[0], x[0])                  # token 0 at offset 0: every angle is 0
    D = 16
    na = x[:, :, : D // 2] ** 2 + x[:, :, D // 2:] ** 2
    nb = y[:, :, : D // 2] ** 2 + y[:, :, D // 2:] ** 2
    assert np.max(np.abs(na - nb)) <= 1e-13


def test_rope_relative_shift_invariance():
    # <rope(q, m), rope(k, n)> depends only on m - n: shifting every position by c
    # (own tokens through the offset, prefix keys through explicit rotation) keeps O.
    S, P, H, D = 8, 4, 2, 16
    q, k, v, rk, pv = _rand(S, H, D), _rand(S, H, D), _rand(S, H, D), _rand(P, H, D), _rand(P, H, D)
    outs = []
    for c in (0, 37):
        pk = oracle.rope(rk, (P,), (D // 2,), (c,))
        outs.append(oracle.attention(oracle.rope(q, (S,), (D // 2,), (P + c,)),
                                     oracle.rope(k, (S,), (D // 2,), (P + c,)), v, pk, pv))
    assert _maxrel(outs[0], outs[1]) <= 1e-12


def test_rope_offset_continues_the_prefix():
    # prefix keys rotated at 0..P-1 plus own tokens at offset P equals attention over
    # the whole rotated sequence of P+S tokens, read at its last S query rows
    S, P, H, D = 6, 5, 2, 8
    xq, xk, xv = _rand(P + S, H, D), _rand(P + S, H, D), _rand(P + S, H, D)
    full = oracle.attention(oracle.rope(xq, (P + S,), (D // 2,), (0,)),
                            oracle.rope(xk, (P + S,), (D // 2,), (0,)), xv, rows=np.arange(P, P + S))
    pk = oracle.rope(xk[:P], (P,), (D // 2,), (0,))
    split = oracle.attention(oracle.rope(xq[P:], (S,), (D // 2,), (P,)),
                             oracle.rope(xk[P:], (S,), (D // 2,), (P,)), xv[P:], pk, xv[:P])
    assert _maxrel(split, full) <= 1e-13


def test_rope_2d_with_unit_axis_reduces_to_1d():
    S, H, p0, p1 = 7, 2, 3, 5
    D = 2 * (p0 + p1)
    x = _rand(S, H, D)
    y = oracle.rope(x, (1, S), (p0, p1), (0, 0))
    # section 0 (pairs 0..p0-1) sits at position 0: unchanged
    assert np.array_equal(y[:, :, :p0], x[:, :, :p0])
    assert np.array_equal(y[:, :, D // 2: D // 2 + p0], x[:, :, D // 2: D // 2 + p0])
    # section 1 is a 1-D RoPE over d = 2*p1 with pairs (p0+u, p0+u+D/2)
    sub = np.concatenate([x[:, :, p0: D // 2], x[:, :, D // 2 + p0:]], 2)
    ys = oracle.rope(sub, (S,), (p1,), (0,))
    assert _maxrel(np.concatenate([y[:, :, p0: D // 2], y[:, :, D // 2 + p0:]], 2), ys) <= 1e-14


def test_rope_interleaved_is_permuted_half_split():
    S, H, D = 9, 2, 16
    x = _rand(S, H, D)
    perm = np.array([2 * j for j in range(D // 2)] + [2 * j + 1 for j in range(D // 2)])
    a = oracle.rope(x, (3, 3), (4, 4), (1, 2), interleaved=True)
    b = oracle.rope(x[:, :, perm], (3, 3), (4, 4), (1, 2), interleaved=False)
    assert np.array_equal(a[:, :, perm], b)


def test_cfg_closed_forms():
    c, u = _rand(100), _rand(100)
    assert np.array_equal(oracle.cfg_combine(c, u, 0.0), u)
    assert np.max(np.abs(oracle.cfg_combine(c, u, 1.0) - c)) <= 4e-16 * np.max(np.abs(c) + np.abs(u))
    a, b = oracle.cfg_combine(c, u, 2.0), oracle.cfg_combine(c, u, 6.0)
    mid = oracle.cfg_combine(c, u, 4.0)
    assert np.max(np.abs(mid - 0.5 * (a + b))) <= 1e-14
