"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Bars: bit-exact for the relayout and for index selection; max slice error
max|g-r| / max(|r|, rms(r)) <= 1e-4 (fp32) / 2e-2 (bf16) for attention; RoPE and CFG
within one bf16 rounding (or fp32 rounding error) of the exact value.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from bidirectional_transformer_attention_amd.pipeline import AttentionStep
from helpers import (TOL, attention_err, cosine, f64, fold_factor, fused_q, global_maxrel, oracle_attention,
                     oracle_rope, sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def bf(x):
    return x.to(torch.bfloat16)


# ---------------------------------------------------------------------------- relayout
@pytest.mark.parametrize("shape,dtype", [((1, 2, 8, 1024, 128), torch.bfloat16), ((1, 2, 8, 128, 128), torch.bfloat16),
                                         ((3, 2, 5, 37, 72), torch.float32), ((2, 2, 3, 7, 4), torch.bfloat16),
                                         ((1, 2, 12, 256, 128), torch.bfloat16), ((2, 2, 1, 1, 8), torch.float32)])
def test_relayout_bitwise(shape, dtype):
    note(f"relayout {shape} {dtype}")
    src = synth.random_tensor(shape, 11, dtype)
    L, _, H, S, D = shape
    d_src = src.to(DEV)
    d_dst = torch.empty((L, 2, S, H, D), dtype=dtype, device=DEV)
    nx.nxattn_kv_relayout(d_src, d_dst, 0)
    back = torch.empty_like(d_src)
    nx.nxattn_kv_relayout(d_dst, back, 1)
    torch.cuda.synchronize()
    ints = torch.int16 if dtype == torch.bfloat16 else torch.int32
    exp = oracle.relayout(src.view(ints).numpy(), 0)
    assert np.array_equal(d_dst.cpu().view(ints).numpy(), exp)
    assert torch.equal(back.cpu().view(ints), src.view(ints))


# ---------------------------------------------------------------------------- rope
ROPE_CASES = [
    ("tiny_f32", None), ("vit_f32", None), ("dit1k_bf16", 8), ("video_bf16", 4),
]


def rope_check(wl, x_cpu, out_gpu, tol):
    for b in range(x_cpu.shape[0]):
        ref = oracle.rope(f64(x_cpu[b]), wl.grid, wl.pairs, wl.offsets[b], wl.theta)
        err = attention_err(f64(out_gpu[b]), ref)
        assert err <= tol, err


@pytest.mark.parametrize("name,heads", ROPE_CASES)
def test_rope_matches_oracle(name, heads):
    wl = synth.WORKLOADS[name]
    H = heads or wl.heads_q
    note(f"rope {name} H={H}")
    x = synth.random_tensor((wl.branches, wl.seq, H, wl.head_dim), 21, wl.torch_dtype)
    d = x.to(DEV)
    nx.nxattn_rope_apply(d, [nx.rope_desc(wl.grid, wl.pairs, wl.offsets[b]) for b in range(wl.branches)])
    torch.cuda.synchronize()
    # bf16: one rounding of the exact value (2^-9 relative) plus fp32 arithmetic
    rope_check(wl, x, d.cpu(), 2.0 ** -8 if wl.dtype == "bf16" else 2e-6)


def test_rope_strided_interleaved_and_per_branch_offsets():
    note("rope strided / interleaved")
    base = synth.random_tensor((2, 48, 6, 64), 22, torch.float32)
    d = base.to(DEV)
    view = d[:, :, 1:5, :]                       # strided heads
    descs = [nx.rope_desc((6, 8), (16, 16), (3, 5), interleaved=True),
             nx.rope_desc((6, 8), (16, 16), (100, 7), interleaved=True)]
    nx.nxattn_rope_apply(view, descs)
    torch.cuda.synchronize()
    out = d.cpu()
    assert torch.equal(out[:, :, 0], base[:, :, 0]) and torch.equal(out[:, :, 5], base[:, :, 5])
    for b, off in enumerate(((3, 5), (100, 7))):
        ref = oracle.rope(f64(base[b, :, 1:5]), (6, 8), (16, 16), off, interleaved=True)
        assert np.max(np.abs(f64(out[b, :, 1:5]) - ref)) <= 2e-6 * max(1.0, np.max(np.abs(ref)))


def test_rope_most_branches():
    # eight descriptors (the most a call takes), each with its own offsets and pair split
    note("rope, 8 branches")
    grid, D = (5, 7), 128
    S = int(np.prod(grid))
    x = synth.random_tensor((8, S, 3, D), 24, torch.bfloat16)
    d = x.to(DEV)
    splits = [(32, 32), (16, 48), (48, 16), (1, 63), (63, 1), (32, 32), (20, 44), (40, 24)]
    offs = [(0, 0), (1, 2), (512, 512), (7, 0), (0, 9), (1000, 3), (65, 66), (2 ** 20, 5)]
    nx.nxattn_rope_apply(d, [nx.rope_desc(grid, splits[b], offs[b]) for b in range(8)])
    torch.cuda.synchronize()
    out = d.cpu()
    for b in range(8):
        ref = oracle.rope(f64(x[b]), grid, splits[b], offs[b])
        err = float(np.max(np.abs(f64(out[b]) - ref) / np.maximum(1.0, np.abs(ref))))
        assert err <= 2.0 ** -8, (b, err)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_global_frequency_ladder(dtype):
    # one theta ladder over all pairs, the sections choose the axis (3-D MRoPE)
    note(f"rope global ladder {dtype}")
    grid, pairs, D = (4, 6, 10), (22, 21, 21), 128
    S = int(np.prod(grid))
    x = synth.random_tensor((2, S, 3, D), 23, dtype)
    d = x.to(DEV)
    offs = ((0, 0, 0), (12, 12, 12))
    nx.nxattn_rope_apply(d, [nx.rope_desc(grid, pairs, offs[b], global_freq=True) for b in range(2)])
    torch.cuda.synchronize()
    out = d.cpu()
    tol = 2.0 ** -8 if dtype == torch.bfloat16 else 2e-6
    for b in range(2):
        ref = oracle.rope(f64(x[b]), grid, pairs, offs[b], global_freq=True)
        assert np.max(np.abs(f64(out[b]) - ref) / np.maximum(1.0, np.abs(ref))) <= tol


def test_rope_integer_positions_exact():
    # pairs (1, 0): the result is (cos phi, sin phi); the GPU must match the oracle at the
    # expected integer position, not at +-1 (u = 0 has a 1-radian step per position)
    note("rope integer positions")
    wl = synth.WORKLOADS["video_bf16"]
    S, D = wl.seq, wl.head_dim
    x = torch.zeros((1, S, 1, D), dtype=torch.float32)
    x[..., : D // 2] = 1.0
    d = x.to(DEV)
    nx.nxattn_rope_apply(d, [nx.rope_desc(wl.grid, wl.pairs, (5, 7, 11))])
    torch.cuda.synchronize()
    got = f64(d.cpu()[0, :, 0])
    pos = oracle.positions(wl.grid, (5, 7, 11))
    j0 = [0, wl.pairs[0], wl.pairs[0] + wl.pairs[1]]     # u = 0 pair of each axis
    for ax in range(3):
        for delta in (-1, 1):
            wrong = np.cos(pos[:, ax] + delta)
            right = np.cos(pos[:, ax])
            g = got[:, j0[ax]]
            assert np.all(np.abs(g - right) < 1e-5)
            assert np.all(np.abs(g - right) < np.abs(g - wrong) + 1e-12)


# ---------------------------------------------------------------------------- cfg
@pytest.mark.parametrize("n,dtype", [(4096 * 32 * 128, torch.bfloat16), (1000003, torch.bfloat16),
                                     (77, torch.float32), (3900 * 16 * 72, torch.float32)])
def test_cfg_matches_oracle(n, dtype):
    note(f"cfg n={n} {dtype}")
    c = synth.random_tensor((n,), 31, dtype)
    u = synth.random_tensor((n,), 32, dtype)
    dc, du = c.to(DEV), u.to(DEV)
    out = torch.empty_like(dc)
    for s in (4.0, 6.0):
        nx.nxattn_cfg_combine(dc, du, out, s)
        torch.cuda.synchronize()
        ref = oracle.cfg_combine(f64(c), f64(u), s)
        got = f64(out.cpu())
        # fp32 fma of exact-widened inputs, then one rounding to the output type
        rel = 2.0 ** -8 if dtype == torch.bfloat16 else 2e-6
        assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-6 * (np.abs(f64(c)) + np.abs(f64(u))) * (1 + s))
    nx.nxattn_cfg_combine(dc, du, out, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), u)                      # s = 0 gives uncond bitwise
    alias = dc.clone()
    nx.nxattn_cfg_combine(alias, du, alias, 4.0)          # out aliases cond
    nx.nxattn_cfg_combine(dc, du, out, 4.0)
    torch.cuda.synchronize()
    assert torch.equal(alias, out)


# ---------------------------------------------------------------------------- attention
def run_fwd(q, k, v, prefix, scale=0.0):
    o = torch.empty_like(q)
    nx.nxattn_fwd(q, k, v, o, prefix, scale)
    torch.cuda.synchronize()
    return o.cpu()


def fwd_case(dtype, B, S, Hq, Hkv, D, plens, seed, scale_v=1.0):
    note(f"fwd {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} P={plens} seed={seed}")
    q = synth.random_tensor((B, S, Hq, D), seed, dtype, scale_v)
    k = synth.random_tensor((B, S, Hkv, D), seed + 1, dtype, scale_v)
    v = synth.random_tensor((B, S, Hkv, D), seed + 2, dtype, scale_v)
    pre = [synth.random_tensor((2, p, Hkv, D), seed + 3 + b, dtype, scale_v) if p else None
           for b, p in enumerate(plens)]
    o = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), [p.to(DEV) if p is not None else None for p in pre])
    tol = TOL["bf16" if dtype == torch.bfloat16 else "f32"]
    for b in range(B):
        ref = oracle.attention(f64(q[b]), f64(k[b]), f64(v[b]),
                               f64(pre[b][0]) if pre[b] is not None else None,
                               f64(pre[b][1]) if pre[b] is not None else None)
        err = attention_err(f64(o[b]), ref)
        assert err <= tol, (b, err)
    return o


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (1, 300, 8, 2, (37,)),        # ragged Sq, prefix straddling a key tile, G = 4
    (2, 129, 4, 4, (64, 0)),      # G = 1, one branch without prefix
    (2, 65, 6, 2, (1, 130)),      # G = 3: query blocks cross heads inside a workgroup
    (1, 1, 8, 1, (0,)),           # a single query and a single key
    (1, 1, 16, 2, (200,)),        # one own token, long prefix
    (1, 33, 16, 2, (31,)),        # G = 8
    (3, 70, 2, 1, (5, 0, 64)),
    (2, 640, 8, 2, (128, 200)),   # whole prefix tiles, then a straddling one (processed last)
    (2, 200, 4, 2, (300, 7)),     # prefix longer than the own tokens; ragged last tile
    (8, 97, 4, 2, (0, 1, 31, 64, 65, 127, 200, 3)),   # the most branches a call takes
])
def test_fwd_bf16_reduced(B, S, Hq, Hkv, P):
    fwd_case(torch.bfloat16, B, S, Hq, Hkv, 128, P, 1000 + S)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,P", [
    (1, 64, 2, 2, 64, (32,)),
    (1, 300, 4, 2, 72, (0,)),
    (2, 97, 3, 3, 72, (13, 64)),
    (1, 1, 2, 1, 64, (0,)),
    (1, 5, 4, 4, 72, (70,)),
    (8, 40, 2, 1, 72, (0, 5, 16, 17, 33, 64, 100, 2)),  # the most branches a call takes
])
def test_fwd_f32_reduced(B, S, Hq, Hkv, D, P):
    fwd_case(torch.float32, B, S, Hq, Hkv, D, P, 2000 + S)


def test_fwd_single_key_returns_v():
    # Skv = 1: the only weight is 1, so o = v (bf16: exactly after rounding; fp32: the
    # normalisation p / l may move the last bit)
    for dtype, D in ((torch.bfloat16, 128), (torch.float32, 72)):
        note(f"fwd single key {dtype}")
        q = synth.random_tensor((2, 1, 4, D), 41, dtype)
        k = synth.random_tensor((2, 1, 2, D), 42, dtype)
        v = synth.random_tensor((2, 1, 2, D), 43, dtype)
        o = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), [])
        exp = v.repeat_interleave(2, dim=2)
        if dtype == torch.bfloat16:
            assert torch.equal(o, exp)
        else:
            assert torch.allclose(o, exp, rtol=4e-7, atol=0)


def test_fwd_constant_v_and_zero_q():
    note("fwd constant V / zero q")
    D, S, P = 128, 150, 70
    row = synth.random_tensor((D,), 44, torch.bfloat16)
    v = row.expand(1, S, 2, D).contiguous()
    pre = torch.stack([synth.random_tensor((P, 2, D), 45, torch.bfloat16), row.expand(P, 2, D)], 0).contiguous()
    q = synth.random_tensor((1, S, 4, D), 46, torch.bfloat16)
    k = synth.random_tensor((1, S, 2, D), 47, torch.bfloat16)
    o = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), [pre.to(DEV)])
    # the weights sum to one: the output is that row, up to the bf16 rounding of P and O
    assert np.max(np.abs(f64(o) - f64(row))) <= 2.0 ** -7 * np.max(np.abs(f64(row)))
    oz = run_fwd(torch.zeros_like(q).to(DEV), k.to(DEV), synth.random_tensor((1, S, 2, D), 48, torch.bfloat16).to(DEV),
                 [pre.to(DEV)])
    assert np.all(np.isfinite(f64(oz)))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 72), (torch.float32, 64)])
def test_fwd_bit_exact_selection(dtype, D):
    """Each query selects exactly one key (others underflow to weight 0); V rows encode
    (key mod 256, key // 256, branch, kv head) so the output must decode bit for bit to
    the expected key of the expected branch and kv head: pins prefix ++ own, the GQA
    mapping and the branch indexing, in both attention kernels."""
    B, S, Hq, Hkv = 2, 200, 8, 2
    plens = (70, 135)
    rng = np.random.default_rng(7)
    cast = bf if dtype == torch.bfloat16 else (lambda x: x)
    for _ in (0,):
        note(f"fwd bit-exact selection {dtype} D={D}")
        q = torch.zeros((B, S, Hq, D))
        k = torch.zeros((B, S, Hkv, D))
        v = torch.full((B, S, Hkv, D), 0.5)          # non-selected rows: must get weight 0
        pre = [torch.stack([torch.zeros((p, Hkv, D)), torch.full((p, Hkv, D), 0.5)], 0) for p in plens]
        expect = np.zeros((B, S, Hq), dtype=np.int64)
        for b in range(B):
            Skv = plens[b] + S
            for g in range(Hkv):
                # active keys: tile edges, the prefix/own boundary, the tail, random others
                cand = {0, 63, 64, 65, plens[b] - 1, plens[b], Skv - 1, Skv - 2, 127, 128}
                cand.update(int(x) for x in rng.choice(Skv, 60, replace=False))
                active = sorted(c for c in cand if 0 <= c < Skv)[:D]
                for dim, j in enumerate(active):
                    kv_k = torch.zeros(D)
                    kv_k[dim] = 48.0
                    code = torch.zeros(D)
                    code[0], code[1], code[2], code[3] = j % 256, j // 256, b, g
                    if j < plens[b]:
                        pre[b][0, j, g] = kv_k
                        pre[b][1, j, g] = code
                    else:
                        k[b, j - plens[b], g] = kv_k
                        v[b, j - plens[b], g] = code
                for hl in range(Hq // Hkv):
                    h = g * (Hq // Hkv) + hl
                    pick = rng.integers(0, len(active), S)
                    for i in range(S):
                        q[b, i, h, pick[i]] = 48.0
                        expect[b, i, h] = active[pick[i]]
        o = run_fwd(cast(q).to(DEV), cast(k).to(DEV), cast(v).to(DEV), [cast(p).to(DEV) for p in pre])
        got = f64(o)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                exp_rows = np.stack([expect[b, :, h] % 256, expect[b, :, h] // 256,
                                     np.full(S, b), np.full(S, g)], 1).astype(np.float64)
                dec = got[b, :, h, :4]
                if dtype == torch.float32:
                    # the single weight is exp(0) = 1 up to the rounding of the fp32 score
                    # arithmetic, and o = (p v) / l with l = p can move v's last bits: the
                    # code is decoded by rounding, after checking it sits within 4 ulp of an
                    # integer
                    assert np.all(np.abs(dec - np.round(dec)) <= 4 * 2.0 ** -23 * np.abs(dec)), (b, h)
                    dec = np.round(dec)
                bad = np.nonzero(np.any(dec != exp_rows, axis=1))[0]
                assert bad.size == 0, (b, h, [(int(i), dec[i].tolist(), exp_rows[i].tolist()) for i in bad[:8]])


@pytest.mark.parametrize("dtype,D,splits", [(torch.bfloat16, 128, 0), (torch.float32, 72, 0),
                                             (torch.bfloat16, 128, 4), (torch.float32, 64, 3)])
def test_fwd_deterministic(dtype, D, splits):
    # the same call twice gives the same bits: one pass, and key ranges plus the merge (a
    # long prefix against few queries, so that the planner does split)
    S, P = (257, 99) if splits == 0 else (64, 3000)
    note(f"fwd determinism {dtype} D={D} splits={splits}")
    q = synth.random_tensor((2, S, 8, D), 51, dtype).to(DEV)
    k = synth.random_tensor((2, S, 2, D), 52, dtype).to(DEV)
    v = synth.random_tensor((2, S, 2, D), 53, dtype).to(DEV)
    pre = [synth.random_tensor((2, P, 2, D), 54, dtype).to(DEV), None]
    lse = [torch.empty((2, 8, S), dtype=torch.float32, device=DEV) for _ in range(2)]
    outs = []
    for i in range(2):
        o = torch.empty_like(q)
        nx.nxattn_fwd(q, k, v, o, pre, lse=lse[i], num_splits=splits)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(lse[0].cpu(), lse[1].cpu())


def test_fwd_key_permutation_invariance():
    note("fwd key permutation")
    S, P, D = 190, 66, 128
    q = synth.random_tensor((1, S, 4, D), 61, torch.bfloat16)
    k = synth.random_tensor((1, S, 1, D), 62, torch.bfloat16)
    v = synth.random_tensor((1, S, 1, D), 63, torch.bfloat16)
    pre = synth.random_tensor((2, P, 1, D), 64, torch.bfloat16)
    K = torch.cat([pre[0], k[0]], 0)
    V = torch.cat([pre[1], v[0]], 0)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(S + P))
    K2, V2 = K[perm], V[perm]
    o1 = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), [pre.to(DEV)])
    o2 = run_fwd(q.to(DEV), K2[P:][None].contiguous().to(DEV), V2[P:][None].contiguous().to(DEV),
                 [torch.stack([K2[:P], V2[:P]], 0).contiguous().to(DEV)])
    assert attention_err(f64(o1[0]), f64(o2[0])) <= TOL["bf16"]


def test_fwd_strided_views():
    note("fwd strided q/k/v/o views")
    D = 128
    qkv = synth.random_tensor((2, 100, 8 + 2 + 2, D), 71, torch.bfloat16).to(DEV)   # fused projection
    q, k, v = qkv[:, :, :8], qkv[:, :, 8:10], qkv[:, :, 10:12]
    obuf = torch.zeros((2, 100, 9, D), dtype=torch.bfloat16, device=DEV)
    o = obuf[:, :, 1:9]
    nx.nxattn_fwd(q, k, v, o, [])
    torch.cuda.synchronize()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for b in range(2):
        ref = oracle.attention(f64(qc[b]), f64(kc[b]), f64(vc[b]))
        assert attention_err(f64(o.cpu()[b]), ref) <= TOL["bf16"]
    assert torch.count_nonzero(obuf[:, :, 0]) == 0


def test_fwd_strided_own_keys_with_prefix():
    # own q/k/v are views of a fused projection (k row stride (Hq + 2 Hkv) D), the prefix
    # is a contiguous [2, P, Hkv, D] slice (row stride Hkv D): whole own tiles and whole
    # prefix tiles are loaded with different row strides; P = 130 straddles a tile
    note("fwd strided own keys + prefix of another stride")
    D, S, Hq, Hkv, P = 128, 600, 8, 2, 130
    qkv = synth.random_tensor((1, S, Hq + 2 * Hkv, D), 81, torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    pre = synth.random_tensor((2, P, Hkv, D), 82, torch.bfloat16)
    o = run_fwd(q, k, v, [pre.to(DEV)])
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ref = oracle.attention(f64(qc[0]), f64(kc[0]), f64(vc[0]), f64(pre[0]), f64(pre[1]))
    assert attention_err(f64(o[0]), ref) <= TOL["bf16"]


@pytest.mark.parametrize("grid,pairs,offsets,P,inter,gf", [
    ((12, 20), (32, 32), ((7, 3), (512, 512)), (70, 0), False, False),      # 2-D, ragged, two branches
    ((240,), (64,), ((32,), (0,)), (0, 33), True, False),                    # 1-D interleaved
    ((3, 5, 8), (22, 21, 21), ((0, 0, 0), (5, 6, 7)), (16, 64), False, False),  # 3-D sections
    ((3, 5, 8), (16, 24, 24), ((2, 0, 0), (9, 9, 9)), (0, 40), False, True),    # 3-D, one global ladder
])
def test_fwd_q_rope_on_load(grid, pairs, offsets, P, inter, gf):
    # q rotated inside the kernel == oracle RoPE of q, then attention (k pre-rotated by
    # the oracle and rounded to bf16); q itself stays unchanged
    S, Hq, Hkv, D = int(np.prod(grid)), 8, 2, 128
    note(f"fwd q_rope grid={grid} pairs={pairs} offsets={offsets} P={P} interleaved={inter}")
    q = synth.random_tensor((2, S, Hq, D), 91, torch.bfloat16)
    k = synth.random_tensor((2, S, Hkv, D), 92, torch.bfloat16)
    v = synth.random_tensor((2, S, Hkv, D), 93, torch.bfloat16)
    pre = [synth.random_tensor((2, p, Hkv, D), 94 + b, torch.bfloat16) if p else None for b, p in enumerate(P)]
    rnd = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    k_rot = torch.stack([rnd(oracle.rope(f64(k[b]), grid, pairs, offsets[b], 10000.0, interleaved=inter,
                                         global_freq=gf)) for b in range(2)])
    descs = [nx.rope_desc(grid, pairs, offsets[b], 10000.0, inter, gf) for b in range(2)]
    qd = q.to(DEV)
    o = torch.empty_like(qd)
    nx.nxattn_fwd(qd, k_rot.to(DEV), v.to(DEV), o, [p.to(DEV) if p is not None else None for p in pre],
                  q_rope=descs)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q)
    for b in range(2):
        q_ex = oracle.rope(f64(q[b]), grid, pairs, offsets[b], 10000.0, interleaved=inter, global_freq=gf)
        pk = f64(pre[b][0]) if pre[b] is not None else None
        pv = f64(pre[b][1]) if pre[b] is not None else None
        ref = oracle.attention(q_ex, f64(k_rot[b]), f64(v[b]), pk, pv)
        err = attention_err(f64(o.cpu()[b]), ref)
        note(f"  branch {b}: error {err:.3e} against the exact oracle (gate {TOL['bf16']:.0e})")
        assert err <= TOL["bf16"], (b, err)


@pytest.mark.parametrize("k_mult", [6.0, 60.0])
def test_fwd_q_rope_score_jumps(k_mult):
    # q rotated on load (the folded softmax, which tries the weights against the running max
    # before computing a tile max): one tile of ordinary prefix keys sets m, then the own
    # keys, scaled up, raise the scores far above it. x6: jumps of tens in log2 units (a
    # tile's weight sum exceeds 2^8, the full update rescales); x60: jumps beyond 128
    # (the first try overflows to inf). Both must match the oracle like ordinary data.
    # Scores 6x and 60x the usual scale make the output that much more sensitive to the one
    # bf16 rounding of the rotated q that any bf16 pipeline takes (at 60x a rounding moves a
    # score by about 0.1 nat), so the gate holds against the oracle's attention of q as the
    # kernel rounds it (the rotation times scale*log2(e), rounded once to bf16); the error
    # against the unrounded q is printed too.
    grid, pairs, S, Hq, Hkv, D = (8, 12), (32, 32), 96, 8, 2, 128
    note(f"fwd q_rope score jumps, own k x{k_mult}")
    q = synth.random_tensor((2, S, Hq, D), 95, torch.bfloat16)
    k = (synth.random_tensor((2, S, Hkv, D), 96, torch.float32) * k_mult).to(torch.bfloat16)
    v = synth.random_tensor((2, S, Hkv, D), 97, torch.bfloat16)
    pre = [synth.random_tensor((2, 64, Hkv, D), 98 + b, torch.bfloat16) for b in range(2)]
    offsets = ((3, 5), (11, 2))
    rnd = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    k_rot = torch.stack([rnd(oracle.rope(f64(k[b]), grid, pairs, offsets[b], 10000.0)) for b in range(2)])
    descs = [nx.rope_desc(grid, pairs, offsets[b]) for b in range(2)]
    o = torch.empty((2, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd(q.to(DEV), k_rot.to(DEV), v.to(DEV), o, [p.to(DEV) for p in pre], q_rope=descs)
    torch.cuda.synchronize()
    got = f64(o.cpu())
    assert np.all(np.isfinite(got))
    for b in range(2):
        q_ex = oracle.rope(f64(q[b]), grid, pairs, offsets[b], 10000.0)
        pk, pv = f64(pre[b][0]), f64(pre[b][1])
        ref = oracle.attention(fused_q(q_ex, D), f64(k_rot[b]), f64(v[b]), pk, pv)
        err = attention_err(got[b], ref)
        e_ex = attention_err(got[b], oracle.attention(q_ex, f64(k_rot[b]), f64(v[b]), pk, pv))
        note(f"  branch {b}: error {err:.3e} against the oracle with q rounded as the kernel rounds it "
             f"(gate {TOL['bf16']:.0e}); {e_ex:.3e} against the unrounded q")
        assert err <= TOL["bf16"], (b, err)


@pytest.mark.parametrize("grid,pairs,offsets", [
    ((8, 8), (32, 32), ((1024, 1024), (16384, 16384))),          # the 2K DiT offset, a long-prefix offset
    ((4, 4, 4), (22, 21, 21), ((100000, 3, 77), (2 ** 24 - 4, 2 ** 24 - 4, 2 ** 24 - 4))),  # up to the limit
])
def test_fwd_q_rope_readout_at_large_positions(grid, pairs, offsets):
    """The rotated q that the kernel multiplies, read out exactly: with the prefix as the
    only keys and a single key e_d per kv head, the log-sum-exp is that query's score,
    ln2 * q~_d, where q~ = bf16(scale * log2(e) * rope(q)) is the kernel's folded rotation.
    Against the oracle's fp64 rotation (times the same factor, rounded to bf16): at most
    one bf16 ulp apart, and only where the exact value sits within the fp32 arithmetic's
    error of a rounding boundary (an angle error of 1e-4 rad would move a few percent of
    the values)."""
    D, Hq, B = 128, 16, 2
    S = int(np.prod(grid))
    note(f"fwd q_rope readout grid={grid} offsets={offsets}")
    q = synth.random_tensor((B, S, Hq, D), 4800, torch.bfloat16)
    qd = q.to(DEV)
    descs = [nx.rope_desc(grid, pairs, offsets[b]) for b in range(B)]
    cf = fold_factor(D)
    got = np.zeros((B, S, Hq, D))
    v = torch.ones((1, Hq, D), dtype=torch.bfloat16)
    o = torch.empty_like(qd)
    read = np.zeros((Hq, D), dtype=bool)
    for t in range(32):
        # kv head h holds the single key e_d: head h reads dims 8h .. 8h + 31 (mod 128)
        k = torch.zeros((1, Hq, D), dtype=torch.bfloat16)
        dims = [(8 * h + t) % D for h in range(Hq)]
        for h, d in enumerate(dims):
            k[0, h, d] = 1.0
        pre = torch.stack([k, v], 0).contiguous().to(DEV)        # [2, 1, Hkv, D]
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        nx.nxattn_fwd(qd, None, None, o, [pre, pre], q_rope=descs, lse=lse, prefix_only=True)
        torch.cuda.synchronize()
        val = lse.cpu().numpy().astype(np.float64) / np.log(2.0)        # [B, Hq, S]
        for h, d in enumerate(dims):
            got[:, :, h, d] = val[:, h, :]
            read[h, d] = True
    # the readout is a bf16 value up to the fp32 products of the log-sum-exp
    gb = torch.from_numpy(got).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.all(np.abs(gb - got) <= 2.0 ** -20 * np.abs(got) + 1e-30)
    ex = np.stack([oracle.rope(f64(q[b]), grid, pairs, offsets[b]) for b in range(B)]) * cf
    rb = torch.from_numpy(ex).to(torch.bfloat16).to(torch.float64).numpy()
    # magnitude of the rotary pair each element belongs to (half-split pairs j, j + 64)
    qa = f64(q)
    pair = np.sqrt(qa ** 2 + np.roll(qa, D // 2, axis=-1) ** 2) * cf
    hd = np.argwhere(read)
    gb, rb, pair = gb[:, :, read], rb[:, :, read], pair[:, :, read]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rb), 1e-30))) - 7)
    miss = gb != rb
    # one bf16 ulp of the result, plus 2^-13 of the pair's magnitude: the fp32 rotation's
    # own rounding where the result cancels (an angle error of 1e-3 rad would exceed it)
    tol = ulp * 1.0001 + 2.0 ** -13 * pair
    rel = np.abs(gb - rb) / tol
    w = np.unravel_index(int(np.argmax(rel)), rel.shape)
    pos = oracle.positions(grid, offsets[w[0]])[w[1]]
    note(f"  values off the rounded exact rotation: {int(miss.sum())} of {miss.size}; worst error "
         f"{float(rel[w]):.3f} of its bound at branch {w[0]} token {w[1]} (positions {pos.tolist()}) head, dim "
         f"{hd[w[2]].tolist()}: {float(gb[w]):.6g} against {float(rb[w]):.6g} (pair {float(pair[w]):.4g})")
    assert np.all(np.abs(gb - rb) <= tol)
    assert miss.mean() <= 2e-3


# ---------------------------------------------------------------------------- whole workloads
def step_case(name, rows_per_branch, seed_rows):
    """The whole step (relayout, RoPE, fused attention, CFG) on sampled rows of a full-size
    workload. Every branch is held to the plain gate against the exact oracle (the
    oracle's own RoPE in fp64, nothing rounded); a second check isolates the fused kernel
    (the oracle's attention over the rotated q and k the kernel actually used). The
    errors are printed for the record."""
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else synth.bench_workload(name.split("+")[0])
    note(f"step {name} (sampled rows {rows_per_branch})")
    inp = synth.make_inputs(wl)
    step = AttentionStep(wl, inp)
    out = step()
    torch.cuda.synchronize()
    o_gpu = step.o.cpu()
    rows = {b: sample_rows(wl.seq, rows_per_branch, seed_rows + b) for b in range(wl.branches)}
    ref = oracle_attention(wl, inp, rows)
    tol = TOL[wl.dtype]
    qg, kg = step.q.cpu(), step.k.cpu()
    # isolation reference: oracle attention over the GPU's own rotated k and, for q rotated
    # on load inside the kernel, the oracle's rotation rounded where the kernel rounds it
    if step.fuse_q_rope:
        q_r = [fused_q(oracle_rope(wl, inp.q, b, rows[b]), wl.head_dim) for b in range(wl.branches)]
        ref_iso = oracle_attention(wl, inp, rows, q_r, [f64(kg[b]) for b in range(wl.branches)],
                                   q_rot_rows_only=True)
    else:
        ref_iso = oracle_attention(wl, inp, rows, [f64(qg[b]) for b in range(wl.branches)],
                                   [f64(kg[b]) for b in range(wl.branches)])
    errs = []
    for b in range(wl.branches):
        g = f64(o_gpu[b][rows[b]])
        e = attention_err(g, ref[b])
        e_iso = attention_err(g, ref_iso[b])
        note(f"  branch {b}: error {e:.3e} against the exact oracle, {e_iso:.3e} against the isolated kernel "
             f"reference (gate {tol:.0e}); global max-rel {global_maxrel(g, ref[b]):.3e}, "
             f"cosine {cosine(g, ref[b]):.9f}")
        errs.append((b, e, e_iso))
    for b, e, e_iso in errs:
        assert e_iso <= tol, (b, e_iso)
        assert e <= tol, (b, e)
    if step.use_cfg:
        r = rows[0]
        both = sorted(set(rows[0]).intersection(rows[1]))
        i0, i1 = np.searchsorted(r, both), np.searchsorted(rows[1], both)
        got = f64(out.cpu()[both])
        # the combine itself: one fp32 fma of the GPU's own branch outputs, rounded once
        own = oracle.cfg_combine(f64(o_gpu[0][both]), f64(o_gpu[1][both]), wl.guidance)
        e_own = attention_err(got, own)
        # end to end: u + s (c - u) carries (1 + s) e_c + s e_u of the branch errors, at most
        # (1 + 2s) times the branch gate
        c = oracle.cfg_combine(ref[0][i0], ref[1][i1], wl.guidance)
        e_cfg = attention_err(got, c)
        note(f"  cfg (s = {wl.guidance}): error {e_cfg:.3e} against the exact oracle (gate "
             f"{tol * (1 + 2 * wl.guidance):.2e}), {e_own:.3e} against the combine of the GPU branches")
        # one bf16 rounding (< 2^-8 relative) after the fp32 fma, or the fp32 fma alone
        assert e_own <= (2.0 ** -8 + 2.0 ** -16 if wl.dtype == "bf16" else 1e-6)
        assert e_cfg <= tol * (1 + 2 * wl.guidance)
    return wl


def test_step_tiny_f32_full():
    step_case("tiny_f32", 64, 1)


def test_step_vit_f32_one_layer_sampled():
    step_case("vit_f32", 300, 2)


def test_step_vit_f32_all_layers_sampled():
    # the 27-layer encoder as the benchmark steps it: every layer on its own seeded inputs
    # (one AttentionStep per layer, all resident), sampled rows of each layer against the
    # oracle at the fp32 gate
    wl = synth.WORKLOADS["vit_f32"]
    note(f"step vit_f32, {wl.layers} layers (sampled rows)")
    inps = [synth.make_inputs(wl, layer=l) for l in range(wl.layers)]
    steps = [AttentionStep(wl, inp) for inp in inps]
    for st in steps:
        st()
    torch.cuda.synchronize()
    worst = 0.0
    for l, (inp, st) in enumerate(zip(inps, steps)):
        rows = {0: sample_rows(wl.seq, 40, 900 + l)}
        ref = oracle_attention(wl, inp, rows)[0]
        e = attention_err(f64(st.o.cpu()[0][rows[0]]), ref)
        worst = max(worst, e)
        assert e <= TOL["f32"], (l, e)
    note(f"  worst layer error {worst:.3e} (gate {TOL['f32']:.0e})")


def test_step_dit1k_bf16_sampled():
    step_case("dit1k_bf16", 96, 3)


@pytest.mark.parametrize("name,q_on_load", [("dit1k_fp8qk+replay", False), ("dit2k_fp8qk", False),
                                             ("dit1k_fp8blk+replay", False), ("dit2k_fp8blk", False),
                                             ("dit1k_fp8blk+replay", True)])
def test_step_fp8qk_sampled(name, q_on_load):
    """The bench configuration of the fp8 score GEMM at full size, with one scale per
    (branch, head) (fp8qk) or per run of 32 head_dim elements (fp8blk; with q_on_load the
    attention kernel rotates, folds and quantizes q itself as it loads it, so q has no
    stored codes).

    1. Isolation: the codes of the step's k (and, fp8qk, q) as nxattn_rope_apply rotates
       them (q times the softmax fold factor), and of each prefix K, bit for bit against
       the oracle's quantization; sampled rows of the attention against the oracle's
       attention of those dequantized codes (fp8blk: with the chain's q below).
    2. The oracle chain alone: the oracle's fp64 RoPE, rounded to bf16 where the path
       stores a rotation (k; q of fp8qk), q times the fold factor, the oracle's
       quantization; the GPU attention against the oracle's attention of that chain's
       dequantized codes, at the bf16 gate. Codes that differ from the chain's (a rounding
       that falls the other way) are counted and printed.
    3. The recipe's own error, printed and not gated: the GPU attention against the
       exact oracle attention of the unquantized inputs.
    """
    from oracle import fp8 as ofp8
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else synth.bench_workload(name.split("+")[0])
    note(f"step {name} (fp8 score GEMM{', q quantized on load' if q_on_load else ''}, sampled rows)")
    inp = synth.make_inputs(wl)
    step = AttentionStep(wl, inp, q_on_load=q_on_load)
    step()
    torch.cuda.synchronize()
    # the step rotates inside the quantizer (and the attention kernel) and leaves q and k as given
    assert torch.equal(step.q.cpu().view(torch.int16), inp.q.view(torch.int16))
    assert torch.equal(step.k.cpu().view(torch.int16), inp.k.view(torch.int16))
    assert step.fold_q
    cf = fold_factor(wl.head_dim)
    qload = step.q_on_load
    if qload:
        quant, deq = ofp8.quantize_fp8_blocks, ofp8.dequantize_fp8_blocks
        k8, ke = (t.cpu().numpy() for t in (step.k8, step.ks))
    elif wl.fp8_blocks:
        quant, deq = ofp8.quantize_fp8_blocks, ofp8.dequantize_fp8_blocks
        q8, qe, k8, ke = (t.cpu().numpy() for t in (step.q8, step.qs, step.k8, step.ks))
    else:
        quant, deq = ofp8.quantize_fp8, ofp8.dequantize_fp8
        q8, qe, k8, ke = (t.cpu().numpy() for t in (step.q8, step.qe, step.k8, step.ke))
    o = step.o.cpu()
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    # 2. the oracle chain (q first: fp8blk's isolated reference takes the chain's q)
    if qload:
        q_chain = np.stack([oracle_rope(wl, inp.q, b) for b in range(wl.branches)]) * float(cf)
        cq, cqe = quant(q_chain)
    else:
        q_chain = torch.stack([bf(oracle_rope(wl, inp.q, b)) for b in range(wl.branches)])
        cq, cqe = quant(f64(q_chain.float() * torch.tensor(cf, dtype=torch.float32)))
    del q_chain
    dq_ch = deq(cq, cqe) / cf
    k_chain = torch.stack([bf(oracle_rope(wl, inp.k, b)) for b in range(wl.branches)])
    ck, cke = quant(f64(k_chain))
    del k_chain
    dk_ch = deq(ck, cke)
    # 1. isolation
    kr = step.k.clone()
    nx.nxattn_rope_apply(kr, step.descs)
    torch.cuda.synchronize()
    rk, rke = quant(f64(kr.cpu()))
    del kr
    assert np.array_equal(k8, rk) and np.array_equal(ke, rke)
    dk_iso = deq(rk, rke)
    if qload:
        dq_iso = dq_ch
        msg_q = "q formed in the kernel"
    else:
        qr = step.q.clone()
        nx.nxattn_rope_apply(qr, step.descs)
        torch.cuda.synchronize()
        rq, rqe = quant(f64(qr.cpu().float() * torch.tensor(cf, dtype=torch.float32)))
        del qr
        assert np.array_equal(q8, rq) and np.array_equal(qe, rqe)
        dq_iso = deq(rq, rqe) / cf
        msg_q = (f"q {int(np.count_nonzero(q8 != cq))} of {q8.size} (exponents "
                 f"{int(np.count_nonzero(qe != cqe))})")
        del rq
    note(f"  codes that differ from the oracle chain's: {msg_q}, k {int(np.count_nonzero(k8 != ck))} of {k8.size} "
         f"(exponents {int(np.count_nonzero(ke != cke))})")
    del cq, ck, rk
    for b in range(wl.branches):
        pre = step.prefix_online[b]
        dpk = pv = pk_ex = None
        if pre is not None:
            pc, pe = quant(f64(pre[0].cpu())[None])
            got_e = step.pks[b].cpu().numpy() if wl.fp8_blocks else step.pke[b].cpu().numpy()
            assert np.array_equal(step.pk8[b].cpu().numpy(), pc)
            assert np.array_equal(got_e, pe if wl.fp8_blocks else pe[0])
            dpk, pv, pk_ex = deq(pc, pe)[0], f64(pre[1].cpu()), f64(pre[0].cpu())
        rows = sample_rows(wl.seq, 48, 700 + b)
        ar = np.arange(len(rows))
        g = f64(o[b][torch.from_numpy(rows)])
        vb = f64(inp.v[b])
        e_iso = attention_err(g, oracle.attention(dq_iso[b][rows], dk_iso[b], vb, dpk, pv, rows=ar))
        e_ch = attention_err(g, oracle.attention(dq_ch[b][rows], dk_ch[b], vb, dpk, pv, rows=ar))
        ex = oracle.attention(oracle_rope(wl, inp.q, b, rows), oracle_rope(wl, inp.k, b), vb, pk_ex, pv, rows=ar)
        e_ex = attention_err(g, ex)
        note(f"  branch {b}: error {e_ch:.3e} against the oracle chain, {e_iso:.3e} against the isolated "
             f"reference (gate {TOL['bf16']:.0e}); the recipe against unquantized attention (not gated): "
             f"{e_ex:.3e}, global max-rel {global_maxrel(g, ex):.3e}, cosine {cosine(g, ex):.9f}")
        assert e_iso <= TOL["bf16"], (b, e_iso)
        assert e_ch <= TOL["bf16"], (b, e_ch)


def test_step_longctx_split_keys_sampled():
    # a short query against a long prefix, keys split into ranges and merged, in the
    # launch configuration the benchmark times
    wl = step_case("longctx_bf16+replay", 48, 6)
    assert wl.splits > 1


def test_step_bench_configuration_sampled():
    # exactly what bench.py times: dit1k with the prefix delivered in the replay layout
    step_case("dit1k_bf16+replay", 64, 6)


def test_step_dit2k_bf16_sampled():
    step_case("dit2k_bf16", 24, 4)


def test_step_video_bf16_sampled():
    step_case("video_bf16", 24, 5)
