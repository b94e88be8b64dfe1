"""GPU parity of the block-scaled FP8 path (one E8M0 scale per run of 32 head_dim elements
of each row): codes and scales bit for bit against the oracle's block quantization, alone
and with RoPE in the same pass, and the attention with the fp8 score GEMM against the
oracle's attention of the dequantized q and k, within the bf16 gate. The inputs give
every run its own power-of-two magnitude, so a scale applied to the wrong run (a lane
half or a key row off) changes the result by factors of 2 and more."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from helpers import TOL, attention_err, f64, fold_factor, lse_err_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def graded(shape, seed, span, dtype=torch.bfloat16):
    """Seeded N(0,1) values (fp32, rounded to dtype) with each 32-element run of the last
    axis times its own power of two 2^u, u uniform in [-span, span]."""
    x = synth.random_tensor(shape, seed, torch.float32)
    runs = x.reshape(*shape[:-1], shape[-1] // 32, 32)
    g = torch.Generator().manual_seed(seed + 77)
    u = torch.randint(-span, span + 1, runs.shape[:-1], generator=g).float()
    return (runs * torch.exp2(u)[..., None]).reshape(shape).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 300, 5, 128), (1, 17, 3, 64), (3, 1, 2, 32), (1, 9, 2, 1024)])
def test_quantize_blocks_bitexact(dtype, shape):
    note(f"quantize fp8 blocks {dtype} {shape}")
    x = graded(shape, 5000 + shape[1], 20, torch.float32)
    x[0, 0, 0, :32] = 0.0                                       # an all-zero run
    x[0, 0, -1, -32:] *= 0.0
    x[0, 0, -1, -1] = 448.0 * 2.0 ** -10                        # a run whose max is exactly 448 * 2^e
    if dtype == torch.float32 and shape[1] > 1:
        x[0, 1, 0, :32] *= 1e-39                                 # fp32 subnormals: e held at -127
    x = x.to(dtype)
    codes, scales = nx.nxattn_quantize_fp8_blocks(x.to(DEV))
    torch.cuda.synchronize()
    rc, rs = ofp8.quantize_fp8_blocks(f64(x))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert int(rs[0, 0, 0, 0]) == 127 and int(rs[0, 0, -1, -1]) == 117


def test_quantize_blocks_strided():
    note("quantize fp8 blocks on a strided view")
    base = graded((2, 40, 6, 128), 5100, 6)
    x = base.to(DEV)[:, :, 1:5, :]
    codes, scales = nx.nxattn_quantize_fp8_blocks(x)
    torch.cuda.synchronize()
    rc, rs = ofp8.quantize_fp8_blocks(f64(base[:, :, 1:5, :]))
    assert np.array_equal(scales.cpu().numpy(), rs) and np.array_equal(codes.cpu().numpy(), rc)


ROPE_CASES = [
    # (B, grid, pairs, heads per tensor, D, interleaved, global_freq)
    (2, (15, 20), (32, 32), (5, 2), 128, False, False),
    (2, (4, 6, 8), (16, 24, 24), (3, 1, 4), 128, True, False),
    (1, (37,), (32,), (4, 2), 64, False, True),
    (1, (21,), (96,), (2, 1), 192, False, False),               # 24 lanes per row: rows straddle waves
    (1, (13,), (128,), (3, 1), 256, True, False),
]


def rope_block_inputs(case, dtype, seed):
    B, grid, pairs, heads, D, inter, gf = case
    S = int(np.prod(grid))
    xs = [graded((B, S, H, D), seed + 10 * t + S, 4, torch.float32).to(dtype).to(DEV) for t, H in enumerate(heads)]
    xs[0][0, 0, 0, :32] = 0                                     # an all-zero run
    descs = [nx.rope_desc(grid, pairs, tuple(3 * b + a for a in range(len(grid))), 10000.0, inter, gf)
             for b in range(B)]
    return xs, descs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", ROPE_CASES)
def test_rope_quantize_blocks_matches_rope_then_quantize(dtype, case):
    note(f"rope+quantize fp8 blocks {dtype} {case}")
    xs, descs = rope_block_inputs(case, dtype, 5200)
    x0 = [x.clone() for x in xs]
    seps = [x.clone() for x in xs]
    for sx in seps:
        nx.nxattn_rope_apply(sx, descs)
    mults = [0.0, 0.0, 3.0][:len(xs)]
    folds = [True, False, False][:len(xs)]
    outs = nx.nxattn_rope_quantize_fp8(xs, descs, mults=mults, folds=folds, blocks=True)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    D = case[4]
    refm = [fold_factor(D) if f else m for m, f in zip(mults, folds)]
    for x, xo, sx, mu, (codes, scales) in zip(xs, x0, seps, refm, outs):
        assert torch.equal(x.view(bits).cpu(), xo.view(bits).cpu())     # x is only read
        sm = sx.cpu().float() * torch.tensor(mu if mu else 1.0, dtype=torch.float32)
        rc, rs = ofp8.quantize_fp8_blocks(f64(sm))
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)


def test_rope_quantize_blocks_noalloc_matches():
    # the no-allocation entry point passes block-scaled calls through (no scratch is used)
    note("rope+quantize fp8 blocks: no-allocation entry point against the plain one")
    case = ROPE_CASES[0]
    xs, descs = rope_block_inputs(case, torch.bfloat16, 5300)
    outs = nx.nxattn_rope_quantize_fp8(xs, descs, folds=[True, False], blocks=True)
    c2 = [torch.empty_like(c) for c, _ in outs]
    s2 = [torch.full_like(s, 0xAB) for _, s in outs]
    nx.nxattn_rope_quantize_fp8_noalloc(xs, descs, c2, s2, folds=[True, False], blocks=True)
    torch.cuda.synchronize()
    for (c, s), cc, ss in zip(outs, c2, s2):
        assert torch.equal(c.cpu(), cc.cpu()) and torch.equal(s.cpu(), ss.cpu())


def block_case(B, S, Hq, Hkv, P, seed, fold=False, span=2, lse=True):
    D = 128
    note(f"fwd fp8 blocks B={B} S={S} Hq={Hq} Hkv={Hkv} P={P} seed={seed} fold={fold} span={span}")
    q = graded((B, S, Hq, D), seed, span)
    k = graded((B, S, Hkv, D), seed + 1, span)
    v = synth.random_tensor((B, S, Hkv, D), seed + 2, torch.bfloat16)
    pk = [graded((p, Hkv, D), seed + 3 + b, span) if p else None for b, p in enumerate(P)]
    pv = [synth.random_tensor((p, Hkv, D), seed + 13 + b, torch.bfloat16) if p else None for b, p in enumerate(P)]
    cf = fold_factor(D)
    if fold:
        descs = [nx.rope_desc((S,), (64,), (5 * b,)) for b in range(B)]
        qd = q.to(DEV)
        [(q8, qs)] = nx.nxattn_rope_quantize_fp8([qd], descs, folds=[True], blocks=True)
        nx.nxattn_rope_apply(qd, descs)
        q = qd.cpu()
        qref = q.float() * torch.tensor(cf, dtype=torch.float32)
    else:
        q8, qs = nx.nxattn_quantize_fp8_blocks(q.to(DEV))
        qref = q
    k8, ks = nx.nxattn_quantize_fp8_blocks(k.to(DEV))
    pk8, pks = [], []
    for b in range(B):
        if pk[b] is None:
            pk8.append(None)
            pks.append(None)
            continue
        c, s = nx.nxattn_quantize_fp8_blocks(pk[b].to(DEV)[None])
        pk8.append(c[0])
        pks.append(s[0])
    o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    ls = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV) if lse else None
    nx.nxattn_fwd_fp8(q8, k8, None, None, v.to(DEV), o, pk8, [t.to(DEV) if t is not None else None for t in pv],
                      lse=ls, q_folded=fold, q_scales=qs, k_scales=ks, prefix_k_scales=pks)
    torch.cuda.synchronize()
    rq, rqs = ofp8.quantize_fp8_blocks(f64(qref))
    rk, rks = ofp8.quantize_fp8_blocks(f64(k))
    assert np.array_equal(q8.cpu().numpy(), rq) and np.array_equal(qs.cpu().numpy(), rqs)
    assert np.array_equal(k8.cpu().numpy(), rk) and np.array_equal(ks.cpu().numpy(), rks)
    dq, dk = ofp8.dequantize_fp8_blocks(rq, rqs), ofp8.dequantize_fp8_blocks(rk, rks)
    if fold:
        dq = dq / cf
    worst = 0.0
    for b in range(B):
        dpk = None
        if pk[b] is not None:
            dpk = ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(f64(pk[b])))
        args = (dq[b], dk[b], f64(v[b]), dpk, f64(pv[b]) if pv[b] is not None else None)
        err = attention_err(f64(o.cpu()[b]), oracle.attention(*args))
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, err)
        if lse:
            rl = oracle.attention_lse(*args)
            assert lse_err_ok(f64(ls.cpu()[b]), rl), (b, float(np.max(np.abs(f64(ls.cpu()[b]) - rl))))
    note(f"  worst branch error {worst:.3e} (gate {TOL['bf16']:.0e})")


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (2, 300, 8, 2, (37, 0)),      # ragged Sq, straddling prefix, a branch without prefix
    (1, 1, 8, 1, (200,)),         # one own token, long prefix
    (2, 640, 8, 2, (128, 200)),   # whole prefix tiles, then a straddling one
    (3, 70, 2, 1, (5, 0, 64)),
    (2, 200, 4, 2, (300, 7)),     # prefix longer than the own tokens; ragged last tile
    (1, 129, 4, 4, (0,)),         # G = 1, no prefix
    (8, 70, 4, 2, (0, 1, 63, 64, 65, 130, 7, 300)),   # the most branches a call takes
])
def test_fwd_fp8_blocks_reduced(B, S, Hq, Hkv, P):
    block_case(B, S, Hq, Hkv, P, 5400 + S)


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (2, 300, 8, 2, (37, 0)),
    (2, 200, 4, 2, (300, 7)),
])
def test_fwd_fp8_blocks_folded_q(B, S, Hq, Hkv, P):
    block_case(B, S, Hq, Hkv, P, 5500 + S, fold=True)


def test_fwd_fp8_blocks_uniform_inputs():
    # plain N(0,1) inputs (the runs of one row then mostly share a scale), q folded
    block_case(2, 257, 8, 2, (64, 3), 5600, fold=True, span=0)


def test_fwd_fp8_blocks_deterministic():
    note("fwd fp8 blocks determinism")
    B, S, Hq, Hkv, D, P = 2, 300, 8, 2, 128, 99
    q = graded((B, S, Hq, D), 5700, 2).to(DEV)
    k = graded((B, S, Hkv, D), 5701, 2).to(DEV)
    v = synth.random_tensor((B, S, Hkv, D), 5702, torch.bfloat16).to(DEV)
    pk = graded((1, P, Hkv, D), 5703, 2).to(DEV)
    pv = synth.random_tensor((P, Hkv, D), 5704, torch.bfloat16).to(DEV)
    descs = [nx.rope_desc((S,), (64,), (7 * b,)) for b in range(B)]
    [(q8, qs), (k8, ks)] = nx.nxattn_rope_quantize_fp8([q, k], descs, folds=[True, False], blocks=True)
    pk8, pks = nx.nxattn_quantize_fp8_blocks(pk)
    outs = []
    for _ in range(2):
        o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
        ls = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        nx.nxattn_fwd_fp8(q8, k8, None, None, v, o, [pk8[0], None], [pv, None], lse=ls, q_folded=True,
                          q_scales=qs, k_scales=ks, prefix_k_scales=[pks[0], None])
        torch.cuda.synchronize()
        outs.append((o.cpu(), ls.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def qload_case(B, S, Hq, Hkv, P, seed, grid=None, pairs=(64,), offsets=None, inter=False, gf=False, span=2,
               q_view=False):
    """nxattn_fwd_fp8 with q rotated, folded and block-quantized on load (keys
    block-quantized without RoPE), checked two ways:
    - isolated: the codes and run scales the kernel formed (q8_out, q_scales_out) are
      dequantized by the oracle, and the output and lse are held to the oracle's attention
      of them (output at the bf16 gate, lse at its own tolerance);
    - the oracle chain: fp64 RoPE of q times the fold factor, block quantization; the
      kernel's codes are compared with the chain's (the kernel rotates in fp32, so a value
      within a few fp32 ulps of a rounding boundary may take the neighbouring code: counted,
      and held to a handful), and the output is held to the bf16 gate against the attention
      of the chain's codes."""
    D = 128
    grid = grid or (S,)
    offsets = offsets or [tuple(5 * b + a for a in range(len(grid))) for b in range(B)]
    note(f"fwd fp8 q on load B={B} S={S} Hq={Hq} Hkv={Hkv} P={P} grid={grid} pairs={pairs} inter={inter} "
         f"gf={gf} offsets={offsets[0]} seed={seed}")
    if q_view:
        qfull = graded((B, S, Hq + 2, D), seed, span)
        q = qfull[:, :, 1:Hq + 1, :]
    else:
        q = graded((B, S, Hq, D), seed, span)
    k = graded((B, S, Hkv, D), seed + 1, span)
    v = synth.random_tensor((B, S, Hkv, D), seed + 2, torch.bfloat16)
    pk = [graded((p, Hkv, D), seed + 3 + b, span) if p else None for b, p in enumerate(P)]
    pv = [synth.random_tensor((p, Hkv, D), seed + 13 + b, torch.bfloat16) if p else None for b, p in enumerate(P)]
    descs = [nx.rope_desc(grid, pairs, offsets[b], 10000.0, inter, gf) for b in range(B)]
    qd = (qfull.to(DEV)[:, :, 1:Hq + 1, :] if q_view else q.to(DEV))
    q_before = qd.clone()
    k8, ks = nx.nxattn_quantize_fp8_blocks(k.to(DEV))
    pk8, pks = [], []
    for b in range(B):
        if pk[b] is None:
            pk8.append(None)
            pks.append(None)
            continue
        c, s_ = nx.nxattn_quantize_fp8_blocks(pk[b].to(DEV)[None])
        pk8.append(c[0])
        pks.append(s_[0])
    o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    ls = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    q8o = torch.full((B, S, Hq, D), 0x7F, dtype=torch.uint8, device=DEV)
    qso = torch.full((B, S, Hq, D // 32), 0xFF, dtype=torch.uint8, device=DEV)
    nx.nxattn_fwd_fp8(None, k8, None, None, v.to(DEV), o, pk8, [t.to(DEV) if t is not None else None for t in pv],
                      lse=ls, k_scales=ks, prefix_k_scales=pks, q=qd, q_rope=descs, q8_out=q8o, q_scales_out=qso)
    torch.cuda.synchronize()
    assert torch.equal(qd.view(torch.int16).cpu(), q_before.view(torch.int16).cpu())   # q is only read
    cf = float(fold_factor(D))
    dk = ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(f64(k)))
    kc, kcs = q8o.cpu().numpy(), qso.cpu().numpy()
    worst_iso = worst_ch = 0.0
    n_code = n_scale = 0
    for b in range(B):
        qr = oracle.rope(f64(q[b]), grid, pairs, offsets[b], 10000.0, interleaved=inter, global_freq=gf) * cf
        cc, cs = ofp8.quantize_fp8_blocks(qr)
        n_code += int(np.count_nonzero(cc != kc[b]))
        n_scale += int(np.count_nonzero(cs != kcs[b]))
        dpk = None
        if pk[b] is not None:
            dpk = ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(f64(pk[b])))
        rest = (dk[b], f64(v[b]), dpk, f64(pv[b]) if pv[b] is not None else None)
        g = f64(o.cpu()[b])
        iso = (ofp8.dequantize_fp8_blocks(kc[b], kcs[b]) / cf,) + rest
        err_iso = attention_err(g, oracle.attention(*iso))
        err_ch = attention_err(g, oracle.attention(ofp8.dequantize_fp8_blocks(cc, cs) / cf, *rest))
        worst_iso, worst_ch = max(worst_iso, err_iso), max(worst_ch, err_ch)
        assert err_iso <= TOL["bf16"], (b, err_iso)
        assert err_ch <= TOL["bf16"], (b, err_ch)
        rl = oracle.attention_lse(*iso)
        assert lse_err_ok(f64(ls.cpu()[b]), rl), (b, float(np.max(np.abs(f64(ls.cpu()[b]) - rl))))
    total = B * S * Hq * D
    note(f"  worst branch error {worst_iso:.3e} against the kernel's own codes, {worst_ch:.3e} against the oracle "
         f"chain (gate {TOL['bf16']:.0e}); codes differing from the chain's: {n_code} of {total}, run scales "
         f"{n_scale} of {total // 32}")
    assert n_code <= max(8, total // 10000) and n_scale <= max(2, total // 320000)


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (2, 300, 8, 2, (37, 0)),
    (1, 1, 8, 1, (200,)),
    (2, 200, 4, 2, (300, 7)),
    (1, 129, 4, 4, (0,)),
])
def test_fwd_fp8_q_on_load_reduced(B, S, Hq, Hkv, P):
    qload_case(B, S, Hq, Hkv, P, 5800 + S)


@pytest.mark.parametrize("kw", [
    dict(grid=(12, 25), pairs=(32, 32)),                         # 2-D, two sections
    dict(grid=(3, 10, 10), pairs=(16, 24, 24), inter=True),      # 3-D, adjacent pairs
    dict(grid=(10, 30), pairs=(32, 32), gf=True),                # one global ladder over both axes
    dict(grid=(300,), pairs=(64,), offsets=[((1 << 24) - 300,), ((1 << 23) + 7,)]),   # positions near 2^24
    dict(grid=(300,), pairs=(64,), q_view=True),                 # q as a strided view
])
def test_fwd_fp8_q_on_load_rope_forms(kw):
    qload_case(2, 300, 8, 2, (40, 0), 5900, **kw)


def test_fwd_fp8_q_on_load_deterministic():
    note("fwd fp8 q on load determinism")
    B, S, Hq, Hkv, D, P = 2, 300, 8, 2, 128, 99
    q = graded((B, S, Hq, D), 6000, 2).to(DEV)
    k = graded((B, S, Hkv, D), 6001, 2).to(DEV)
    v = synth.random_tensor((B, S, Hkv, D), 6002, torch.bfloat16).to(DEV)
    pk = graded((1, P, Hkv, D), 6003, 2).to(DEV)
    pv = synth.random_tensor((P, Hkv, D), 6004, torch.bfloat16).to(DEV)
    descs = [nx.rope_desc((S,), (64,), (7 * b,)) for b in range(B)]
    [(k8, ks)] = nx.nxattn_rope_quantize_fp8([k], descs, blocks=True)
    pk8, pks = nx.nxattn_quantize_fp8_blocks(pk)
    outs = []
    for _ in range(2):
        o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
        nx.nxattn_fwd_fp8(None, k8, None, None, v, o, [pk8[0], None], [pv, None], k_scales=ks,
                          prefix_k_scales=[pks[0], None], q=q, q_rope=descs)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.equal(outs[0], outs[1])
