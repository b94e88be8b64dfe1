"""GPU parity of the FP8 path: the E4M3 quantization bit for bit against the oracle, and
the attention with the fp8 score GEMM against the oracle's attention of the dequantized
q and k (the recipe's definition), within the bf16 gate (P and P.V are the bf16 path's)."""
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


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 300, 5, 128), (1, 17, 3, 72), (3, 1, 2, 8)])
def test_quantize_bitexact(dtype, shape):
    note(f"quantize fp8 {dtype} {shape}")
    B, S, H, D = shape
    x = synth.random_tensor(shape, 4000 + S, torch.float32)
    mult = torch.tensor([1.0, 300.0, 1e-3, 0.0, 7.0][:H] + [1.0] * max(0, H - 5))
    x = (x * mult[None, None, :, None]).to(dtype)              # head 3 (if any): all zero
    if H > 2:
        x[0, 0, 2, 0] = torch.tensor(448.0 * 2.0 ** -10, dtype=dtype)   # an exact 448 * 2^e amax
    codes, exps = nx.nxattn_quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    rc, re = ofp8.quantize_fp8(f64(x))
    assert np.array_equal(exps.cpu().numpy(), re)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_strided_and_tiny():
    note("quantize fp8 strided view, fp32 subnormal slice")
    base = synth.random_tensor((2, 40, 6, 64), 4100, torch.float32)
    base[:, :, 3, :] *= 1e-39                                   # fp32 subnormals: e clamps at -127
    x = base.to(DEV)[:, :, 1:5, :]
    codes, exps = nx.nxattn_quantize_fp8(x)
    torch.cuda.synchronize()
    rc, re = ofp8.quantize_fp8(f64(base[:, :, 1:5, :]))
    assert np.array_equal(exps.cpu().numpy(), re) and np.array_equal(codes.cpu().numpy(), rc)
    assert int(re[:, 2].min()) == -127


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", [
    # (B, grid, pairs, heads per tensor, D, interleaved, global_freq)
    ((2, (15, 20), (32, 32), (5,), 128, False, False)),
    ((2, (15, 20), (32, 32), (5, 2), 128, False, False)),
    ((2, (4, 6, 8), (16, 24, 24), (3, 1, 4), 128, True, False)),
    ((1, (37,), (36,), (4, 2, 1, 3), 72, False, True)),
])
def test_rope_quantize_matches_rope_then_quantize(dtype, case):
    B, grid, pairs, heads, D, inter, gf = case
    S = int(np.prod(grid))
    note(f"rope+quantize fp8 {dtype} B={B} grid={grid} heads={heads} D={D} inter={inter} gf={gf}")
    mult = torch.tensor([1.0, 300.0, 1e-3, 0.0, 7.0])
    xs = []
    for t, H in enumerate(heads):
        x = synth.random_tensor((B, S, H, D), 4200 + 10 * t + S, torch.float32)
        m = torch.roll(mult, t)[:H] if H <= 5 else torch.ones(H)
        xs.append((x * m[None, None, :, None]).to(dtype).to(DEV))    # some heads all zero
    descs = [nx.rope_desc(grid, pairs, tuple(3 * b + a for a in range(len(grid))), 10000.0, inter, gf)
             for b in range(B)]
    ws = torch.full((max(4, nx.quantize_fp8_workspace_bytes(B, S, sum(heads))),), 0x7f, dtype=torch.uint8,
                    device=DEV)                                              # stale workspace contents
    x0 = [x.clone() for x in xs]
    seps = [x.clone() for x in xs]
    for sx in seps:
        nx.nxattn_rope_apply(sx, descs)
    # per tensor: the softmax fold factor formed by the library, none (0 and 1), a plain 3
    mults = [0.0, 0.0, 3.0, 1.0][:len(xs)]
    folds = [True, False, False, False][:len(xs)]
    outs = nx.nxattn_rope_quantize_fp8(xs, descs, workspace=ws, mults=mults, folds=folds)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    refm = [fold_factor(D) if f else m for m, f in zip(mults, folds)]
    for x, xo, sx, mu, (codes, exps) in zip(xs, x0, seps, refm, outs):
        assert torch.equal(x.view(bits).cpu(), xo.view(bits).cpu())     # x is only read
        # the oracle's codes of the stored rotation times mult (one fp32 multiply)
        sm = sx.cpu().float() * torch.tensor(mu if mu else 1.0, dtype=torch.float32)
        rc, re = ofp8.quantize_fp8(f64(sm))
        assert np.array_equal(exps.cpu().numpy(), re)
        assert np.array_equal(codes.cpu().numpy(), rc)


def test_rope_quantize_strided_then_smaller():
    note("rope+quantize fp8 on strided views of one buffer, then a smaller input on the same workspace")
    B, grid, pairs, H, D = 2, (8, 12), (32, 32), 6, 128
    S = 96
    base = synth.random_tensor((B, S, H + 2, D), 4300, torch.float32).to(torch.bfloat16).to(DEV)
    qv, kv = base[:, :, 1:H + 1, :], base[:, :, 0:3, :]           # overlapping read-only inputs
    descs = [nx.rope_desc(grid, pairs, (b, 2 * b)) for b in range(B)]
    ws = torch.empty(max(4, nx.quantize_fp8_workspace_bytes(B, S, H + 3)), dtype=torch.uint8, device=DEV)
    base0 = base.clone()
    seps = [qv.clone(), kv.clone()]
    for sx in seps:
        nx.nxattn_rope_apply(sx, descs)
    outs = nx.nxattn_rope_quantize_fp8([qv, kv], descs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16).cpu(), base0.view(torch.int16).cpu())
    for sx, (codes, exps) in zip(seps, outs):
        rc, re = ofp8.quantize_fp8(f64(sx.cpu()))
        assert np.array_equal(exps.cpu().numpy(), re) and np.array_equal(codes.cpu().numpy(), rc)
    small = (synth.random_tensor((1, 24, 2, D), 4301, torch.float32) * 1e-3).to(torch.bfloat16).to(DEV)
    sep2 = small.clone()
    d2 = [nx.rope_desc((24,), (64,), (9,))]
    nx.nxattn_rope_apply(sep2, d2)
    [(codes2, exps2)] = nx.nxattn_rope_quantize_fp8([small], d2, workspace=ws)   # maxima of the call above remain
    torch.cuda.synchronize()
    rc2, re2 = ofp8.quantize_fp8(f64(sep2.cpu()))
    assert np.array_equal(exps2.cpu().numpy(), re2) and np.array_equal(codes2.cpu().numpy(), rc2)


def fp8_case(B, S, Hq, Hkv, P, seed, pre_mult=1.0, lse=True, fold=False):
    D = 128
    note(f"fwd fp8 B={B} S={S} Hq={Hq} Hkv={Hkv} P={P} prefix x{pre_mult} seed={seed} fold={fold}")
    q = synth.random_tensor((B, S, Hq, D), seed, torch.bfloat16)
    k = synth.random_tensor((B, S, Hkv, D), seed + 1, torch.bfloat16)
    v = synth.random_tensor((B, S, Hkv, D), seed + 2, torch.bfloat16)
    pk = [(synth.random_tensor((p, Hkv, D), seed + 3 + b, torch.float32) * pre_mult).to(torch.bfloat16) if p else None
          for b, p in enumerate(P)]
    pv = [synth.random_tensor((p, Hkv, D), seed + 13 + b, torch.bfloat16) if p else None for b, p in enumerate(P)]
    cf = fold_factor(D)
    if fold:
        # q rotated and multiplied by softmax_scale*log2(e) inside the quantizer; the
        # reference takes the GPU's rotation (parity-tested on its own) times cf in fp32
        descs = [nx.rope_desc((S,), (64,), (5 * b,)) for b in range(B)]
        qd = q.to(DEV)
        [(q8, qe)] = nx.nxattn_rope_quantize_fp8([qd], descs, folds=[True])
        nx.nxattn_rope_apply(qd, descs)
        q = qd.cpu()
        qref = q.float() * torch.tensor(cf, dtype=torch.float32)
    else:
        q8, qe = nx.nxattn_quantize_fp8(q.to(DEV))
        qref = q
    k8, ke = nx.nxattn_quantize_fp8(k.to(DEV))
    pk8, pke = [], torch.zeros((B, Hkv), dtype=torch.int8, device=DEV)
    for b in range(B):
        if pk[b] is None:
            pk8.append(None)
            continue
        c, e = nx.nxattn_quantize_fp8(pk[b].to(DEV)[None])
        pk8.append(c[0])
        pke[b] = e[0]
    o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    ls = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV) if lse else None
    nx.nxattn_fwd_fp8(q8, k8, qe, ke, v.to(DEV), o, pk8, [t.to(DEV) if t is not None else None for t in pv],
                      pke if any(P) else None, lse=ls, q_folded=fold)
    torch.cuda.synchronize()
    # the reference dequantizes the oracle's own codes (equal to the GPU's: checked here too);
    # folded q codes stand for cf * q, so their dequantized values are divided by cf
    rq, rqe = ofp8.quantize_fp8(f64(qref))
    rk, rke = ofp8.quantize_fp8(f64(k))
    assert np.array_equal(q8.cpu().numpy(), rq) and np.array_equal(k8.cpu().numpy(), rk)
    dq, dk = ofp8.dequantize_fp8(rq, rqe), ofp8.dequantize_fp8(rk, rke)
    if fold:
        dq = dq / cf
    for b in range(B):
        dpk = None
        if pk[b] is not None:
            c, e = ofp8.quantize_fp8(f64(pk[b])[None])
            dpk = ofp8.dequantize_fp8(c, e)[0]
        args = (dq[b], dk[b], f64(v[b]), dpk, f64(pv[b]) if pv[b] is not None else None)
        ref = oracle.attention(*args)
        err = attention_err(f64(o.cpu()[b]), ref)
        assert err <= TOL["bf16"], (b, err)
        if lse:
            rl = oracle.attention_lse(*args)
            assert lse_err_ok(f64(ls.cpu()[b]), rl), (b, float(np.max(np.abs(f64(ls.cpu()[b]) - rl))))


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (2, 300, 8, 2, (37, 0)),      # ragged Sq, straddling prefix, a branch without prefix
    (1, 1, 8, 1, (200,)),         # one own token, long prefix
    (2, 640, 8, 2, (128, 200)),   # whole prefix tiles, then a straddling one
    (3, 70, 2, 1, (5, 0, 64)),
    (2, 200, 4, 2, (300, 7)),     # prefix longer than the own tokens; ragged last tile
    (1, 129, 4, 4, (0,)),         # G = 1, no prefix
    (8, 70, 4, 2, (0, 1, 63, 64, 65, 130, 7, 300)),   # the most branches a call takes
])
def test_fwd_fp8_reduced(B, S, Hq, Hkv, P):
    fp8_case(B, S, Hq, Hkv, P, 4200 + S)


def test_fwd_fp8_prefix_scale_differs():
    # prefix keys 100x larger than own keys: their exponents differ by ~7, so the tile that
    # straddles the prefix end mixes two E8M0 row scales
    fp8_case(2, 160, 8, 2, (100, 30), 4300, pre_mult=100.0)


@pytest.mark.parametrize("B,S,Hq,Hkv,P", [
    (2, 300, 8, 2, (37, 0)),
    (1, 1, 8, 1, (200,)),
    (2, 200, 4, 2, (300, 7)),
])
def test_fwd_fp8_folded_q(B, S, Hq, Hkv, P):
    # q's codes carry softmax_scale*log2(e): same attention as the unfolded call
    fp8_case(B, S, Hq, Hkv, P, 4400 + S, fold=True)


def test_fwd_fp8_folded_q_prefix_scale_differs():
    fp8_case(2, 160, 8, 2, (100, 30), 4500, pre_mult=100.0, fold=True)


def test_fwd_fp8_deterministic():
    # the same fp8 attention call twice gives the same bits (q folded, prefix on one branch)
    note("fwd fp8 determinism")
    B, S, Hq, Hkv, D, P = 2, 300, 8, 2, 128, 99
    q = synth.random_tensor((B, S, Hq, D), 4600, torch.bfloat16).to(DEV)
    k = synth.random_tensor((B, S, Hkv, D), 4601, torch.bfloat16).to(DEV)
    v = synth.random_tensor((B, S, Hkv, D), 4602, torch.bfloat16).to(DEV)
    pk = synth.random_tensor((1, P, Hkv, D), 4603, torch.bfloat16).to(DEV)
    pv = synth.random_tensor((P, Hkv, D), 4604, torch.bfloat16).to(DEV)
    descs = [nx.rope_desc((S,), (64,), (7 * b,)) for b in range(B)]
    [(q8, qe), (k8, ke)] = nx.nxattn_rope_quantize_fp8([q, k], descs, folds=[True, False])
    pk8, pe = nx.nxattn_quantize_fp8(pk)
    pke = torch.zeros((B, Hkv), dtype=torch.int8, device=DEV)
    pke[0] = pe[0]
    outs = []
    for _ in range(2):
        o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
        ls = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        nx.nxattn_fwd_fp8(q8, k8, qe, ke, v, o, [pk8[0], None], [pv, None], pke, lse=ls, q_folded=True)
        torch.cuda.synchronize()
        outs.append((o.cpu(), ls.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
