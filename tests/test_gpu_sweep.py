"""Seeded random sweeps over the shapes and options of the fused launches, each against the
separate calls it replaces, bit for bit. Those separate calls are held to the oracle by
the parity tests, so every case here inherits their gates.

- the branch-pair launch (nxattn_fwd with cfg_out: both CFG branches per workgroup and the
  guidance combination in the epilogue; LingBot-Video page, "Key Parameters") against
  nxattn_fwd over both branches followed by nxattn_cfg_combine: any sequence length, GQA
  group, prefix lengths (zero, straddling tiles), prefix-only keys, strided q/k/v views,
  q rotated on load or stored, with and without the branch outputs and the log-sum-exp;
- the same for the fp8 score GEMM (block scales, one exponent per slice, q quantized on
  load);
- the RoPE of one tensor with prefix relayouts in the same launch against
  nxattn_rope_apply and one nxattn_kv_relayout per job (NeoPP page, "KV file layout").
Each case prints its parameters before it runs."""
import sys

import numpy as np
import pytest
import torch

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def bits(t):
    return t.view({torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8}[t.dtype])


def same(a, b):
    return torch.equal(bits(a), bits(b))


def rnd(shape, seed, dtype=torch.bfloat16):
    return synth.random_tensor(shape, seed, dtype).to(DEV)


def view_of(shape, seed, pad_h, pad_d, dtype=torch.bfloat16):
    """A [B, S, H, D] view into a larger tensor (pad_h more heads, pad_d more columns), or a
    contiguous tensor when both pads are 0."""
    B, S, H, Dd = shape
    base = rnd((B, S, H + pad_h, Dd + pad_d), seed, dtype)
    return base[:, :, :H, :Dd]


# ------------------------------------------------------------------ branch pairs, bf16
def pair_case(i):
    rng = np.random.default_rng(7100 + i)
    S = int(rng.integers(1, 700))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
    prefix_only = bool(rng.random() < 0.15)
    P = tuple(int(rng.integers(1, 400)) if (prefix_only or rng.random() < 0.75) else 0 for _ in range(2))
    return dict(S=S, Hq=Hq, Hkv=Hkv, P=P, prefix_only=prefix_only, rope=bool(rng.random() < 0.5),
                strided=bool(rng.random() < 0.5), keep_o=bool(rng.random() < 0.5),
                lse=bool(rng.random() < 0.5), g=round(float(rng.uniform(-3.0, 9.0)), 3),
                offsets=tuple(int(rng.integers(0, 5000)) for _ in range(2)))


@pytest.mark.parametrize("i", range(24))
def test_pair_sweep(i):
    c = pair_case(i)
    note(f"pair sweep {i}: {c}")
    S, Hq, Hkv, P = c["S"], c["Hq"], c["Hkv"], c["P"]
    pad = (1, 8) if c["strided"] else (0, 0)
    q = view_of((2, S, Hq, D), 7200 + i, *pad)
    k = view_of((2, S, Hkv, D), 7300 + i, *pad)
    v = view_of((2, S, Hkv, D), 7400 + i, *pad)
    assert k.stride() == v.stride()
    pre = [rnd((2, p, Hkv, D), 7500 + 2 * i + b) if p else None for b, p in enumerate(P)]
    descs = [nx.rope_desc((S,), (64,), (c["offsets"][b],), 10000.0) for b in range(2)] if c["rope"] else None

    def lse_buf():
        return torch.full((2, Hq, S), float("nan"), dtype=torch.float32, device=DEV) if c["lse"] else None

    kw = dict(q_rope=descs, prefix_only=c["prefix_only"])
    o_ref, lse_ref = torch.empty((2, S, Hq, D), dtype=torch.bfloat16, device=DEV), lse_buf()
    out_ref = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd(q, k, v, o_ref, pre, lse=lse_ref, **kw)
    nx.nxattn_cfg_combine(o_ref[0], o_ref[1], out_ref, c["g"])
    o_f = torch.full((2, S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV) if c["keep_o"] else None
    lse_f = lse_buf()
    out_f = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd(q, k, v, o_f, pre, lse=lse_f, cfg_out=out_f, guidance=c["g"], **kw)
    torch.cuda.synchronize()
    assert same(out_f, out_ref), "guided output differs from the separate path"
    if o_f is not None:
        assert same(o_f, o_ref), "branch outputs differ"
    if lse_f is not None:
        assert same(lse_f, lse_ref), "lse differs"


# ------------------------------------------------------------------ branch pairs, fp8 score GEMM
def fp8_case(i):
    rng = np.random.default_rng(7600 + i)
    mode = ["blocks", "slice", "q_on_load"][i % 3]
    S = int(rng.integers(1, 600))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    P = tuple(int(rng.integers(1, 300)) if rng.random() < 0.75 else 0 for _ in range(2))
    return dict(mode=mode, S=S, Hq=Hq, Hkv=Hkv, P=P, keep_o=bool(rng.random() < 0.5),
                g=round(float(rng.uniform(-3.0, 9.0)), 3), offsets=tuple(int(rng.integers(0, 3000)) for _ in range(2)))


@pytest.mark.parametrize("i", range(12))
def test_fp8_pair_sweep(i):
    c = fp8_case(i)
    note(f"fp8 pair sweep {i}: {c}")
    S, Hq, Hkv, P, mode = c["S"], c["Hq"], c["Hkv"], c["P"], c["mode"]
    q = rnd((2, S, Hq, D), 7700 + i)
    k = rnd((2, S, Hkv, D), 7800 + i)
    v = rnd((2, S, Hkv, D), 7900 + i)
    pk = [rnd((1, p, Hkv, D), 8000 + 2 * i + b) if p else None for b, p in enumerate(P)]
    pv = [rnd((p, Hkv, D), 8100 + 2 * i + b) if p else None for b, p in enumerate(P)]
    if mode == "slice":
        q8, qe = nx.nxattn_quantize_fp8(q)
        k8, ke = nx.nxattn_quantize_fp8(k)
        pre = [nx.nxattn_quantize_fp8(x) if x is not None else (None, None) for x in pk]
        pke = torch.zeros((2, Hkv), dtype=torch.int8, device=DEV)
        for b, (_, e) in enumerate(pre):
            if e is not None:
                pke[b] = e[0]
        pk8 = [cd[0] if cd is not None else None for cd, _ in pre]
        args, kw = (q8, k8, qe, ke, v), {}
        pargs = (pk8, pv, pke)
    else:
        k8, ks = nx.nxattn_quantize_fp8_blocks(k)
        pre = [nx.nxattn_quantize_fp8_blocks(x) if x is not None else (None, None) for x in pk]
        pk8 = [cd[0] if cd is not None else None for cd, _ in pre]
        kw = dict(k_scales=ks, prefix_k_scales=[s_[0] if s_ is not None else None for _, s_ in pre])
        if mode == "blocks":
            q8, qs = nx.nxattn_quantize_fp8_blocks(q)
            args = (q8, k8, None, None, v)
            kw["q_scales"] = qs
        else:
            args = (None, k8, None, None, v)
            kw["q"] = q
            kw["q_rope"] = [nx.rope_desc((S,), (64,), (c["offsets"][b],), 10000.0) for b in range(2)]
        pargs = (pk8, pv, None)
    o_ref = torch.empty_like(q)
    out_ref = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd_fp8(*args, o_ref, *pargs, **kw)
    nx.nxattn_cfg_combine(o_ref[0], o_ref[1], out_ref, c["g"])
    o_f = torch.full_like(q, float("nan")) if c["keep_o"] else None
    out_f = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd_fp8(*args, o_f, *pargs, cfg_out=out_f, guidance=c["g"], **kw)
    torch.cuda.synchronize()
    assert same(out_f, out_ref), "guided output differs from the separate path"
    if o_f is not None:
        assert same(o_f, o_ref), "branch outputs differ"


# ------------------------------------------------------------------ RoPE with relayouts
def grid_of(rng, S_max):
    n = int(rng.integers(1, 4))
    if n == 1:
        return (int(rng.integers(1, S_max)),)
    if n == 2:
        return (int(rng.integers(1, 30)), int(rng.integers(1, 30)))
    return (int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 9)))


def pairs_of(rng, n, half):
    if n == 1:
        return (half,)
    cuts = sorted(int(x) for x in rng.choice(np.arange(1, half), size=n - 1, replace=False))
    edges = [0, *cuts, half]
    return tuple(edges[j + 1] - edges[j] for j in range(n))


@pytest.mark.parametrize("i", range(12))
def test_rope_relayout_sweep(i):
    rng = np.random.default_rng(8200 + i)
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    Dd = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 9))
    grid = grid_of(rng, 400)
    S = int(np.prod(grid))
    pairs = pairs_of(rng, len(grid), Dd // 2)
    inter = bool(rng.random() < 0.3)
    gf = bool(rng.random() < 0.2)
    offs = [tuple(int(rng.integers(0, 20000)) for _ in grid) for _ in range(B)]
    jobs = []
    for j in range(int(rng.integers(0, 4))):
        L, Hj, Pj, Dj = int(rng.integers(1, 3)), int(rng.integers(1, 6)), int(rng.integers(0, 300)), int(rng.choice([64, 128]))
        jobs.append(((L, 2, Hj, Pj, Dj), int(rng.integers(0, 2))))
    note(f"rope+relayout sweep {i}: {dtype} B={B} grid={grid} pairs={pairs} H={H} D={Dd} interleaved={inter} "
         f"global={gf} offsets={offs} jobs={jobs}")
    x0 = rnd((B, S, H, Dd), 8300 + i, dtype)
    descs = [nx.rope_desc(grid, pairs, offs[b], 10000.0, inter, gf) for b in range(B)]
    pairs_t = []
    for jn, ((L, two, Hj, Pj, Dj), d) in enumerate(jobs):
        replay = (L, two, Hj, Pj, Dj)
        online = (L, two, Pj, Hj, Dj)
        src = rnd(replay if d == 0 else online, 8400 + 10 * i + jn, dtype)
        pairs_t.append((src, torch.full(online if d == 0 else replay, float("nan"), dtype=dtype, device=DEV), d))
    x_ref = x0.clone()
    nx.nxattn_rope_apply(x_ref, descs)
    refs = []
    for src, dst, d in pairs_t:
        r = torch.full_like(dst, float("nan"))
        if src.numel():
            nx.nxattn_kv_relayout(src, r, d)
        refs.append(r)
    x = x0.clone()
    nx.nxattn_rope_apply_relayout(x, descs, pairs_t)
    torch.cuda.synchronize()
    assert same(x, x_ref), "rotation differs"
    for jn, ((_, dst, _), r) in enumerate(zip(pairs_t, refs)):
        assert torch.equal(torch.isnan(dst.float()), torch.isnan(r.float())), f"job {jn}: coverage differs"
        assert same(dst.nan_to_num(0), r.nan_to_num(0)), f"job {jn} differs"
