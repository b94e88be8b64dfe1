"""Classifier-free guidance folded into the attention call (cfg_out): each workgroup runs
both CFG branches of its query rows and writes the combination itself (LingBot-Video
page, "Key Parameters": guidance_scale; NeoPP page: the cond and uncond KV branches).

The bar is the separate path, bit for bit: nxattn_fwd's branch outputs (and lse), then
nxattn_cfg_combine on them. The parity tests hold that separate path to the oracle, so
the folded call inherits those gates exactly."""
import sys

import pytest
import torch

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from bidirectional_transformer_attention_amd.pipeline import AttentionStep

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_FP8 = 128


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def same(a, b):
    return torch.equal(bits(a), bits(b))


# (S, Hq, Hkv, prefix lengths, rotate q on load, lse, guidance)
CASES = [
    (150, 4, 2, (70, 13), True, True, 4.0),       # ragged last tile, prefix straddling a tile
    (96, 3, 3, (0, 64), False, False, 4.0),       # stored q; 9 query blocks: one wave group idle
    (1, 8, 1, (5, 0), True, False, 7.5),          # one query row, GQA 8, one branch without prefix
    (1024, 32, 8, (512, 128), True, True, 4.0),   # the 1K DiT's heads and prefixes, 1024 tokens
    (200, 4, 4, (33, 33), False, True, -1.25),    # any finite guidance
]


@pytest.mark.parametrize("S,Hq,Hkv,P,rope,with_lse,g", CASES)
def test_fwd_cfg_out_equals_separate_path(S, Hq, Hkv, P, rope, with_lse, g):
    D = 128
    note(f"fwd cfg_out S={S} Hq={Hq} Hkv={Hkv} P={P} q_rope={rope} lse={with_lse} guidance={g}")
    q = synth.random_tensor((2, S, Hq, D), 301 + S, torch.bfloat16).to(DEV)
    k = synth.random_tensor((2, S, Hkv, D), 302 + S, torch.bfloat16).to(DEV)
    v = synth.random_tensor((2, S, Hkv, D), 303 + S, torch.bfloat16).to(DEV)
    pre = [synth.random_tensor((2, p, Hkv, D), 304 + b, torch.bfloat16).to(DEV) if p else None
           for b, p in enumerate(P)]
    descs = [nx.rope_desc((S,), (64,), (P[b],), 10000.0) for b in range(2)] if rope else None

    def lse_buf():
        return torch.full((2, Hq, S), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None

    # the separate path
    o_ref, lse_ref = torch.empty_like(q), lse_buf()
    out_ref = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd(q, k, v, o_ref, pre, q_rope=descs, lse=lse_ref)
    nx.nxattn_cfg_combine(o_ref[0], o_ref[1], out_ref, g)
    # folded, branch outputs stored too
    o_f, lse_f = torch.full_like(q, float("nan")), lse_buf()
    out_f = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd(q, k, v, o_f, pre, q_rope=descs, lse=lse_f, cfg_out=out_f, guidance=g)
    # folded, no branch outputs, into a strided view (padding must stay untouched)
    big = torch.full((S, Hq + 1, D + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    out_n = big[:, :Hq, :D]
    nx.nxattn_fwd(q, k, v, None, pre, q_rope=descs, cfg_out=out_n, guidance=g)
    torch.cuda.synchronize()
    assert same(o_f, o_ref), "branch outputs differ from the one-branch-per-workgroup launch"
    assert same(out_f, out_ref), "combination differs from nxattn_cfg_combine of the branch outputs"
    assert same(out_n, out_ref), "combination without branch outputs differs"
    assert torch.isnan(big[:, Hq:, :].float()).all() and torch.isnan(big[:, :, D:].float()).all(), \
        "cfg_out wrote outside its view"
    if with_lse:
        assert same(lse_f, lse_ref), "lse differs"


def test_fwd_cfg_out_deterministic():
    S, Hq, Hkv, D = 300, 8, 2, 128
    note("fwd cfg_out determinism")
    q = synth.random_tensor((2, S, Hq, D), 311, torch.bfloat16).to(DEV)
    k = synth.random_tensor((2, S, Hkv, D), 312, torch.bfloat16).to(DEV)
    v = synth.random_tensor((2, S, Hkv, D), 313, torch.bfloat16).to(DEV)
    pre = [synth.random_tensor((2, 40, Hkv, D), 314, torch.bfloat16).to(DEV), None]
    outs = []
    for _ in range(3):
        out = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        nx.nxattn_fwd(q, k, v, None, pre, cfg_out=out, guidance=4.0)
        outs.append(out)
    torch.cuda.synchronize()
    assert all(same(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("name", ["dit1k_bf16", "dit2k_bf16"])
def test_step_fused_cfg_equals_separate_pass(name):
    # the step bench.py times (combination inside the attention call, no branch outputs)
    # against the step with the separate combine pass, at full size
    wl = synth.bench_workload(name)
    note(f"step {wl.name}: guidance inside the attention call against the separate pass")
    inp = synth.make_inputs(wl)
    sep = AttentionStep(wl, inp, fuse_cfg=False)
    out_sep = sep().clone()
    o_sep = sep.o.clone()
    keep = AttentionStep(wl, inp, fuse_cfg=True, keep_branches=True)
    out_keep = keep().clone()
    lean = AttentionStep(wl, inp, fuse_cfg=True, keep_branches=False)
    out_lean = lean().clone()
    torch.cuda.synchronize()
    assert sep.use_cfg and keep.fuse_cfg and lean.fuse_cfg and not lean.keep_branches
    assert same(keep.o, o_sep), "branch outputs differ"
    assert same(out_keep, out_sep), "combination differs (branch outputs stored)"
    assert same(out_lean, out_sep), "combination differs (no branch outputs)"


# ------------------------------------------------------------------ the fp8 score GEMM
@pytest.mark.parametrize("S,Hq,Hkv,P,blocks,g", [
    (150, 4, 2, (70, 13), True, 4.0),      # block scales, ragged and straddling tiles
    (96, 3, 3, (0, 64), True, -1.25),      # one branch without prefix, 9 query blocks
    (150, 4, 2, (70, 13), False, 6.0),     # one exponent per (branch, head)
])
def test_fwd_fp8_cfg_out_equals_separate_path(S, Hq, Hkv, P, blocks, g):
    D = 128
    note(f"fwd_fp8 cfg_out S={S} Hq={Hq} Hkv={Hkv} P={P} blocks={blocks} guidance={g}")
    q = synth.random_tensor((2, S, Hq, D), 321 + S, torch.bfloat16).to(DEV)
    k = synth.random_tensor((2, S, Hkv, D), 322 + S, torch.bfloat16).to(DEV)
    v = synth.random_tensor((2, S, Hkv, D), 323 + S, torch.bfloat16).to(DEV)
    pk = [synth.random_tensor((1, p, Hkv, D), 324 + b, torch.bfloat16).to(DEV) if p else None for b, p in enumerate(P)]
    pv = [synth.random_tensor((p, Hkv, D), 326 + b, torch.bfloat16).to(DEV) if p else None for b, p in enumerate(P)]
    if blocks:
        q8, qs = nx.nxattn_quantize_fp8_blocks(q)
        k8, ks = nx.nxattn_quantize_fp8_blocks(k)
        pre = [nx.nxattn_quantize_fp8_blocks(x) if x is not None else (None, None) for x in pk]
        kw = dict(q_scales=qs, k_scales=ks, prefix_k_scales=[s_[0] if s_ is not None else None for _, s_ in pre])
        qe = ke = pke = None
    else:
        q8, qe = nx.nxattn_quantize_fp8(q)
        k8, ke = nx.nxattn_quantize_fp8(k)
        pre = [nx.nxattn_quantize_fp8(x) if x is not None else (None, None) for x in pk]
        # prefix exponents [B, Hkv]: row b from branch b's prefix (0 where there is none)
        pke = torch.zeros((2, Hkv), dtype=torch.int8, device=DEV)
        for b, (_, e) in enumerate(pre):
            if e is not None:
                pke[b] = e[0]
        kw = {}
    pk8 = [c[0] if c is not None else None for c, _ in pre]
    args = (q8, k8, qe, ke, v)
    o_ref = torch.empty_like(q)
    out_ref = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd_fp8(*args, o_ref, pk8, pv, pke, **kw)
    nx.nxattn_cfg_combine(o_ref[0], o_ref[1], out_ref, g)
    o_f = torch.full_like(q, float("nan"))
    out_f = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd_fp8(*args, o_f, pk8, pv, pke, cfg_out=out_f, guidance=g, **kw)
    out_n = torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_fwd_fp8(*args, None, pk8, pv, pke, cfg_out=out_n, guidance=g, **kw)
    torch.cuda.synchronize()
    assert same(o_f, o_ref), "branch outputs differ"
    assert same(out_f, out_ref), "combination differs from nxattn_cfg_combine of the branch outputs"
    assert same(out_n, out_ref), "combination without branch outputs differs"


@pytest.mark.parametrize("name,q_on_load", [("dit1k_fp8blk", False), ("dit1k_fp8blk", True), ("dit1k_fp8qk", False)])
def test_step_fp8_fused_cfg_equals_separate_pass(name, q_on_load):
    wl = synth.bench_workload(name)
    note(f"step {wl.name}{' (q quantized on load)' if q_on_load else ''}: guidance inside the attention call "
         f"against the separate pass")
    inp = synth.make_inputs(wl)
    sep = AttentionStep(wl, inp, fuse_cfg=False, q_on_load=q_on_load)
    out_sep = sep().clone()
    o_sep = sep.o.clone()
    keep = AttentionStep(wl, inp, fuse_cfg=True, keep_branches=True, q_on_load=q_on_load)
    out_keep = keep().clone()
    lean = AttentionStep(wl, inp, fuse_cfg=True, keep_branches=False, q_on_load=q_on_load)
    out_lean = lean().clone()
    torch.cuda.synchronize()
    assert keep.fuse_cfg and lean.fuse_cfg
    assert same(keep.o, o_sep), "branch outputs differ"
    assert same(out_keep, out_sep), "combination differs (branch outputs stored)"
    assert same(out_lean, out_sep), "combination differs (no branch outputs)"


@pytest.mark.parametrize("blocks", [True, False])
def test_fwd_fp8_cfg_out_deterministic(blocks):
    S, Hq, Hkv = 300, 8, 2
    note(f"fwd_fp8 cfg_out determinism (blocks={blocks})")
    q = synth.random_tensor((2, S, Hq, D_FP8), 331, torch.bfloat16).to(DEV)
    k = synth.random_tensor((2, S, Hkv, D_FP8), 332, torch.bfloat16).to(DEV)
    v = synth.random_tensor((2, S, Hkv, D_FP8), 333, torch.bfloat16).to(DEV)
    pk = synth.random_tensor((1, 40, Hkv, D_FP8), 334, torch.bfloat16).to(DEV)
    pv = synth.random_tensor((40, Hkv, D_FP8), 335, torch.bfloat16).to(DEV)
    if blocks:
        q8, qs = nx.nxattn_quantize_fp8_blocks(q)
        k8, ks = nx.nxattn_quantize_fp8_blocks(k)
        pk8, pks = nx.nxattn_quantize_fp8_blocks(pk)
        args = (q8, k8, None, None, v)
        kw = dict(q_scales=qs, k_scales=ks, prefix_k_scales=[pks[0], None])
        pke = None
    else:
        q8, qe = nx.nxattn_quantize_fp8(q)
        k8, ke = nx.nxattn_quantize_fp8(k)
        pk8, pe = nx.nxattn_quantize_fp8(pk)
        args = (q8, k8, qe, ke, v)
        kw = {}
        pke = torch.zeros((2, Hkv), dtype=torch.int8, device=DEV)
        pke[0] = pe[0]
    outs = []
    for _ in range(3):
        out = torch.full((S, Hq, D_FP8), float("nan"), dtype=torch.bfloat16, device=DEV)
        nx.nxattn_fwd_fp8(*args, None, [pk8[0], None], [pv, None], pke, cfg_out=out, guidance=4.0, **kw)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0].float()).any()
    assert all(same(outs[0], o) for o in outs[1:])
