"""The RoPE of k and the prefix relayouts in one launch (nxattn_rope_apply_relayout): bit for
bit the separate calls, nxattn_rope_apply and one nxattn_kv_relayout per job (NeoPP page,
"KV file layout"; KLiteInfer page, "架构": the RoPE operators). The separate calls are held
to the oracle by the parity tests."""
import sys

import pytest
import torch

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from bidirectional_transformer_attention_amd.pipeline import AttentionStep

pytestmark = pytest.mark.gpu
DEV = "cuda"


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


def relayout_pair(shape_replay, direction, seed, dtype):
    """(src, dst) tensors of one job: direction 0 takes replay [L,2,H,S,D] to online, 1 the
    inverse."""
    L, _, H, S, D = shape_replay
    src_shape = shape_replay if direction == 0 else (L, 2, S, H, D)
    dst_shape = (L, 2, S, H, D) if direction == 0 else shape_replay
    src = synth.random_tensor(src_shape, seed, dtype).to(DEV)
    return src, torch.full(dst_shape, float("nan"), dtype=dtype, device=DEV)


@pytest.mark.parametrize("dtype,B,S,H,D,jobs", [
    (torch.bfloat16, 2, 300, 8, 128, [((1, 2, 8, 512, 128), 0), ((1, 2, 8, 128, 128), 0)]),   # the 1K DiT's prefixes
    (torch.bfloat16, 2, 97, 3, 64, [((2, 2, 3, 33, 64), 1), ((1, 2, 3, 1, 64), 0), ((3, 2, 1, 70, 64), 0)]),
    (torch.float32, 1, 150, 4, 72, [((1, 2, 4, 40, 72), 0)]),
    (torch.bfloat16, 2, 64, 2, 128, []),                                                    # no jobs
    (torch.bfloat16, 2, 64, 2, 128, [((1, 2, 2, 0, 128), 0), ((1, 2, 2, 9, 128), 1)]),      # a zero-size job
])
def test_rope_relayout_equals_separate_calls(dtype, B, S, H, D, jobs):
    note(f"rope+relayout {dtype} B={B} S={S} H={H} D={D} jobs={[(s, d) for s, d in jobs]}")
    x0 = synth.random_tensor((B, S, H, D), 331 + S, dtype).to(DEV)
    descs = [nx.rope_desc((S,), (D // 2,), (13 * b,)) for b in range(B)]
    pairs = [relayout_pair(shp, d, 340 + i, dtype) for i, (shp, d) in enumerate(jobs)]
    # separate calls
    x_ref = x0.clone()
    nx.nxattn_rope_apply(x_ref, descs)
    refs = []
    for (src, dst), (_, d) in zip(pairs, jobs):
        r = torch.full_like(dst, float("nan"))
        if src.numel():
            nx.nxattn_kv_relayout(src, r, d)
        refs.append(r)
    # one launch
    x = x0.clone()
    nx.nxattn_rope_apply_relayout(x, descs, [(src, dst, d) for (src, dst), (_, d) in zip(pairs, jobs)])
    torch.cuda.synchronize()
    assert same(x, x_ref), "rotation differs"
    for i, ((_, dst), r) in enumerate(zip(pairs, refs)):
        assert torch.equal(torch.isnan(dst.float()), torch.isnan(r.float())) and same(dst.nan_to_num(0), r.nan_to_num(0)), \
            f"job {i} differs"


def test_rope_relayout_jobs_alone():
    # no rotation work (batch 0): the jobs still run
    note("relayout jobs without rotation work")
    src, dst = relayout_pair((1, 2, 8, 128, 128), 0, 351, torch.bfloat16)
    ref = torch.empty_like(dst)
    nx.nxattn_kv_relayout(src, ref, 0)
    x = torch.empty((0, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    nx.nxattn_rope_apply_relayout(x, [], [(src, dst, 0)])
    torch.cuda.synchronize()
    assert same(dst, ref)


@pytest.mark.parametrize("name", ["dit1k_bf16", "video_bf16", "longctx_bf16"])
def test_step_fused_prep_equals_separate_calls(name):
    wl = synth.bench_workload(name)
    note(f"step {wl.name}: relayouts in the RoPE launch against separate calls")
    inp = synth.make_inputs(wl)
    sep = AttentionStep(wl, inp, fuse_prep=False)
    out_sep = sep().clone()
    fused = AttentionStep(wl, inp, fuse_prep=True)
    out_f = fused().clone()
    torch.cuda.synchronize()
    assert fused.fuse_prep and not sep.fuse_prep
    assert same(fused.k, sep.k), "rotated k differs"
    for a, b in zip(fused.prefix_online, sep.prefix_online):
        if a is not None:
            assert same(a, b), "relaid prefix differs"
    assert same(out_f, out_sep), "step output differs"
