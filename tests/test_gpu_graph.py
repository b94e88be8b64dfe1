"""The attention step captured as one HIP graph (what bench.py times): every replay gives,
bit for bit, the output of the same step run as eager launches, with eager work (restoring
the inputs a step rotates in place, poisoning the outputs) and synchronisations between
the replays. Nothing in a step may record a memset or allocate: a replay that skipped or
repeated a launch, or read a stale buffer, would differ."""
import sys

import pytest
import torch

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from bidirectional_transformer_attention_amd.pipeline import AttentionStep, capture_steps

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("name,q_on_load", [("dit1k_bf16", False), ("dit1k_fp8qk", False), ("dit1k_fp8blk", False),
                                             ("dit1k_fp8blk", True), ("longctx_bf16", False)])
def test_step_graph_replays_match_eager(name, q_on_load):
    wl = synth.bench_workload(name)
    note(f"step graph {wl.name}{' (q quantized on load)' if q_on_load else ''}: replays against the eager step")
    step = AttentionStep(wl, synth.make_inputs(wl), q_on_load=q_on_load)
    q0, k0 = step.q.clone(), step.k.clone()
    out = step()                                   # eager
    torch.cuda.synchronize()
    ref = out.clone()
    graph = step.capture()                         # its warm-up calls may rotate q, k again
    for i in range(3):
        step.q.copy_(q0)
        step.k.copy_(k0)
        out.fill_(float("nan"))
        step.o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), f"replay {i} differs from the eager step"
        _ = (step.o.float() * 2).sum().item()      # unrelated eager work between replays


def test_layers_graph_replays_match_eager():
    # two layers of the fp32 ViT step (each on its own inputs) recorded into one graph
    wl = synth.bench_workload("vit_f32")
    note("step graph vit_f32, two layers in one graph")
    steps = [AttentionStep(wl, synth.make_inputs(wl, layer=l)) for l in range(2)]
    q0 = [st.q.clone() for st in steps]
    k0 = [st.k.clone() for st in steps]
    refs = [st().clone() for st in steps]
    torch.cuda.synchronize()
    graph = capture_steps(steps)
    for i in range(3):
        for st, q, k in zip(steps, q0, k0):
            st.q.copy_(q)
            st.k.copy_(k)
            st.o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for st, r in zip(steps, refs):
            assert torch.equal(bits(st.o), bits(r)), f"replay {i} differs from the eager step"
