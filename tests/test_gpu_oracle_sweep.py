"""Seeded random sweeps against the CPU fp64 oracle, through the C ABI: nxattn_fwd over random
shapes and option mixes (KLiteInfer page, "架构": softmax(q k^T / sqrt(d)) v over the keys
[prefix ++ own]; NeoPP page: conditioning KV prefixes, split key ranges), and
nxattn_rope_apply over random grids, pair splits and offsets (KLiteInfer page, "架构":
RoPE / 2-D RoPE / MRoPE). Gates: the attention gate (1e-4 fp32, 2e-2 bf16, max slice error),
the log-sum-exp bound 1e-3 + 1e-4 |lse|, RoPE within one bf16 rounding (2^-8) or 2e-6 (fp32).
With q rotated on load the reference q is the oracle's rotation rounded once at the
kernel's documented point (times scale * log2 e, to bf16). Each case prints its
parameters before it runs."""
import sys

import numpy as np
import pytest
import torch

import oracle
import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth
from helpers import TOL, attention_err, f64, fused_q, lse_err_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    nx.load()


def fwd_case(i):
    rng = np.random.default_rng(9100 + i)
    bf16 = i % 4 != 3
    B = int(rng.integers(1, 4))
    S = int(rng.integers(1, 400))
    Hkv = int(rng.choice([1, 2, 3, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    D = 128 if bf16 else int(rng.choice([64, 72]))
    P = tuple(int(rng.integers(1, 300)) if rng.random() < 0.7 else 0 for _ in range(B))
    prefix_only = all(p > 0 for p in P) and rng.random() < 0.2
    return dict(bf16=bf16, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, P=P, prefix_only=bool(prefix_only),
                lse=bool(rng.random() < 0.5), splits=int(rng.choice([0, 0, 2, 3, 5])),
                rope=bool(bf16 and rng.random() < 0.5), offsets=tuple(int(rng.integers(0, 8000)) for _ in range(B)))


@pytest.mark.parametrize("i", range(20))
def test_fwd_oracle_sweep(i):
    c = fwd_case(i)
    note(f"fwd oracle sweep {i}: {c}")
    dtype = torch.bfloat16 if c["bf16"] else torch.float32
    B, S, Hq, Hkv, D, P = c["B"], c["S"], c["Hq"], c["Hkv"], c["D"], c["P"]
    q = synth.random_tensor((B, S, Hq, D), 9200 + i, dtype)
    k = synth.random_tensor((B, S, Hkv, D), 9300 + i, dtype)
    v = synth.random_tensor((B, S, Hkv, D), 9400 + i, dtype)
    pre = [synth.random_tensor((2, p, Hkv, D), 9500 + 4 * i + b, dtype) if p else None for b, p in enumerate(P)]
    descs = [nx.rope_desc((S,), (64,), (c["offsets"][b],), 10000.0) for b in range(B)] if c["rope"] else None
    o = torch.full((B, S, Hq, D), float("nan"), dtype=dtype, device=DEV)
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV) if c["lse"] else None
    own = (None, None) if c["prefix_only"] else (k.to(DEV), v.to(DEV))
    nx.nxattn_fwd(q.to(DEV), *own, o, [p.to(DEV) if p is not None else None for p in pre], q_rope=descs,
                  lse=lse, prefix_only=c["prefix_only"], num_splits=c["splits"])
    torch.cuda.synchronize()
    tol = TOL["bf16" if c["bf16"] else "f32"]
    got = f64(o.cpu())
    for b in range(B):
        qx = fused_q(oracle.rope(f64(q[b]), (S,), (64,), (c["offsets"][b],), 10000.0), D) if c["rope"] else f64(q[b])
        pk = f64(pre[b][0]) if pre[b] is not None else None
        pv = f64(pre[b][1]) if pre[b] is not None else None
        args = (qx, pk, pv) if c["prefix_only"] else (qx, f64(k[b]), f64(v[b]), pk, pv)
        ref = oracle.attention(*args)
        err = attention_err(got[b], ref)
        note(f"  branch {b}: error {err:.3e} (gate {tol:.0e})")
        assert err <= tol, (b, err)
        if lse is not None:
            rl = oracle.attention_lse(*args)
            assert lse_err_ok(f64(lse[b].cpu()), rl), (b, float(np.max(np.abs(f64(lse[b].cpu()) - rl))))


def pairs_of(rng, n, half):
    if n == 1:
        return (half,)
    cuts = sorted(int(x) for x in rng.choice(np.arange(1, half), size=n - 1, replace=False))
    edges = [0, *cuts, half]
    return tuple(edges[j + 1] - edges[j] for j in range(n))


@pytest.mark.parametrize("i", range(12))
def test_rope_oracle_sweep(i):
    rng = np.random.default_rng(9600 + i)
    dtype = torch.bfloat16 if i % 3 != 2 else torch.float32
    n = int(rng.integers(1, 4))
    grid = tuple(int(rng.integers(1, 400 if n == 1 else (28 if n == 2 else 9))) for _ in range(n))
    D = int(rng.choice([64, 128]))
    pairs = pairs_of(rng, n, D // 2)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 7))
    inter, gf = bool(rng.random() < 0.3), bool(rng.random() < 0.2)
    theta = float(rng.choice([10000.0, 1000000.0]))
    offs = [tuple(int(rng.integers(0, 20000)) for _ in grid) for _ in range(B)]
    note(f"rope oracle sweep {i}: {dtype} B={B} grid={grid} pairs={pairs} H={H} D={D} theta={theta} "
         f"interleaved={inter} global={gf} offsets={offs}")
    S = int(np.prod(grid))
    x = synth.random_tensor((B, S, H, D), 9700 + i, dtype)
    d = x.to(DEV)
    nx.nxattn_rope_apply(d, [nx.rope_desc(grid, pairs, offs[b], theta, inter, gf) for b in range(B)])
    torch.cuda.synchronize()
    out = f64(d.cpu())
    tol = 2.0 ** -8 if dtype == torch.bfloat16 else 2e-6
    for b in range(B):
        ref = oracle.rope(f64(x[b]), grid, pairs, offs[b], theta, interleaved=inter, global_freq=gf)
        err = attention_err(out[b], ref)
        assert err <= tol, (b, err)
