"""GPU parity of the log-sum-exp output, prefix-only keys, split key ranges and the merge
of attention over disjoint key sets, through the C ABI, against the CPU fp64 oracle.

Bars: the attention gate (max slice error 1e-4 fp32 / 2e-2 bf16) for outputs; the
log-sum-exp within 1e-3 + 1e-4*|lse| (natural log) of the oracle's; the merge alone
within its fp32 arithmetic plus one output rounding.
"""
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


def make_case(dtype, B, S, Hq, Hkv, D, plens, seed, scale_v=1.0):
    q = synth.random_tensor((B, S, Hq, D), seed, dtype, scale_v)
    k = synth.random_tensor((B, S, Hkv, D), seed + 1, dtype, scale_v)
    v = synth.random_tensor((B, S, Hkv, D), seed + 2, dtype, scale_v)
    pre = [synth.random_tensor((2, p, Hkv, D), seed + 3 + b, dtype, scale_v) if p else None
           for b, p in enumerate(plens)]
    return q, k, v, pre


def oracle_ref(q, k, v, pre, b, prefix_only=False, rows=None):
    """(o [R, Hq, D], lse [Hq, R]) of branch b over [prefix ++ own], or the prefix alone."""
    pk = f64(pre[b][0]) if pre[b] is not None else None
    pv = f64(pre[b][1]) if pre[b] is not None else None
    if prefix_only:
        args = (f64(q[b]), pk, pv)
    else:
        args = (f64(q[b]), f64(k[b]), f64(v[b]), pk, pv)
    return oracle.attention(*args, rows=rows), oracle.attention_lse(*args, rows=rows)


def check(o, lse, q, k, v, pre, dtype, prefix_only=False):
    tol = TOL["bf16" if dtype == torch.bfloat16 else "f32"]
    for b in range(q.shape[0]):
        ro, rl = oracle_ref(q, k, v, pre, b, prefix_only)
        err = attention_err(f64(o[b]), ro)
        assert err <= tol, (b, err)
        if lse is not None:
            lerr = float(np.max(np.abs(f64(lse[b]) - rl)))
            assert lse_err_ok(f64(lse[b]), rl), (b, lerr)


def dev(*ts):
    return [t.to(DEV) if t is not None else None for t in ts]


BF16_CASES = [
    (2, 300, 8, 2, (37, 0)),      # ragged Sq, straddling prefix, a branch without prefix
    (1, 1, 8, 1, (200,)),         # one own token, long prefix
    (2, 640, 8, 2, (128, 200)),   # whole prefix tiles, then a straddling one
    (3, 70, 2, 1, (5, 0, 64)),
]
F32_CASES = [
    (2, 97, 3, 3, 72, (13, 64)),
    (1, 300, 4, 2, 64, (0,)),
]


def _all_cases():
    for c in BF16_CASES:
        yield (torch.bfloat16,) + c[:4] + (128,) + c[4:]
    for c in F32_CASES:
        yield (torch.float32,) + c


@pytest.mark.parametrize("dtype,B,S,Hq,Hkv,D,P", list(_all_cases()))
def test_fwd_lse(dtype, B, S, Hq, Hkv, D, P):
    note(f"fwd lse {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} P={P}")
    q, k, v, pre = make_case(dtype, B, S, Hq, Hkv, D, P, 3000 + S)
    dq, dk, dv = dev(q, k, v)
    o = torch.empty_like(dq)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    nx.nxattn_fwd(dq, dk, dv, o, dev(*pre), lse=lse)
    torch.cuda.synchronize()
    check(o.cpu(), lse.cpu(), q, k, v, pre, dtype)
    # with lse the output is the one of a call without it, bit for bit
    o2 = torch.empty_like(dq)
    nx.nxattn_fwd(dq, dk, dv, o2, dev(*pre))
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o2.cpu())


@pytest.mark.parametrize("dtype,D,P", [(torch.bfloat16, 128, (1, 64, 200)), (torch.float32, 72, (130, 7, 64))])
def test_fwd_prefix_only(dtype, D, P):
    note(f"fwd prefix_only {dtype} P={P}")
    B, S, Hq, Hkv = len(P), 150, 8, 2
    q, k, v, pre = make_case(dtype, B, S, Hq, Hkv, D, P, 3100)
    dq, = dev(q)
    o = torch.empty_like(dq)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    nx.nxattn_fwd(dq, None, None, o, dev(*pre), lse=lse, prefix_only=True)
    torch.cuda.synchronize()
    check(o.cpu(), lse.cpu(), q, k, v, pre, dtype, prefix_only=True)


SPLIT_CASES = [
    # dtype, B, S, Hq, Hkv, D, P, splits
    (torch.bfloat16, 2, 300, 8, 2, 128, (37, 0), 2),
    (torch.bfloat16, 2, 300, 8, 2, 128, (37, 0), 16),     # more splits than tiles: 1-tile ranges
    (torch.bfloat16, 2, 200, 4, 2, 128, (1000, 7), 3),    # long vs short branch: uneven range counts
    (torch.bfloat16, 1, 1, 8, 1, 128, (200,), 4),         # one own token
    (torch.bfloat16, 3, 70, 2, 1, 128, (5, 0, 64), 5),
    (torch.float32, 2, 97, 3, 3, 72, (13, 640), 4),
    (torch.float32, 1, 64, 2, 2, 64, (32,), 2),
    # the most branches and the most key ranges a call takes
    (torch.bfloat16, 8, 60, 4, 1, 128, (0, 300, 64, 1, 129, 700, 5, 40), 16),
    (torch.float32, 8, 33, 2, 2, 64, (900, 0, 3, 64, 65, 2, 31, 200), 16),
]


@pytest.mark.parametrize("dtype,B,S,Hq,Hkv,D,P,ns", SPLIT_CASES)
def test_fwd_split_keys(dtype, B, S, Hq, Hkv, D, P, ns):
    note(f"fwd split {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} P={P} splits={ns}")
    q, k, v, pre = make_case(dtype, B, S, Hq, Hkv, D, P, 3200 + S + ns)
    dq, dk, dv = dev(q, k, v)
    o = torch.empty_like(dq)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    ws = torch.empty(nx.fwd_workspace_bytes(B, S, Hq, D, ns), dtype=torch.uint8, device=DEV)
    ws.fill_(0xff)                                        # contents on entry must not matter
    nx.nxattn_fwd(dq, dk, dv, o, dev(*pre), lse=lse, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    check(o.cpu(), lse.cpu(), q, k, v, pre, dtype)
    # without the lse output, the same o
    o2 = torch.empty_like(dq)
    nx.nxattn_fwd(dq, dk, dv, o2, dev(*pre), num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o2.cpu())


def test_split_request_on_a_full_problem_is_one_pass():
    # a problem that already fills the GPU: the ranges would be shorter than a fair
    # share, so the call runs as one pass and matches the plain call bit for bit
    note("fwd split request on a full-size problem")
    B, S, Hq, Hkv, D, P = 2, 4096, 32, 8, 128, (512, 128)
    q, k, v, pre = make_case(torch.bfloat16, B, S, Hq, Hkv, D, P, 3250)
    dq, dk, dv = dev(q, k, v)
    dp = dev(*pre)
    o1, o2 = torch.empty_like(dq), torch.empty_like(dq)
    nx.nxattn_fwd(dq, dk, dv, o1, dp)
    nx.nxattn_fwd(dq, dk, dv, o2, dp, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2.cpu())


def test_fwd_split_with_q_rope_and_prefix_only():
    # every option at once: q rotated on load, keys = prefix only, split ranges, lse
    note("fwd split + q_rope + prefix_only")
    B, S, Hq, Hkv, D, P = 2, 96, 8, 2, 128, (700, 65)
    q, k, v, pre = make_case(torch.bfloat16, B, S, Hq, Hkv, D, P, 3300)
    descs = [nx.rope_desc((8, 12), (32, 32), (P[b], P[b])) for b in range(B)]
    q_rot = torch.stack([torch.from_numpy(fused_q(oracle.rope(f64(q[b]), (8, 12), (32, 32), (P[b], P[b])), D))
                         for b in range(B)])
    dq, = dev(q)
    o = torch.empty_like(dq)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    nx.nxattn_fwd(dq, None, None, o, dev(*pre), q_rope=descs, lse=lse, prefix_only=True, num_splits=6)
    torch.cuda.synchronize()
    # the isolation reference: the oracle's rotation, rounded at the kernel's documented point
    check(o.cpu(), lse.cpu(), q_rot, k, v, pre, torch.bfloat16, prefix_only=True)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_merge_of_separate_calls(dtype, D):
    # own keys in one call, the prefix in another (prefix_only), merged: the full result
    note(f"merge of own-only and prefix-only calls {dtype}")
    B, S, Hq, Hkv, P = 2, 200, 8, 2, (300, 77)
    q, k, v, pre = make_case(dtype, B, S, Hq, Hkv, D, P, 3400)
    dq, dk, dv = dev(q, k, v)
    o_own, o_pre = torch.empty_like(dq), torch.empty_like(dq)
    l_own = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    l_pre = torch.empty_like(l_own)
    nx.nxattn_fwd(dq, dk, dv, o_own, [], lse=l_own)
    nx.nxattn_fwd(dq, None, None, o_pre, dev(*pre), lse=l_pre, prefix_only=True)
    o = torch.empty_like(dq)
    lse = torch.empty_like(l_own)
    nx.nxattn_attn_merge([o_own, o_pre], [l_own, l_pre], o, lse)
    torch.cuda.synchronize()
    # bf16: each part is rounded once before the merge rounds again
    check(o.cpu(), lse.cpu(), q, k, v, pre, dtype)
    # in place: the result accumulates into the first part
    nx.nxattn_attn_merge([o_own, o_pre], [l_own, l_pre], o_own, l_own)
    torch.cuda.synchronize()
    assert torch.equal(o_own.cpu(), o.cpu()) and torch.equal(l_own.cpu(), lse.cpu())


@pytest.mark.parametrize("dtype,D,n", [(torch.bfloat16, 128, 3), (torch.float32, 72, 16), (torch.float32, 64, 1)])
def test_merge_matches_oracle(dtype, D, n):
    note(f"merge alone {dtype} D={D} parts={n}")
    B, S, H = 2, 77, 5
    rng = np.random.default_rng(3500 + n)
    parts = [synth.random_tensor((B, S, H, D), 3500 + p, dtype) for p in range(n)]
    lses = [torch.from_numpy(rng.normal(0.0, 3.0, (B, H, S))).to(torch.float32) for _ in range(n)]
    if n > 1:
        # empty parts: lse = -inf, output NaN (must be ignored)
        mask = torch.from_numpy(rng.random((B, H, S)) < 0.3)
        lses[1][mask] = -float("inf")
        parts[1] = parts[1].clone()
        parts[1].permute(0, 2, 1, 3)[mask] = float("nan")
    o = torch.empty((B, S, H, D), dtype=dtype, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    nx.nxattn_attn_merge(dev(*parts), dev(*lses), o, lse)
    torch.cuda.synchronize()
    go, gl = f64(o.cpu()), f64(lse.cpu())
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    rnd = 2.0 ** -8 if dtype == torch.bfloat16 else 1e-6
    for b in range(B):
        ro, rl = oracle.merge_partials([f64(p[b]) for p in parts], [f64(x[b]) for x in lses])
        bound = max(float(np.nanmax(np.abs(f64(p[b])))) for p in parts)
        assert np.all(np.abs(go[b] - ro) <= rnd * np.abs(ro) + 1e-6 * bound)
        assert np.max(np.abs(gl[b] - rl)) <= 1e-5 * max(1.0, float(np.max(np.abs(rl))))


def test_merge_strided_views():
    note("merge strided views")
    B, S, H, D = 1, 40, 6, 128
    big = [synth.random_tensor((B, S, H + 2, D), 3600 + p, torch.bfloat16).to(DEV) for p in range(2)]
    parts = [t[:, :, 1:H + 1] for t in big]
    lses = [torch.randn((B, H, S), generator=torch.Generator().manual_seed(3610 + p)).to(DEV) for p in range(2)]
    out_big = torch.zeros((B, S, H + 3, D), dtype=torch.bfloat16, device=DEV)
    o = out_big[:, :, 2:H + 2]
    nx.nxattn_attn_merge(parts, lses, o)
    torch.cuda.synchronize()
    ro, _ = oracle.merge_partials([f64(p[0]) for p in parts], [f64(x[0]) for x in lses])
    assert np.all(np.abs(f64(o[0]) - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-5)
    ob = out_big.cpu()
    assert torch.all(ob[:, :, :2] == 0) and torch.all(ob[:, :, H + 2:] == 0)
