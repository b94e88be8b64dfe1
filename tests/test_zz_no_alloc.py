"""The no-allocation entry point (nxattn_rope_quantize_fp8_noalloc) against the plain one
(nxattn_rope_quantize_fp8 with a caller's workspace): the same codes and exponents bit for
bit, on two calls in a row on the library's static scratch, the second with a smaller
input whose values are far smaller (maxima left over from the first call would change its
exponents)."""
import sys

import numpy as np
import pytest
import torch

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def _case(B, grid, pairs, heads, D, seed, scale, dtype):
    S = int(np.prod(grid))
    xs = [(synth.random_tensor((B, S, H, D), seed + t, torch.float32) * scale).to(dtype).to(DEV)
          for t, H in enumerate(heads)]
    descs = [nx.rope_desc(grid, pairs, tuple(5 * b + a for a in range(len(grid)))) for b in range(B)]
    return xs, descs


def _both(xs, descs, folds):
    ref = nx.nxattn_rope_quantize_fp8(xs, descs, folds=folds)
    codes = [torch.full(x.shape, 0x55, dtype=torch.uint8, device=DEV) for x in xs]
    exps = [torch.full((x.shape[0], x.shape[2]), 99, dtype=torch.int8, device=DEV) for x in xs]
    got = nx.nxattn_rope_quantize_fp8_noalloc(xs, descs, codes, exps, folds=folds)
    torch.cuda.synchronize()
    for (rc, re), (gc, ge) in zip(ref, got):
        assert torch.equal(ge.cpu(), re.cpu())
        assert torch.equal(gc.cpu(), rc.cpu())
    return got


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call_twice(dtype):
    note(f"rope+quantize fp8 without allocation {dtype}: a large call, then a smaller one")
    xs, descs = _case(2, (48, 64), (32, 32), (32, 8), 128, 4700, 1.0, dtype)
    _both(xs, descs, [True, False])
    # the second call: fewer slices and values 1e-3 of the first call's
    xs2, descs2 = _case(1, (5, 7, 9), (16, 24, 24), (3, 1), 128, 4710, 1e-3, dtype)
    got = _both(xs2, descs2, [False, True])
    assert int(got[0][1].cpu().max()) < 0            # exponents of the small values, not stale ones


def test_noalloc_rejects_more_slices_than_its_scratch():
    note("rope+quantize fp8 without allocation: too many (branch, head) slices")
    x = torch.zeros((8, 1, 257, 8), dtype=torch.bfloat16, device=DEV)       # 8 * 257 = 2056 > 2048 slices
    codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    exps = torch.empty((8, 257), dtype=torch.int8, device=DEV)
    with pytest.raises(nx.NxattnError) as ei:
        nx.nxattn_rope_quantize_fp8_noalloc([x], [nx.rope_desc((1,), (4,), (0,))] * 8, [codes], [exps])
    assert ei.value.status == 2 and "2048" in str(ei.value)
