"""Seeded synthetic inputs for the attention hot path (input generation only).

This module draws random tensors and records the workload shapes. It holds none of
the method's arithmetic: no positions, no rotation, no softmax. Both the HIP path
and the CPU oracle consume what it produces, so the two sides read identical bytes.

Workloads (their shapes stand in for data that is not available: KV dumps, images,
checkpoints):

* ``tiny_f32``   fp32 MHA, 1 branch, 2 heads, D 64, 64 own tokens, 32 prefix tokens,
                 1-D RoPE at offset 32, q/k/v ~ N(0,1).
* ``vit_f32``    fp32 bidirectional self-attention of a 27-layer vision encoder:
                 3900 tokens on a 60x65 patch grid, 2-D RoPE, 16 heads, D 72, no
                 prefix, values ~ N(0,1)*0.5, one independent seed per layer
                 (KLiteInfer page, "精度与性能" perf table: book.jpg, 3900 patches).
* ``dit1k_bf16`` 1024x1024 text-to-image DiT step: 64x64 latent grid (4096 tokens),
                 2-D RoPE offset by 512, 32 q / 8 kv heads, D 128, two CFG branches
                 with prefixes of 512 (cond) and 128 (uncond) tokens, guidance 4.0
                 (NeoPP page, "KV file layout" and "Shell launchers").
* ``dit2k_bf16`` 2048x2048 DiT step: 128x128 grid (16384 tokens), prefixes 1024 /
                 128, offset 1024, prefix supplied in the replay layout [2,H,S,D].
* ``video_bf16`` video DiT step: 21 latent frames x 30x52 patches (32760 tokens),
                 3-D RoPE (t,h,w), 12 heads, D 128, prefixes of 256, guidance 6.0
                 (LingBot-Video page, "Key Parameters": multiples of 16, 4n+1 frames).
* ``longctx_bf16`` a short query against a long conditioning prefix: 32x32 latent
                 grid (1024 tokens) with 2-D RoPE offset by 16384, 32 q / 8 kv heads,
                 D 128, prefixes of 16384 (cond) and 256 (uncond) tokens, guidance
                 4.0. Not one of the pages' measured shapes: it stands for a DiT
                 conditioned on a long injected KV cache (NeoPP page, intro), where one
                 workgroup per query block leaves most of the GPU idle; the step splits
                 the keys into 2 ranges.
* ``dit1k_fp8qk``, ``dit2k_fp8qk`` the 1K and 2K DiT steps (same shapes and seeds) with
                 q and k quantized each step to FP8 E4M3 for the score GEMM (the pages
                 name fp8 DiT variants, NeoPP "Run the replay examples"), one scale per
                 (branch, head).
* ``dit1k_fp8blk``, ``dit2k_fp8blk`` the same with one scale per run of 32 head_dim
                 elements of each row.

Seeds: ``1_000_000*c + 1000*layer + 10*branch + t`` with t = 0 q, 1 own k, 2 own v,
3 prefix k, 4 prefix v; values drawn in fp32 on the CPU with ``torch.Generator`` and
cast (round-to-nearest-even) to bf16 where the workload is bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import torch

T_Q, T_K, T_V, T_PK, T_PV = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cid: int                      # seed namespace of the workload
    dtype: str                    # "f32" or "bf16"
    branches: int                 # CFG branches (batch of the attention call)
    grid: Tuple[int, ...]         # own-token grid, row-major, axis 0 slowest
    pairs: Tuple[int, ...]        # rotary pairs per axis (sum = head_dim / 2)
    offsets: Tuple[Tuple[int, ...], ...]   # per branch, per axis position offset
    prefix_len: Tuple[int, ...]   # per branch conditioning prefix length
    heads_q: int
    heads_kv: int
    head_dim: int
    value_scale: float = 1.0
    layers: int = 1
    guidance: float = 1.0
    prefix_layout: str = "online"  # "online" [2,P,H,D] or "replay" [2,H,P,D]
    theta: float = 10000.0
    splits: int = 0               # key ranges per branch in the attention call (0: one pass)
    qk_fp8: bool = False          # q and k quantized to E4M3 for the score GEMM (bf16 tensors in)
    fp8_blocks: bool = False      # qk_fp8 with one scale per 32-element run instead of per head

    @property
    def seq(self) -> int:
        n = 1
        for g in self.grid:
            n *= g
        return n

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def flops(self, branches: Optional[List[int]] = None) -> float:
        """Attention flops 4*Sq*Skv*Hq*D summed over the given branches."""
        bs = range(self.branches) if branches is None else branches
        return float(sum(4 * self.seq * (self.prefix_len[b] + self.seq) * self.heads_q * self.head_dim
                         for b in bs))


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, "f32", 1, (64,), (32,), ((32,),), (32,), 2, 2, 64),
    "vit_f32": Workload("vit_f32", 2, "f32", 1, (60, 65), (18, 18), ((0, 0),), (0,), 16, 16, 72,
                        value_scale=0.5, layers=27),
    "dit1k_bf16": Workload("dit1k_bf16", 3, "bf16", 2, (64, 64), (32, 32), ((512, 512), (512, 512)),
                           (512, 128), 32, 8, 128, guidance=4.0),
    "dit2k_bf16": Workload("dit2k_bf16", 4, "bf16", 2, (128, 128), (32, 32), ((1024, 1024), (1024, 1024)),
                           (1024, 128), 32, 8, 128, guidance=4.0, prefix_layout="replay"),
    "video_bf16": Workload("video_bf16", 5, "bf16", 2, (21, 30, 52), (22, 21, 21), ((0, 0, 0), (0, 0, 0)),
                           (256, 256), 12, 12, 128, guidance=6.0),
    "longctx_bf16": Workload("longctx_bf16", 6, "bf16", 2, (32, 32), (32, 32), ((16384, 16384), (16384, 16384)),
                             (16384, 256), 32, 8, 128, guidance=4.0, splits=2),
}
# the DiT steps with the fp8 score GEMM: same shapes and seeds, q and k quantized each step
# with one scale per (branch, head) (fp8qk) or per run of 32 head_dim elements (fp8blk)
for _n in ("dit1k_bf16", "dit2k_bf16"):
    _w = WORKLOADS[_n]
    WORKLOADS[_n.replace("bf16", "fp8qk")] = dataclasses.replace(_w, name=_n.replace("bf16", "fp8qk"), qk_fp8=True)
    WORKLOADS[_n.replace("bf16", "fp8blk")] = dataclasses.replace(_w, name=_n.replace("bf16", "fp8blk"), qk_fp8=True,
                                                                  fp8_blocks=True)


def bench_workload(name: str) -> Workload:
    """The timed configuration of a workload: its prefix arrives in the replay layout
    [2, H, P, D] (as the KV-replay path loads it), so every step also relays it."""
    wl = WORKLOADS[name]
    if any(p > 0 for p in wl.prefix_len) and wl.prefix_layout != "replay":
        wl = dataclasses.replace(wl, name=wl.name + "+replay", prefix_layout="replay")
    return wl


def seed_of(cid: int, layer: int, branch: int, tensor: int) -> int:
    return 1_000_000 * cid + 1000 * layer + 10 * branch + tensor


def draw(shape, seed: int, scale: float = 1.0, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """N(0,1)*scale drawn in fp32 on the CPU from a seeded generator, cast to dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


@dataclasses.dataclass
class Inputs:
    """One layer of one workload, on the CPU.

    q [B,Sq,Hq,D]; k, v [B,Sq,Hkv,D] (own tokens); prefix[b] is [2,P_b,Hkv,D] in the
    online layout (K at index 0, V at index 1) or [2,Hkv,P_b,D] in the replay layout,
    or None when P_b == 0.
    """
    wl: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    prefix: List[Optional[torch.Tensor]]


def make_inputs(wl: Workload, layer: int = 0, seq: Optional[int] = None,
                prefix_len: Optional[Tuple[int, ...]] = None, heads_q: Optional[int] = None,
                heads_kv: Optional[int] = None, value_scale: Optional[float] = None) -> Inputs:
    """Seeded inputs of a workload; sizes may be overridden for reduced parity cases."""
    S = wl.seq if seq is None else seq
    P = wl.prefix_len if prefix_len is None else prefix_len
    Hq = wl.heads_q if heads_q is None else heads_q
    Hkv = wl.heads_kv if heads_kv is None else heads_kv
    sc = wl.value_scale if value_scale is None else value_scale
    D = wl.head_dim
    dt = wl.torch_dtype
    B = wl.branches
    qs, ks, vs, pre = [], [], [], []
    for b in range(B):
        qs.append(draw((S, Hq, D), seed_of(wl.cid, layer, b, T_Q), sc, dt))
        ks.append(draw((S, Hkv, D), seed_of(wl.cid, layer, b, T_K), sc, dt))
        vs.append(draw((S, Hkv, D), seed_of(wl.cid, layer, b, T_V), sc, dt))
        if P[b] == 0:
            pre.append(None)
            continue
        shp = (P[b], Hkv, D) if wl.prefix_layout == "online" else (Hkv, P[b], D)
        pk = draw(shp, seed_of(wl.cid, layer, b, T_PK), sc, dt)
        pv = draw(shp, seed_of(wl.cid, layer, b, T_PV), sc, dt)
        pre.append(torch.stack([pk, pv], 0).contiguous())
    return Inputs(wl, torch.stack(qs, 0).contiguous(), torch.stack(ks, 0).contiguous(),
                  torch.stack(vs, 0).contiguous(), pre)


def random_tensor(shape, seed: int, dtype: torch.dtype = torch.float32, scale: float = 1.0) -> torch.Tensor:
    """A seeded N(0,1)*scale tensor of any shape (used by reduced and edge-case tests)."""
    return draw(shape, seed, scale, dtype)
