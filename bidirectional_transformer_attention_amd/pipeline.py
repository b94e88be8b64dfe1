"""One attention step of a DiT / ViT layer, chained from the four C-ABI calls.

    relayout (replay -> online, when the prefix arrives in the replay layout)
    -> RoPE on own k, and on own q unless the attention kernel rotates q as it loads it
       (the bf16 path; every branch with its own offsets)
    -> fused attention over [prefix ++ own] for all branches in one launch (or, with
       key splits, one launch over key ranges plus one merge launch)
    -> CFG combine of branch 0 (cond) and branch 1 (uncond) when guidance applies.
With the fp8 score GEMM (``qk_fp8`` workloads) q is rotated by the RoPE kernel too, and q,
own k and each prefix K are quantized to E4M3 before the attention call.

Only tensor allocation and argument marshalling happen here; every step runs in the HIP
library. The prefix of branch b is passed as one layer slice [2, P_b, Hkv, D] of the
online cache (NeoPP page, "KV file layout").
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import binding as nx
from .synth import Inputs, Workload


class AttentionStep:
    def __init__(self, wl: Workload, inp: Inputs, device: str = "cuda", fuse_q_rope: Optional[bool] = None,
                 splits: Optional[int] = None, fold_q: bool = True):
        self.wl = wl
        # fp8: q's codes carry softmax_scale*log2(e), so the attention's softmax takes one
        # exp2 per score with no multiply in front
        self.fold_q = bool(fold_q) and wl.qk_fp8
        self.splits = wl.splits if splits is None else int(splits)
        # bf16: q is rotated inside the attention kernel (no separate pass over q)
        self.fuse_q_rope = (wl.dtype == "bf16" and not wl.qk_fp8) if fuse_q_rope is None else bool(fuse_q_rope)
        if wl.qk_fp8 and self.fuse_q_rope:
            raise ValueError("the fp8 score GEMM takes q already rotated and quantized")
        dev = torch.device(device)
        self.q = inp.q.to(dev)
        self.k = inp.k.to(dev)
        self.v = inp.v.to(dev)
        self.B, self.S, self.Hq, self.D = self.q.shape
        self.Hkv = self.k.shape[2]
        # prefix as stored (replay [1,2,H,P,D] or online [2,P,H,D]) and the online buffers
        self.prefix_src: List[Optional[torch.Tensor]] = []
        self.prefix_online: List[Optional[torch.Tensor]] = []
        for p in inp.prefix:
            if p is None:
                self.prefix_src.append(None)
                self.prefix_online.append(None)
            elif wl.prefix_layout == "replay":
                src = p.to(dev).unsqueeze(0).contiguous()                 # [1, 2, H, P, D]
                self.prefix_src.append(src)
                self.prefix_online.append(torch.empty((2, src.shape[3], src.shape[2], src.shape[4]),
                                                      dtype=src.dtype, device=dev))
            else:
                on = p.to(dev).contiguous()                               # [2, P, H, D]
                self.prefix_src.append(None)
                self.prefix_online.append(on)
        self.descs = [nx.rope_desc(wl.grid, wl.pairs, wl.offsets[b], wl.theta) for b in range(self.B)]
        self.o = torch.empty_like(self.q)
        # workspace of the key-range partials, allocated once outside the step
        self.workspace = None
        if self.splits > 1:
            n = nx.fwd_workspace_bytes(self.B, self.S, self.Hq, self.D, self.splits)
            self.workspace = torch.empty(n, dtype=torch.uint8, device=dev)
        if wl.qk_fp8:
            # E4M3 codes, exponents and the quantizer's workspace, allocated once
            self.q8 = torch.empty(self.q.shape, dtype=torch.uint8, device=dev)
            self.k8 = torch.empty(self.k.shape, dtype=torch.uint8, device=dev)
            self.qe = torch.empty((self.B, self.Hq), dtype=torch.int8, device=dev)
            self.ke = torch.empty((self.B, self.Hkv), dtype=torch.int8, device=dev)
            self.pke = torch.zeros((self.B, self.Hkv), dtype=torch.int8, device=dev)
            self.pk8 = [None if p is None else torch.empty((1, p.shape[1], self.Hkv, self.D), dtype=torch.uint8,
                                                           device=dev) for p in self.prefix_online]
            plen = max([p.shape[1] for p in self.prefix_online if p is not None] + [1])
            n = max(nx.quantize_fp8_workspace_bytes(self.B, self.S, self.Hq + self.Hkv),
                    nx.quantize_fp8_workspace_bytes(1, plen, self.Hkv))
            self.qws = torch.empty(max(4, n), dtype=torch.uint8, device=dev)
        self.use_cfg = self.B == 2 and wl.guidance > 1.0
        self.out = torch.empty_like(self.q[0]) if self.use_cfg else None

    def relayout(self) -> None:
        for src, dst in zip(self.prefix_src, self.prefix_online):
            if src is not None:
                nx.nxattn_kv_relayout(src, dst.unsqueeze(0), 0)

    def rope(self) -> None:
        if self.wl.qk_fp8:
            return                      # rotated inside quantize(): only the codes are needed
        if not self.fuse_q_rope:
            nx.nxattn_rope_apply(self.q, self.descs)
        nx.nxattn_rope_apply(self.k, self.descs)

    def quantize(self) -> None:
        """E4M3 codes of the rotated q and k (one call for both: the rotation evaluated
        inside the quantizer's passes, q and k left as given) and of each prefix K (fp8
        workloads only)."""
        if not self.wl.qk_fp8:
            return
        nx.nxattn_rope_quantize_fp8([self.q, self.k], self.descs, [self.q8, self.k8], [self.qe, self.ke], self.qws,
                                    mults=[nx.fold_factor(self.D) if self.fold_q else 0.0, 0.0])
        for b, p in enumerate(self.prefix_online):
            if p is not None:
                nx.nxattn_quantize_fp8(p[0].unsqueeze(0), self.pk8[b], self.pke[b:b + 1], self.qws)

    def attention(self) -> None:
        if self.wl.qk_fp8:
            nx.nxattn_fwd_fp8(self.q8, self.k8, self.qe, self.ke, self.v, self.o,
                              [None if p is None else p[0] for p in self.pk8],
                              [None if p is None else p[1] for p in self.prefix_online],
                              self.pke if any(p is not None for p in self.prefix_online) else None,
                              q_folded=self.fold_q)
            return
        nx.nxattn_fwd(self.q, self.k, self.v, self.o, self.prefix_online,
                      q_rope=self.descs if self.fuse_q_rope else None,
                      num_splits=self.splits, workspace=self.workspace)

    def cfg(self) -> None:
        if self.use_cfg:
            nx.nxattn_cfg_combine(self.o[0], self.o[1], self.out, self.wl.guidance)

    def __call__(self) -> torch.Tensor:
        self.relayout()
        self.rope()
        self.quantize()
        self.attention()
        self.cfg()
        return self.out if self.use_cfg else self.o
