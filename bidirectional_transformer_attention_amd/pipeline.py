"""One attention step of a DiT / ViT layer, chained from the four C-ABI calls.

    relayout (replay -> online, when the prefix arrives in the replay layout)
    -> RoPE on own k, and on own q unless the attention kernel rotates q as it loads it
       (the bf16 path; every branch with its own offsets); the relayouts run as extra
       workgroups of the launch that rotates k (``fuse_prep``)
    -> fused attention over [prefix ++ own] for all branches in one launch (or, with
       key splits, one launch over key ranges plus one merge launch)
    -> CFG combine of branch 0 (cond) and branch 1 (uncond) when guidance applies: with
       one key range (bf16 or fp8 score GEMM), inside the attention call (each workgroup runs
       both branches of its query rows and writes the combination; ``keep_branches``
       also stores the branch outputs), else as a separate pass.
With the fp8 score GEMM (``qk_fp8`` workloads) q and own k are rotated and quantized to
E4M3 in one call before the attention call, with one scale per (branch, head) or, for
``fp8_blocks`` workloads, one per run of 32 head_dim elements (a single pass without a
workspace). With ``q_on_load`` (block scales only) that call quantizes only k and the
attention kernel rotates, folds and quantizes q as it loads it. Each prefix K is quantized once, when the step is set up: the
injected conditioning cache is the same for every denoising step (NeoPP page, intro), so
its codes are too.

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
                 splits: Optional[int] = None, fold_q: bool = True, q_on_load: bool = False,
                 fuse_cfg: Optional[bool] = None, keep_branches: bool = True, fuse_prep: Optional[bool] = None):
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
        self.blocks = wl.qk_fp8 and wl.fp8_blocks
        # block scaling only: q rotated, folded and quantized by the attention kernel as it
        # loads it (no q codes in memory) instead of by the quantize call
        self.q_on_load = bool(q_on_load) and self.blocks
        if wl.qk_fp8:
            # E4M3 codes, their exponents (per (branch, head)) or block scales (per run of
            # 32 elements, E8M0 codes) and the quantizer's workspace, allocated once
            self.q8 = None if self.q_on_load else torch.empty(self.q.shape, dtype=torch.uint8, device=dev)
            self.k8 = torch.empty(self.k.shape, dtype=torch.uint8, device=dev)
            self.pk8 = [None if p is None else torch.empty((1, p.shape[1], self.Hkv, self.D), dtype=torch.uint8,
                                                           device=dev) for p in self.prefix_online]
            if self.blocks:
                nb = self.D // 32
                self.qs = None if self.q_on_load else torch.empty((self.B, self.S, self.Hq, nb), dtype=torch.uint8,
                                                                  device=dev)
                self.ks = torch.empty((self.B, self.S, self.Hkv, nb), dtype=torch.uint8, device=dev)
                self.pks = [None if p is None else torch.empty((1, p.shape[1], self.Hkv, nb), dtype=torch.uint8,
                                                               device=dev) for p in self.prefix_online]
            else:
                self.qe = torch.empty((self.B, self.Hq), dtype=torch.int8, device=dev)
                self.ke = torch.empty((self.B, self.Hkv), dtype=torch.int8, device=dev)
                self.pke = torch.zeros((self.B, self.Hkv), dtype=torch.int8, device=dev)
                plen = max([p.shape[1] for p in self.prefix_online if p is not None] + [1])
                n = max(nx.quantize_fp8_workspace_bytes(self.B, self.S, self.Hq + self.Hkv),
                        nx.quantize_fp8_workspace_bytes(1, plen, self.Hkv))
                self.qws = torch.empty(max(4, n), dtype=torch.uint8, device=dev)
        self.use_cfg = self.B == 2 and wl.guidance > 1.0
        self.out = torch.empty_like(self.q[0]) if self.use_cfg else None
        # bf16 with one key range: the attention kernel serves both branches of its query
        # rows and writes the guidance combination itself (no combine pass); with
        # keep_branches it also stores the two branch outputs in o
        can_fuse = self.use_cfg and wl.dtype == "bf16" and self.splits <= 1
        self.fuse_cfg = can_fuse if fuse_cfg is None else bool(fuse_cfg)
        if self.fuse_cfg and not can_fuse:
            raise ValueError("the guidance combination folds into the bf16 / fp8 attention call with one key "
                             "range only")
        self.keep_branches = bool(keep_branches) or not self.fuse_cfg
        # the prefix relayouts ride in the launch that rotates k (fp8 workloads rotate
        # inside their quantizer instead, and relay once when set up)
        self.fuse_prep = (not wl.qk_fp8 and any(p is not None for p in self.prefix_src)) if fuse_prep is None \
            else bool(fuse_prep) and not wl.qk_fp8
        if wl.qk_fp8:
            self.relayout(always=True)
            self.quantize_prefix()

    def quantize_prefix(self) -> None:
        """E4M3 codes of each prefix K (fp8 workloads), once per conditioning cache."""
        for b, p in enumerate(self.prefix_online):
            if p is None:
                continue
            if self.blocks:
                nx.nxattn_quantize_fp8_blocks(p[0].unsqueeze(0), self.pk8[b], self.pks[b])
            else:
                nx.nxattn_quantize_fp8(p[0].unsqueeze(0), self.pk8[b], self.pke[b:b + 1], self.qws)

    def relayout_jobs(self) -> list:
        return [(src, dst.unsqueeze(0), 0) for src, dst in zip(self.prefix_src, self.prefix_online) if src is not None]

    def relayout(self, always: bool = False) -> None:
        if self.fuse_prep and not always:
            return                      # done in rope()
        for src, dst, d in self.relayout_jobs():
            nx.nxattn_kv_relayout(src, dst, d)

    def rope(self) -> None:
        if self.wl.qk_fp8:
            return                      # rotated inside quantize(): only the codes are needed
        if not self.fuse_q_rope:
            nx.nxattn_rope_apply(self.q, self.descs)
        if self.fuse_prep:
            nx.nxattn_rope_apply_relayout(self.k, self.descs, self.relayout_jobs())
        else:
            nx.nxattn_rope_apply(self.k, self.descs)

    def quantize(self) -> None:
        """E4M3 codes of the rotated q and k (one call for both: the rotation evaluated
        inside the quantizer's passes, q and k left as given; fp8 workloads only). q's
        codes carry the softmax fold factor, which the library forms."""
        if not self.wl.qk_fp8:
            return
        if self.q_on_load:
            nx.nxattn_rope_quantize_fp8([self.k], self.descs, [self.k8], [self.ks], blocks=True)
            return
        if self.blocks:
            nx.nxattn_rope_quantize_fp8([self.q, self.k], self.descs, [self.q8, self.k8], [self.qs, self.ks],
                                        folds=[self.fold_q, False], blocks=True)
            return
        nx.nxattn_rope_quantize_fp8([self.q, self.k], self.descs, [self.q8, self.k8], [self.qe, self.ke], self.qws,
                                    folds=[self.fold_q, False])

    def attention(self) -> None:
        # with the guidance combination inside the call: the guided output, and the branch
        # outputs only if kept
        o = self.o if self.keep_branches else None
        g = dict(cfg_out=self.out, guidance=self.wl.guidance) if self.fuse_cfg else {}
        if self.q_on_load:
            nx.nxattn_fwd_fp8(None, self.k8, None, None, self.v, o,
                              [None if p is None else p[0] for p in self.pk8],
                              [None if p is None else p[1] for p in self.prefix_online],
                              k_scales=self.ks, prefix_k_scales=[None if p is None else p[0] for p in self.pks],
                              q=self.q, q_rope=self.descs, **g)
            return
        if self.blocks:
            nx.nxattn_fwd_fp8(self.q8, self.k8, None, None, self.v, o,
                              [None if p is None else p[0] for p in self.pk8],
                              [None if p is None else p[1] for p in self.prefix_online],
                              q_folded=self.fold_q, q_scales=self.qs, k_scales=self.ks,
                              prefix_k_scales=[None if p is None else p[0] for p in self.pks], **g)
            return
        if self.wl.qk_fp8:
            nx.nxattn_fwd_fp8(self.q8, self.k8, self.qe, self.ke, self.v, o,
                              [None if p is None else p[0] for p in self.pk8],
                              [None if p is None else p[1] for p in self.prefix_online],
                              self.pke if any(p is not None for p in self.prefix_online) else None,
                              q_folded=self.fold_q, **g)
            return
        if self.fuse_cfg:
            nx.nxattn_fwd(self.q, self.k, self.v, o, self.prefix_online,
                          q_rope=self.descs if self.fuse_q_rope else None, **g)
            return
        nx.nxattn_fwd(self.q, self.k, self.v, self.o, self.prefix_online,
                      q_rope=self.descs if self.fuse_q_rope else None,
                      num_splits=self.splits, workspace=self.workspace)

    def cfg(self) -> None:
        if self.use_cfg and not self.fuse_cfg:
            nx.nxattn_cfg_combine(self.o[0], self.o[1], self.out, self.wl.guidance)

    def __call__(self) -> torch.Tensor:
        self.relayout()
        self.rope()
        self.quantize()
        self.attention()
        self.cfg()
        return self.out if self.use_cfg else self.o

    def capture(self, warmup: int = 2) -> "torch.cuda.CUDAGraph":
        """Record one step (the same launches as a call, on the same buffers) into a HIP
        graph; see ``capture_steps``."""
        return capture_steps([self], warmup)


def capture_steps(steps: List[AttentionStep], warmup: int = 2) -> "torch.cuda.CUDAGraph":
    """Record the given steps, one after another (the layers of a multi-layer step), into
    one HIP graph; ``graph.replay()`` then runs them with one submission, for callers
    that drive the step from a captured loop. A step allocates nothing and clears nothing with memset,
    so it can be captured. Like a call, a replay rotates k in place (bf16 path) and
    overwrites the outputs."""
    side = torch.cuda.Stream()                      # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            for st in steps:
                st()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for st in steps:
            st()
    torch.cuda.synchronize()
    return graph
