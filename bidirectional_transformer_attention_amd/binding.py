"""ctypes binding of libnxattn.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their data
pointers, sizes, strides and the current HIP stream to the C ABI declared in
include/nxattn.h, and raises NxattnError on a nonzero status. There is no fallback:
if the library is not built, or a tensor is not on the GPU, the call fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree library; NXATTN_LIBRARY names another build of it (for instance one with
# host-side sanitizers)
LIB_PATH = os.environ.get("NXATTN_LIBRARY") or os.path.join(_HERE, "libnxattn.so")

NXATTN_F32 = 0
NXATTN_BF16 = 1
MAX_BRANCHES = 8
MAX_SPLITS = 16

SYMBOLS = ("nxattn_kv_relayout", "nxattn_rope_apply", "nxattn_rope_apply_relayout", "nxattn_fwd", "nxattn_fwd_workspace_size",
           "nxattn_attn_merge", "nxattn_quantize_fp8_workspace_size", "nxattn_quantize_fp8",
           "nxattn_quantize_fp8_blocks", "nxattn_rope_quantize_fp8", "nxattn_rope_quantize_fp8_noalloc", "nxattn_fwd_fp8",
           "nxattn_cfg_combine", "nxattn_status_string", "nxattn_last_error", "nxattn_version")


class NxattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"nxattn status {status}: {msg}")
        self.status = status


class RopeDesc(ctypes.Structure):
    _fields_ = [("n_axes", ctypes.c_int32), ("grid", ctypes.c_int32 * 3), ("pairs", ctypes.c_int32 * 3),
                ("offset", ctypes.c_int32 * 3), ("theta", ctypes.c_double), ("interleaved", ctypes.c_int32),
                ("global_freq", ctypes.c_int32)]


class RelayoutJob(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("layers", ctypes.c_int64),
                ("kv_heads", ctypes.c_int64), ("seq", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("dir", ctypes.c_int32)]


class Fp8Tensor(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("heads", ctypes.c_int64), ("strides", ctypes.c_int64 * 3),
                ("codes", ctypes.c_void_p), ("exps", ctypes.c_void_p), ("mult", ctypes.c_float),
                ("fold_softmax", ctypes.c_int32), ("scales", ctypes.c_void_p)]


MAX_FP8_TENSORS = 4


class FwdArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("seq_q", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("q_strides", ctypes.c_int64 * 3), ("kv_strides", ctypes.c_int64 * 3),
                ("o_strides", ctypes.c_int64 * 3),
                ("prefix_kv", ctypes.c_void_p * MAX_BRANCHES), ("prefix_len", ctypes.c_int32 * MAX_BRANCHES),
                ("scale", ctypes.c_float), ("q_rope", ctypes.POINTER(RopeDesc)),
                ("lse", ctypes.c_void_p), ("prefix_only", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("cfg_out", ctypes.c_void_p), ("cfg_strides", ctypes.c_int64 * 2), ("guidance", ctypes.c_float)]


class FwdFp8Args(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_q", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q8", ctypes.c_void_p), ("k8", ctypes.c_void_p), ("q_exp", ctypes.c_void_p),
                ("k_exp", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("v_strides", ctypes.c_int64 * 3), ("o_strides", ctypes.c_int64 * 3),
                ("prefix_k8", ctypes.c_void_p * MAX_BRANCHES), ("prefix_v", ctypes.c_void_p * MAX_BRANCHES),
                ("prefix_len", ctypes.c_int32 * MAX_BRANCHES), ("prefix_k_exp", ctypes.c_void_p),
                ("scale", ctypes.c_float), ("lse", ctypes.c_void_p), ("q_folded", ctypes.c_int32),
                ("q_scales", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("prefix_k_scales", ctypes.c_void_p * MAX_BRANCHES),
                ("q", ctypes.c_void_p), ("q_strides", ctypes.c_int64 * 3), ("q_rope", ctypes.POINTER(RopeDesc)),
                ("q8_out", ctypes.c_void_p), ("q_scales_out", ctypes.c_void_p),
                ("cfg_out", ctypes.c_void_p), ("cfg_strides", ctypes.c_int64 * 2), ("guidance", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnxattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bidirectional_transformer_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.nxattn_kv_relayout.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.nxattn_kv_relayout.restype = i32
    lib.nxattn_rope_apply.argtypes = [vp, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64), i32,
                                      ctypes.POINTER(RopeDesc), vp]
    lib.nxattn_rope_apply.restype = i32
    lib.nxattn_rope_apply_relayout.argtypes = [vp, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64), i32,
                                               ctypes.POINTER(RopeDesc), ctypes.POINTER(RelayoutJob), ctypes.c_int32, vp]
    lib.nxattn_rope_apply_relayout.restype = i32
    lib.nxattn_fwd.argtypes = [ctypes.POINTER(FwdArgs), vp]
    lib.nxattn_fwd.restype = i32
    lib.nxattn_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(ctypes.c_int64)]
    lib.nxattn_fwd_workspace_size.restype = i32
    lib.nxattn_attn_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int32, i64, i64, i64, i64,
                                      ctypes.POINTER(ctypes.c_int64), i32, vp, ctypes.POINTER(ctypes.c_int64), vp,
                                      vp]
    lib.nxattn_attn_merge.restype = i32
    lib.nxattn_quantize_fp8_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.nxattn_quantize_fp8_workspace_size.restype = i32
    lib.nxattn_quantize_fp8.argtypes = [vp, i32, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64), vp, vp, vp,
                                        i64, vp]
    lib.nxattn_quantize_fp8.restype = i32
    lib.nxattn_quantize_fp8_blocks.argtypes = [vp, i32, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64), vp, vp,
                                               vp]
    lib.nxattn_quantize_fp8_blocks.restype = i32
    lib.nxattn_rope_quantize_fp8.argtypes = [ctypes.POINTER(Fp8Tensor), i32, i32, i64, i64, i64,
                                             ctypes.POINTER(RopeDesc), vp, i64, vp]
    lib.nxattn_rope_quantize_fp8.restype = i32
    lib.nxattn_rope_quantize_fp8_noalloc.argtypes = [ctypes.POINTER(Fp8Tensor), i32, i32, i64, i64, i64,
                                                     ctypes.POINTER(RopeDesc), vp]
    lib.nxattn_rope_quantize_fp8_noalloc.restype = i32
    lib.nxattn_fwd_fp8.argtypes = [ctypes.POINTER(FwdFp8Args), vp]
    lib.nxattn_fwd_fp8.restype = i32
    lib.nxattn_cfg_combine.argtypes = [vp, vp, vp, i64, ctypes.c_float, i32, vp]
    lib.nxattn_cfg_combine.restype = i32
    lib.nxattn_status_string.argtypes = [i32]
    lib.nxattn_status_string.restype = ctypes.c_char_p
    lib.nxattn_last_error.argtypes = []
    lib.nxattn_last_error.restype = ctypes.c_char_p
    lib.nxattn_version.argtypes = []
    lib.nxattn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nxattn_status_string(status).decode()


def last_error() -> str:
    return load().nxattn_last_error().decode()


def version() -> str:
    return load().nxattn_version().decode()


def _check(status: int) -> None:
    if status != 0:
        raise NxattnError(status, f"{status_string(status)}: {last_error()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NXATTN_F32
    if t.dtype == torch.bfloat16:
        return NXATTN_BF16
    raise NxattnError(2, f"unsupported tensor dtype {t.dtype}")


def _gpu(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise NxattnError(1, "tensors must be on the GPU (HIP device)")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def rope_desc(grid: Sequence[int], pairs: Sequence[int], offset: Sequence[int], theta: float = 10000.0,
              interleaved: bool = False, global_freq: bool = False) -> RopeDesc:
    d = RopeDesc()
    d.n_axes = len(grid)
    for a in range(3):
        d.grid[a] = int(grid[a]) if a < len(grid) else 1
        d.pairs[a] = int(pairs[a]) if a < len(pairs) else 0
        d.offset[a] = int(offset[a]) if a < len(offset) else 0
    d.theta = float(theta)
    d.interleaved = 1 if interleaved else 0
    d.global_freq = 1 if global_freq else 0
    return d


# ---------------------------------------------------------------------------------------
def _relayout_sizes(src: torch.Tensor, dst: torch.Tensor, direction: int):
    """(L, H, S, D) of a relayout of src into dst (checked as nxattn_kv_relayout takes them)."""
    _gpu(src, dst)
    if src.dim() != 5 or dst.dim() != 5 or src.shape[1] != 2:
        raise NxattnError(1, "relayout expects 5-D [L, 2, ., ., D] tensors")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise NxattnError(1, "relayout expects contiguous tensors")
    if src.dtype != dst.dtype:
        raise NxattnError(1, "src and dst dtypes differ")
    L, _, A, B, D = src.shape
    H, S = (A, B) if direction == 0 else (B, A)
    if tuple(dst.shape) != (L, 2, B, A, D):
        raise NxattnError(1, f"dst shape {tuple(dst.shape)} does not match {(L, 2, B, A, D)}")
    return L, H, S, D


def nxattn_kv_relayout(src: torch.Tensor, dst: torch.Tensor, direction: int, stream=None) -> None:
    """dir 0: src replay [L,2,H,S,D] -> dst online [L,2,S,H,D]; dir 1: the inverse."""
    L, H, S, D = _relayout_sizes(src, dst, direction)
    _check(load().nxattn_kv_relayout(src.data_ptr(), dst.data_ptr(), L, H, S, D, _dtype_code(src),
                                     int(direction), _stream(stream)))


def nxattn_rope_apply(x: torch.Tensor, descs: List[RopeDesc], stream=None) -> None:
    """In-place RoPE on x [B, S, H, D] (strided, D contiguous); one descriptor per branch."""
    _gpu(x)
    if x.dim() != 4:
        raise NxattnError(1, "x must be [B, S, H, D]")
    B, S, H, D = x.shape
    if x.stride(3) != 1:
        raise NxattnError(1, "the head_dim dimension must be contiguous")
    if len(descs) != B:
        raise NxattnError(1, "one RopeDesc per batch entry is required")
    st = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    arr = (RopeDesc * max(1, B))(*descs)
    _check(load().nxattn_rope_apply(x.data_ptr(), B, S, H, D, st, _dtype_code(x), arr, _stream(stream)))


def nxattn_rope_apply_relayout(x: torch.Tensor, descs: List[RopeDesc],
                               jobs: Sequence[tuple] = (), stream=None) -> None:
    """nxattn_rope_apply(x, descs) and, in the same launch, nxattn_kv_relayout(src, dst,
    direction) for each (src, dst, direction) in jobs (tensors of x's dtype)."""
    _gpu(x)
    if x.dim() != 4:
        raise NxattnError(1, "x must be [B, S, H, D]")
    B, S, H, D = x.shape
    if x.stride(3) != 1:
        raise NxattnError(1, "the head_dim dimension must be contiguous")
    if len(descs) != B:
        raise NxattnError(1, "one RopeDesc per batch entry is required")
    if len(jobs) > MAX_BRANCHES:
        raise NxattnError(1, f"at most {MAX_BRANCHES} relayout jobs")
    arr_j = (RelayoutJob * max(1, len(jobs)))()
    for i, (src, dst, direction) in enumerate(jobs):
        if src.dtype != x.dtype:
            raise NxattnError(1, "relayout jobs must have x's dtype")
        L, Hk, Sk, Dk = _relayout_sizes(src, dst, direction)
        j = arr_j[i]
        j.src, j.dst, j.layers, j.kv_heads, j.seq, j.head_dim, j.dir = (src.data_ptr(), dst.data_ptr(), L, Hk, Sk,
                                                                         Dk, int(direction))
    st = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    arr = (RopeDesc * max(1, B))(*descs)
    _check(load().nxattn_rope_apply_relayout(x.data_ptr(), B, S, H, D, st, _dtype_code(x), arr, arr_j, len(jobs),
                                             _stream(stream)))


def make_fwd_args(q: torch.Tensor, k: Optional[torch.Tensor], v: Optional[torch.Tensor], o: Optional[torch.Tensor],
                  prefix: Sequence[Optional[torch.Tensor]], scale: float = 0.0,
                  q_rope: Optional[Sequence[RopeDesc]] = None, lse: Optional[torch.Tensor] = None,
                  prefix_only: bool = False, num_splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, cfg_out: Optional[torch.Tensor] = None,
                  guidance: float = 0.0) -> FwdArgs:
    """FwdArgs for the tensors; q_rope (one RopeDesc per batch entry) is kept alive on
    the returned object for as long as it is in use. k and v may be None with
    prefix_only (heads_kv then comes from the first prefix); o may be None with cfg_out."""
    B, S, Hq, D = q.shape
    a = FwdArgs()
    a.dtype = _dtype_code(q)
    hkv = k.shape[2] if k is not None else next(p.shape[2] for p in prefix if p is not None)
    a.batch, a.seq_q, a.heads_q, a.heads_kv, a.head_dim = B, S, Hq, hkv, D
    a.q = q.data_ptr()
    a.o = o.data_ptr() if o is not None else None
    a.k = k.data_ptr() if k is not None else None
    a.v = v.data_ptr() if v is not None else None
    for i in range(3):
        a.q_strides[i] = q.stride(i)
        a.kv_strides[i] = k.stride(i) if k is not None else 0
        a.o_strides[i] = o.stride(i) if o is not None else 0
    for b in range(MAX_BRANCHES):
        p = prefix[b] if b < len(prefix) else None
        if p is None or p.numel() == 0:
            a.prefix_kv[b] = None
            a.prefix_len[b] = 0
        else:
            a.prefix_kv[b] = p.data_ptr()
            a.prefix_len[b] = p.shape[1]
    a.scale = float(scale)
    if q_rope is not None:
        arr = (RopeDesc * len(q_rope))(*q_rope)
        a._q_rope_keep = arr
        a.q_rope = ctypes.cast(arr, ctypes.POINTER(RopeDesc))
    a.lse = lse.data_ptr() if lse is not None else None
    a.prefix_only = 1 if prefix_only else 0
    a.num_splits = int(num_splits)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    if cfg_out is not None:
        a.cfg_out = cfg_out.data_ptr()
        a.cfg_strides[0], a.cfg_strides[1] = cfg_out.stride(0), cfg_out.stride(1)
        a.guidance = float(guidance)
    return a


def fwd_workspace_bytes(batch: int, seq_q: int, heads_q: int, head_dim: int, num_splits: int) -> int:
    """Bytes of workspace nxattn_fwd needs for num_splits key ranges (0 if <= 1)."""
    a = FwdArgs()
    a.batch, a.seq_q, a.heads_q, a.head_dim, a.num_splits = batch, seq_q, heads_q, head_dim, num_splits
    n = ctypes.c_int64(0)
    _check(load().nxattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def nxattn_fwd(q: torch.Tensor, k: Optional[torch.Tensor], v: Optional[torch.Tensor], o: Optional[torch.Tensor],
               prefix: Sequence[Optional[torch.Tensor]] = (), scale: float = 0.0, stream=None,
               q_rope: Optional[Sequence[RopeDesc]] = None, lse: Optional[torch.Tensor] = None,
               prefix_only: bool = False, num_splits: int = 0,
               workspace: Optional[torch.Tensor] = None, cfg_out: Optional[torch.Tensor] = None,
               guidance: float = 0.0) -> None:
    """o = attention(q, [prefix_k ++ k], [prefix_v ++ v]) for every branch.

    q, o [B,S,Hq,D]; k, v [B,S,Hkv,D] (same strides); prefix[b] contiguous [2,P_b,Hkv,D] or None.
    q_rope: None (q already rotated) or one RopeDesc per batch entry, to rotate q on load
    (bf16 only); q itself is left unchanged.
    lse: None or a contiguous fp32 [B, Hq, S] output for the log-sum-exp of the scores.
    prefix_only: the keys are the prefix rows alone (k and v may then be None).
    num_splits > 1: split every branch's keys into that many ranges merged by a second
    kernel; workspace is a device tensor of at least fwd_workspace_bytes() bytes (one is
    allocated with torch when None).
    cfg_out: None, or a [S, Hq, D] tensor of q's dtype (last dim contiguous) that receives
    the guidance combination of the two branches (batch 2: branch 0 cond, 1 uncond),
    computed by the attention kernel; o may then be None (branch outputs not stored).
    """
    own = [t for t in (k, v) if t is not None]
    _gpu(q, o, *own, lse, workspace, cfg_out, *[p for p in prefix if p is not None])
    if o is None and cfg_out is None:
        raise NxattnError(1, "o is required unless cfg_out is given")
    if cfg_out is not None and (cfg_out.dim() != 3 or tuple(cfg_out.shape) != (q.shape[1], q.shape[2], q.shape[3])
                                or cfg_out.stride(2) != 1 or cfg_out.dtype != q.dtype):
        raise NxattnError(1, "cfg_out must be [S, Hq, D] of q's dtype with a contiguous last dim")
    if not prefix_only and len(own) != 2:
        raise NxattnError(1, "k and v are required unless prefix_only")
    if q.dim() != 4 or (o is not None and o.dim() != 4) or any(t.dim() != 4 for t in own):
        raise NxattnError(1, "q, k, v, o must be 4-D [B, S, H, D]")
    if len(own) == 2 and (k.shape != v.shape or k.stride() != v.stride()):
        raise NxattnError(1, "k and v must have the same shape and strides")
    if len(own) == 1:
        raise NxattnError(1, "give both k and v, or neither")
    if (o is not None and o.shape != q.shape) or any(q.shape[0] != t.shape[0] or q.shape[1] != t.shape[1]
                                                     or q.shape[3] != t.shape[3] for t in own):
        raise NxattnError(1, "inconsistent q/k/v/o shapes")
    if prefix_only and (len(prefix) != q.shape[0] or any(p is None for p in prefix)):
        raise NxattnError(1, "prefix_only needs one prefix per batch entry")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1])):
        raise NxattnError(1, "lse must be a contiguous float32 [B, Hq, S] tensor")
    if len(prefix) not in (0, q.shape[0]):
        raise NxattnError(1, "prefix must have one entry per batch entry")
    given = [p for p in prefix if p is not None]
    hkv = k.shape[2] if k is not None else (given[0].shape[2] if given and given[0].dim() == 4 else -1)
    for p in given:
        if (not p.is_contiguous() or p.dim() != 4 or p.shape[0] != 2
                or p.shape[2] != hkv or p.shape[3] != q.shape[3] or p.dtype != q.dtype):
            raise NxattnError(1, "prefix entries must be contiguous [2, P, Hkv, D] of q's dtype")
    for t in (*own, *([o] if o is not None else [])):
        if t.dtype != q.dtype:
            raise NxattnError(1, "q, k, v, o dtypes differ")
    if q_rope is not None and len(q_rope) != q.shape[0]:
        raise NxattnError(1, "q_rope must have one descriptor per batch entry")
    if num_splits > 1 and workspace is None:
        n = fwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3], num_splits)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    a = make_fwd_args(q, k, v, o, prefix, scale, q_rope, lse, prefix_only, num_splits, workspace, cfg_out, guidance)
    _check(load().nxattn_fwd(ctypes.byref(a), _stream(stream)))


def nxattn_attn_merge(parts_o: Sequence[torch.Tensor], parts_lse: Sequence[torch.Tensor], o: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Merge attention results over disjoint key sets (o and lse of each part).

    parts_o[p] [B,S,H,D] (all with the same strides and o's dtype), parts_lse[p] contiguous
    fp32 [B,H,S]; o [B,S,H,D] may be exactly one of the parts; lse (optional) [B,H,S] fp32
    may be exactly one of parts_lse.
    """
    _gpu(o, lse, *parts_o, *parts_lse)
    n = len(parts_o)
    if n != len(parts_lse) or n == 0:
        raise NxattnError(1, "one lse per part and at least one part are required")
    if o.dim() != 4:
        raise NxattnError(1, "o must be [B, S, H, D]")
    B, S, H, D = o.shape
    for t in parts_o:
        if t.shape != o.shape or t.stride() != parts_o[0].stride() or t.dtype != o.dtype:
            raise NxattnError(1, "parts must share o's shape and dtype and one set of strides")
    for t in (*parts_lse, *([lse] if lse is not None else [])):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, S):
            raise NxattnError(1, "lse tensors must be contiguous float32 [B, H, S]")
    if o.stride(3) != 1 or parts_o[0].stride(3) != 1:
        raise NxattnError(1, "the head_dim dimension must be contiguous")
    po = (ctypes.c_void_p * n)(*[t.data_ptr() for t in parts_o])
    pl = (ctypes.c_void_p * n)(*[t.data_ptr() for t in parts_lse])
    pst = (ctypes.c_int64 * 3)(*parts_o[0].stride()[:3])
    ost = (ctypes.c_int64 * 3)(*o.stride()[:3])
    _check(load().nxattn_attn_merge(po, pl, n, B, S, H, D, pst, _dtype_code(o), o.data_ptr(), ost,
                                    lse.data_ptr() if lse is not None else None, _stream(stream)))


def nxattn_cfg_combine(cond: torch.Tensor, uncond: torch.Tensor, out: torch.Tensor, guidance: float,
                       stream=None) -> None:
    """out = uncond + guidance * (cond - uncond) over contiguous tensors of equal size."""
    _gpu(cond, uncond, out)
    if not (cond.is_contiguous() and uncond.is_contiguous() and out.is_contiguous()):
        raise NxattnError(1, "cfg tensors must be contiguous")
    if cond.numel() != uncond.numel() or cond.numel() != out.numel():
        raise NxattnError(1, "cfg tensors differ in size")
    if cond.dtype != uncond.dtype or cond.dtype != out.dtype:
        raise NxattnError(1, "cfg dtypes differ")
    _check(load().nxattn_cfg_combine(cond.data_ptr(), uncond.data_ptr(), out.data_ptr(), cond.numel(),
                                     float(guidance), _dtype_code(cond), _stream(stream)))


def quantize_fp8_workspace_bytes(batch: int, seq: int, heads: int) -> int:
    n = ctypes.c_int64(0)
    _check(load().nxattn_quantize_fp8_workspace_size(batch, seq, heads, ctypes.byref(n)))
    return int(n.value)


def _quant_outputs(x, codes, exps):
    if x.dim() != 4 or x.stride(3) != 1:
        raise NxattnError(1, "x must be [B, S, H, D] with D contiguous")
    B, S, H, D = x.shape
    if codes is None:
        codes = torch.empty((B, S, H, D), dtype=torch.uint8, device=x.device)
    if exps is None:
        exps = torch.empty((B, H), dtype=torch.int8, device=x.device)
    if codes.dtype != torch.uint8 or tuple(codes.shape) != (B, S, H, D) or not codes.is_contiguous():
        raise NxattnError(1, "codes must be a contiguous uint8 [B, S, H, D] tensor")
    if exps.dtype != torch.int8 or tuple(exps.shape) != (B, H) or not exps.is_contiguous():
        raise NxattnError(1, "exps must be a contiguous int8 [B, H] tensor")
    return codes, exps


def nxattn_quantize_fp8(x: torch.Tensor, codes: Optional[torch.Tensor] = None, exps: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """E4M3 codes (uint8, contiguous [B,S,H,D]) and per-(b,h) exponents (int8 [B,H]) of x
    [B,S,H,D] (bf16 or f32, strided, D contiguous); outputs and the workspace are
    allocated with torch when not given. Returns (codes, exps)."""
    _gpu(x, codes, exps, workspace)
    codes, exps = _quant_outputs(x, codes, exps)
    B, S, H, D = x.shape
    if workspace is None:
        workspace = torch.empty(max(4, quantize_fp8_workspace_bytes(B, S, H)), dtype=torch.uint8, device=x.device)
    st = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    _check(load().nxattn_quantize_fp8(x.data_ptr(), _dtype_code(x), B, S, H, D, st, codes.data_ptr(), exps.data_ptr(),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return codes, exps


def _block_outputs(x, codes, scales):
    if x.dim() != 4 or x.stride(3) != 1:
        raise NxattnError(1, "x must be [B, S, H, D] with D contiguous")
    B, S, H, D = x.shape
    if D % 32 != 0:
        raise NxattnError(2, "block scales need head_dim a multiple of 32")
    if codes is None:
        codes = torch.empty((B, S, H, D), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, S, H, D // 32), dtype=torch.uint8, device=x.device)
    if codes.dtype != torch.uint8 or tuple(codes.shape) != (B, S, H, D) or not codes.is_contiguous():
        raise NxattnError(1, "codes must be a contiguous uint8 [B, S, H, D] tensor")
    if scales.dtype != torch.uint8 or tuple(scales.shape) != (B, S, H, D // 32) or not scales.is_contiguous():
        raise NxattnError(1, "scales must be a contiguous uint8 [B, S, H, D / 32] tensor")
    return codes, scales


def nxattn_quantize_fp8_blocks(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                               scales: Optional[torch.Tensor] = None, stream=None):
    """E4M3 codes (uint8, contiguous [B,S,H,D]) and one E8M0 scale code per 32-element run
    (uint8 [B,S,H,D/32]) of x [B,S,H,D] (bf16 or f32, strided, D contiguous, D % 32 == 0);
    outputs allocated with torch when not given. Returns (codes, scales)."""
    _gpu(x, codes, scales)
    codes, scales = _block_outputs(x, codes, scales)
    B, S, H, D = x.shape
    st = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    _check(load().nxattn_quantize_fp8_blocks(x.data_ptr(), _dtype_code(x), B, S, H, D, st, codes.data_ptr(),
                                             scales.data_ptr(), _stream(stream)))
    return codes, scales


def nxattn_rope_quantize_fp8(xs: Sequence[torch.Tensor], descs: List[RopeDesc],
                             codes: Optional[Sequence[torch.Tensor]] = None,
                             exps: Optional[Sequence[torch.Tensor]] = None,
                             workspace: Optional[torch.Tensor] = None,
                             mults: Optional[Sequence[float]] = None,
                             folds: Optional[Sequence[bool]] = None, blocks: bool = False, stream=None):
    """Codes and exponents (as nxattn_quantize_fp8) of each x in xs ([B,S,H_t,D], one
    dtype, shared B, S, D and positions) rotated as nxattn_rope_apply would rotate it and,
    where mults gives a factor other than 0 or 1, multiplied by it in fp32 after the
    rotation's rounding; where folds[t] is true the library multiplies by the softmax
    fold factor instead (the codes nxattn_fwd_fp8 takes with q_folded; mults[t] > 0 then
    gives the softmax scale). With blocks, each 32-element run gets its own scale (as
    nxattn_quantize_fp8_blocks; `exps` then holds the uint8 [B,S,H_t,D/32] scale tensors
    and no workspace is used). The x are not modified. Returns [(codes, exps or scales)]
    in the order of xs."""
    xs = list(xs)
    if not 1 <= len(xs) <= MAX_FP8_TENSORS:
        raise NxattnError(1, f"need 1 to {MAX_FP8_TENSORS} tensors")
    codes = list(codes) if codes is not None else [None] * len(xs)
    exps = list(exps) if exps is not None else [None] * len(xs)
    _gpu(*xs, *[c for c in codes if c is not None], *[e for e in exps if e is not None], workspace)
    outs = _rope_quant_outputs(xs, descs, codes, exps, blocks)
    B, S, _, D = xs[0].shape
    total = sum(x.shape[2] for x in xs)
    if workspace is None and not blocks:
        workspace = torch.empty(max(4, quantize_fp8_workspace_bytes(B, S, total)), dtype=torch.uint8,
                                device=xs[0].device)
    arr = _fp8_tensors(xs, outs, mults, folds, blocks)
    darr = (RopeDesc * max(1, B))(*descs)
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().nxattn_rope_quantize_fp8(arr, len(xs), _dtype_code(xs[0]), B, S, D, darr, wp, wb,
                                           _stream(stream)))
    return outs


def nxattn_rope_quantize_fp8_noalloc(xs: Sequence[torch.Tensor], descs: List[RopeDesc],
                                     codes: Sequence[torch.Tensor], exps: Sequence[torch.Tensor],
                                     mults: Optional[Sequence[float]] = None,
                                     folds: Optional[Sequence[bool]] = None, blocks: bool = False, stream=None):
    """nxattn_rope_quantize_fp8 into the given codes and exps (with blocks: the block
    scales) without a workspace (the library's static scratch holds the running maxima);
    nothing is allocated here either. Returns [(codes, exps)] in the order of xs."""
    xs = list(xs)
    if not 1 <= len(xs) <= MAX_FP8_TENSORS:
        raise NxattnError(1, f"need 1 to {MAX_FP8_TENSORS} tensors")
    codes, exps = list(codes), list(exps)
    if len(codes) != len(xs) or len(exps) != len(xs) or any(t is None for t in codes + exps):
        raise NxattnError(1, "codes and exps must be given for every tensor")
    _gpu(*xs, *codes, *exps)
    outs = _rope_quant_outputs(xs, descs, codes, exps, blocks)
    B, S, _, D = xs[0].shape
    arr = _fp8_tensors(xs, outs, mults, folds, blocks)
    darr = (RopeDesc * max(1, B))(*descs)
    _check(load().nxattn_rope_quantize_fp8_noalloc(arr, len(xs), _dtype_code(xs[0]), B, S, D, darr, _stream(stream)))
    return outs


def _rope_quant_outputs(xs, descs, codes, exps, blocks=False):
    B, S, _, D = xs[0].shape
    outs = []
    for x, c, e in zip(xs, codes, exps):
        if x.dim() != 4 or (x.shape[0], x.shape[1], x.shape[3]) != (B, S, D) or x.dtype != xs[0].dtype:
            raise NxattnError(1, "tensors must share batch, seq, head_dim and dtype")
        c, e = _block_outputs(x, c, e) if blocks else _quant_outputs(x, c, e)
        outs.append((c, e))
    if len(descs) != B:
        raise NxattnError(1, "one RopeDesc per batch entry is required")
    return outs


def _fp8_tensors(xs, outs, mults, folds, blocks=False):
    arr = (Fp8Tensor * len(xs))()
    for i, (x, (c, e)) in enumerate(zip(xs, outs)):
        arr[i].x, arr[i].heads = x.data_ptr(), x.shape[2]
        for k in range(3):
            arr[i].strides[k] = x.stride(k)
        arr[i].codes = c.data_ptr()
        if blocks:
            arr[i].exps, arr[i].scales = None, e.data_ptr()
        else:
            arr[i].exps, arr[i].scales = e.data_ptr(), None
        arr[i].mult = float(mults[i]) if mults is not None else 0.0
        arr[i].fold_softmax = 1 if (folds is not None and folds[i]) else 0
    return arr


def nxattn_fwd_fp8(q8: Optional[torch.Tensor], k8: torch.Tensor, q_exp: Optional[torch.Tensor],
                   k_exp: Optional[torch.Tensor], v: torch.Tensor,
                   o: Optional[torch.Tensor], prefix_k8: Sequence[Optional[torch.Tensor]] = (),
                   prefix_v: Sequence[Optional[torch.Tensor]] = (), prefix_k_exp: Optional[torch.Tensor] = None,
                   scale: float = 0.0, lse: Optional[torch.Tensor] = None, q_folded: bool = False,
                   q_scales: Optional[torch.Tensor] = None, k_scales: Optional[torch.Tensor] = None,
                   prefix_k_scales: Sequence[Optional[torch.Tensor]] = (), q: Optional[torch.Tensor] = None,
                   q_rope: Optional[Sequence[RopeDesc]] = None, q8_out: Optional[torch.Tensor] = None,
                   q_scales_out: Optional[torch.Tensor] = None, stream=None,
                   cfg_out: Optional[torch.Tensor] = None, guidance: float = 0.0) -> None:
    """Attention with the fp8 score GEMM: q8 [B,S,Hq,128], k8 [B,S,Hkv,128] uint8 codes
    (contiguous), q_exp [B,Hq], k_exp [B,Hkv] int8; v [B,S,Hkv,128] and o [B,S,Hq,128] bf16;
    prefix_k8[b] uint8 [P_b,Hkv,128] and prefix_v[b] bf16 [P_b,Hkv,128] contiguous (or None),
    prefix_k_exp int8 [B,Hkv]. With q_folded, q8 holds the codes of q times
    softmax_scale*log2(e) (see nxattn_rope_quantize_fp8's folds) and scale is not used.
    Block scales: q_scales [B,S,Hq,4], k_scales [B,S,Hkv,4] and prefix_k_scales[b]
    [P_b,Hkv,4] (uint8 E8M0 codes, contiguous) in place of the exponents (which are then
    None). With q_rope (one RopeDesc per batch entry), q8 is None and q (bf16
    [B,S,Hq,128], head_dim contiguous) is rotated, folded and block-quantized on load; the
    keys take block scales; q8_out [B,S,Hq,128] and q_scales_out [B,S,Hq,4] (uint8,
    contiguous, optional) receive the codes and run scales formed on load.
    cfg_out: None, or a bf16 [S, Hq, 128] tensor (last dim contiguous) that receives the
    guidance combination of the two branches (batch 2), as with nxattn_fwd; o may then
    be None."""
    _gpu(q8, k8, q_exp, k_exp, v, o, prefix_k_exp, lse, q_scales, k_scales, q, q8_out, q_scales_out, cfg_out,
         *[t for t in prefix_k8 if t is not None], *[t for t in prefix_v if t is not None],
         *[t for t in prefix_k_scales if t is not None])
    qrope = q_rope is not None
    if qrope:
        if q8 is not None or q is None or q.dtype != torch.bfloat16 or q.dim() != 4 or q.stride(3) != 1:
            raise NxattnError(1, "q_rope takes q (bf16 [B, S, Hq, 128], head_dim contiguous) and no q8")
        B, S, Hq, D = q.shape
        if len(q_rope) != B:
            raise NxattnError(1, "one RopeDesc per batch entry is required")
    else:
        if q is not None or q8 is None:
            raise NxattnError(1, "q8 is required (q only with q_rope)")
        B, S, Hq, D = q8.shape
    Hkv = k8.shape[2]
    for t in ((k8,) if qrope else (q8, k8)):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 4:
            raise NxattnError(1, "q8 and k8 must be contiguous uint8 [B, S, H, D] tensors")
    if o is None and cfg_out is None:
        raise NxattnError(1, "o is required unless cfg_out is given")
    if (tuple(k8.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D)
            or (o is not None and tuple(o.shape) != (B, S, Hq, D))):
        raise NxattnError(1, "inconsistent q8/k8/v/o shapes")
    if v.dtype != torch.bfloat16 or v.stride(3) != 1 or (o is not None and (o.dtype != torch.bfloat16
                                                                             or o.stride(3) != 1)):
        raise NxattnError(1, "v and o must be bf16 with head_dim contiguous")
    if cfg_out is not None and (cfg_out.dim() != 3 or tuple(cfg_out.shape) != (S, Hq, D) or cfg_out.stride(2) != 1
                                or cfg_out.dtype != torch.bfloat16):
        raise NxattnError(1, "cfg_out must be bf16 [S, Hq, 128] with a contiguous last dim")
    block = q_scales is not None or qrope
    if block:
        if q_exp is not None or k_exp is not None or prefix_k_exp is not None:
            raise NxattnError(1, "block scales exclude the per-slice exponents")
        checks = ((k_scales, (B, S, Hkv, 4)),) if qrope else ((q_scales, (B, S, Hq, 4)), (k_scales, (B, S, Hkv, 4)))
        if qrope and q_scales is not None:
            raise NxattnError(1, "q_rope forms q's scales itself: q_scales must be None")
        for t, shp in checks:
            if t is None or t.dtype != torch.uint8 or tuple(t.shape) != shp or not t.is_contiguous():
                raise NxattnError(1, "q_scales / k_scales must be contiguous uint8 [B, S, H, 4] tensors")
    else:
        if k_scales is not None or any(t is not None for t in prefix_k_scales):
            raise NxattnError(1, "k_scales / prefix_k_scales need q_scales")
        for t, shp in ((q_exp, (B, Hq)), (k_exp, (B, Hkv))):
            if t is None or t.dtype != torch.int8 or tuple(t.shape) != shp or not t.is_contiguous():
                raise NxattnError(1, "exponents must be contiguous int8 [B, H] tensors")
    if len(prefix_k8) not in (0, B) or len(prefix_v) != len(prefix_k8):
        raise NxattnError(1, "prefix_k8 and prefix_v need one entry per batch entry")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, S)):
        raise NxattnError(1, "lse must be a contiguous float32 [B, Hq, S] tensor")
    a = FwdFp8Args()
    a.batch, a.seq_q, a.heads_q, a.heads_kv, a.head_dim = B, S, Hq, Hkv, D
    a.q_folded = 1 if q_folded else 0
    a.q8 = q8.data_ptr() if q8 is not None else None
    a.k8 = k8.data_ptr()
    a.q_exp = q_exp.data_ptr() if q_exp is not None else None
    a.k_exp = k_exp.data_ptr() if k_exp is not None else None
    a.q_scales = q_scales.data_ptr() if q_scales is not None else None
    a.k_scales = k_scales.data_ptr() if block else None
    if qrope:
        a.q = q.data_ptr()
        for i in range(3):
            a.q_strides[i] = q.stride(i)
        arr = (RopeDesc * len(q_rope))(*q_rope)
        a._q_rope_keep = arr
        a.q_rope = ctypes.cast(arr, ctypes.POINTER(RopeDesc))
        if (q8_out is None) != (q_scales_out is None):
            raise NxattnError(1, "q8_out and q_scales_out go together")
        if q8_out is not None:
            for t, shp in ((q8_out, (B, S, Hq, D)), (q_scales_out, (B, S, Hq, 4))):
                if t.dtype != torch.uint8 or tuple(t.shape) != shp or not t.is_contiguous():
                    raise NxattnError(1, "q8_out / q_scales_out must be contiguous uint8 [B, S, Hq, 128 / 4] tensors")
            a.q8_out, a.q_scales_out = q8_out.data_ptr(), q_scales_out.data_ptr()
    a.v = v.data_ptr()
    a.o = o.data_ptr() if o is not None else None
    for i in range(3):
        a.v_strides[i] = v.stride(i)
        a.o_strides[i] = o.stride(i) if o is not None else 0
    if cfg_out is not None:
        a.cfg_out = cfg_out.data_ptr()
        a.cfg_strides[0], a.cfg_strides[1] = cfg_out.stride(0), cfg_out.stride(1)
        a.guidance = float(guidance)
    for b in range(MAX_BRANCHES):
        pk = prefix_k8[b] if b < len(prefix_k8) else None
        pv = prefix_v[b] if b < len(prefix_v) else None
        if pk is None or pk.numel() == 0:
            a.prefix_k8[b] = None
            a.prefix_v[b] = None
            a.prefix_k_scales[b] = None
            a.prefix_len[b] = 0
            continue
        if (pk.dtype != torch.uint8 or not pk.is_contiguous() or pv is None or pv.dtype != torch.bfloat16
                or not pv.is_contiguous() or pk.shape != pv.shape or pk.dim() != 3 or pk.shape[1:] != (Hkv, D)):
            raise NxattnError(1, "prefix entries must be contiguous [P, Hkv, 128] (uint8 codes, bf16 values)")
        a.prefix_k8[b] = pk.data_ptr()
        a.prefix_v[b] = pv.data_ptr()
        a.prefix_len[b] = pk.shape[0]
        if block:
            ps = prefix_k_scales[b] if b < len(prefix_k_scales) else None
            if (ps is None or ps.dtype != torch.uint8 or not ps.is_contiguous()
                    or tuple(ps.shape) != (pk.shape[0], Hkv, 4)):
                raise NxattnError(1, "prefix_k_scales entries must be contiguous uint8 [P, Hkv, 4] tensors")
            a.prefix_k_scales[b] = ps.data_ptr()
        else:
            a.prefix_k_scales[b] = None
    a.prefix_k_exp = prefix_k_exp.data_ptr() if prefix_k_exp is not None else None
    a.scale = float(scale)
    a.lse = lse.data_ptr() if lse is not None else None
    _check(load().nxattn_fwd_fp8(ctypes.byref(a), _stream(stream)))
