"""The C-ABI library loads, exports every symbol include/nxattn.h declares, and rejects
bad arguments on the host before anything is launched (CPU only: no call here reaches
the GPU; validation returns first)."""
import ctypes
import os
import re

import pytest

import bidirectional_transformer_attention_amd as nx
from bidirectional_transformer_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nxattn.h")

OK, INVALID, UNSUPPORTED, ALIGN = 0, 1, 2, 3
FAKE = 0x7f0000000000  # a 16-byte aligned address that validation never dereferences


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        binding_build()
    return nx.load()


def binding_build():
    from bidirectional_transformer_attention_amd import build
    build.build(verbose=False)


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(nxattn_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_four_calls():
    syms = declared_symbols()
    for s in ("nxattn_kv_relayout", "nxattn_rope_apply", "nxattn_fwd", "nxattn_cfg_combine"):
        assert s in syms


def test_every_declared_symbol_is_exported(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert set(declared_symbols()) == set(binding.SYMBOLS)


def test_version_and_status_strings(lib):
    assert re.match(r"\d+\.\d+\.\d+", nx.version())
    assert nx.status_string(0) == "ok"
    for code in (1, 2, 3, 4):
        assert nx.status_string(code) != "ok"
    assert nx.status_string(99) == "unknown status"


# ----------------------------------------------------------------------------- fwd
def fwd_args(**kw):
    a = binding.FwdArgs()
    a.dtype, a.batch, a.seq_q, a.heads_q, a.heads_kv, a.head_dim = 1, 2, 64, 8, 2, 128
    a.q = a.k = a.v = FAKE
    a.o = FAKE + (1 << 32)
    for i, s in enumerate((64 * 8 * 128, 8 * 128, 128)):
        a.q_strides[i] = s
        a.o_strides[i] = s
    for i, s in enumerate((64 * 2 * 128, 2 * 128, 128)):
        a.kv_strides[i] = s
    for b in range(8):
        a.prefix_kv[b] = None
        a.prefix_len[b] = 0
    a.scale = 0.0
    for key, val in kw.items():
        if key in ("prefix_kv", "prefix_len", "q_strides", "kv_strides", "o_strides", "cfg_strides"):
            for i, x in enumerate(val):
                getattr(a, key)[i] = x
        else:
            setattr(a, key, val)
    return a


def call_fwd(lib, a):
    return lib.nxattn_fwd(ctypes.byref(a) if a is not None else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), UNSUPPORTED),
    (dict(head_dim=64), UNSUPPORTED),                  # bf16 needs 128
    (dict(dtype=0, head_dim=128), UNSUPPORTED),        # f32 needs 64 or 72
    (dict(heads_q=6, heads_kv=4), INVALID),
    (dict(batch=9), UNSUPPORTED),
    (dict(batch=-1), INVALID),
    (dict(seq_q=-5), INVALID),
    (dict(heads_kv=0), INVALID),
    (dict(q=None), INVALID),
    (dict(q=FAKE + 8), ALIGN),
    (dict(q_strides=(64 * 8 * 128, 8 * 128 + 4, 128)), ALIGN),
    (dict(kv_strides=(-256, 256, 128)), INVALID),
    (dict(prefix_len=(5, 0)), INVALID),                # P > 0 needs a pointer
    (dict(prefix_kv=(FAKE, None)), INVALID),           # pointer needs P > 0
    (dict(prefix_kv=(FAKE + 8, None), prefix_len=(5, 0)), ALIGN),
    (dict(prefix_len=(-1, 0)), INVALID),
    (dict(o=FAKE), INVALID),                           # o overlaps q
    (dict(scale=float("nan")), INVALID),
    # a 64-row key tile must span under 2 GiB (32-bit buffer offsets); the bound itself passes
    # validation up to the overlap check
    (dict(kv_strides=(64 * 2 ** 24, 2 ** 24, 128)), UNSUPPORTED),
    (dict(dtype=0, head_dim=64, kv_strides=(64 * 2 ** 23, 2 ** 23, 64)), UNSUPPORTED),
])
def test_fwd_rejects(lib, kw, code):
    assert call_fwd(lib, fwd_args(**kw)) == code
    assert nx.last_error() != ""


def _bad_global_freq():
    d = binding.rope_desc((64,), (64,), (0,))
    d.global_freq = 2
    return d


def _with_q_rope(a, descs):
    arr = (binding.RopeDesc * len(descs))(*descs)
    a._keep = arr
    a.q_rope = ctypes.cast(arr, ctypes.POINTER(binding.RopeDesc))
    return a


@pytest.mark.parametrize("kw,descs,code", [
    # f32 cannot rotate q on load
    (dict(dtype=0, head_dim=64), [binding.rope_desc((64,), (32,), (0,))] * 2, UNSUPPORTED),
    # grid product must equal seq_q (64)
    (dict(), [binding.rope_desc((8, 4), (32, 32), (0, 0))] * 2, INVALID),
    # 2 * sum(pairs) must equal head_dim (128)
    (dict(), [binding.rope_desc((8, 8), (16, 16), (0, 0))] * 2, INVALID),
    # theta must exceed 1
    (dict(), [binding.rope_desc((64,), (64,), (0,), theta=0.5)] * 2, INVALID),
    # global_freq is 0 or 1
    (dict(), [_bad_global_freq()] * 2, INVALID),
    # a valid q_rope does not skip the other checks (o overlaps q: nothing launches)
    (dict(o=FAKE), [binding.rope_desc((8, 8), (32, 32), (4, 4))] * 2, INVALID),
    # offsets are non-negative
    (dict(), [binding.rope_desc((8, 8), (32, 32), (0, -1))] * 2, INVALID),
    # positions on load stay below 2^24 (the last one here is 2^24)
    (dict(), [binding.rope_desc((8, 8), (32, 32), (0, 0)), binding.rope_desc((8, 8), (32, 32), (2 ** 24 - 7, 0))],
     UNSUPPORTED),
    # offset + grid - 1 must fit int32
    (dict(), [binding.rope_desc((64,), (64,), (2 ** 31 - 10,))] * 2, INVALID),
])
def test_fwd_q_rope_rejects(lib, kw, descs, code):
    assert call_fwd(lib, _with_q_rope(fwd_args(**kw), descs)) == code
    assert nx.last_error() != ""


GB = 1 << 30
WS = FAKE + 8 * GB          # a workspace / lse address clear of q, k, v and o


@pytest.mark.parametrize("kw,code,msg", [
    (dict(lse=FAKE + 8 * GB + 2), ALIGN, "lse"),
    (dict(lse=FAKE), INVALID, "lse overlaps q"),
    (dict(lse=FAKE + (1 << 32) + 64), INVALID, "lse overlaps o"),
    (dict(prefix_only=2), INVALID, "prefix_only"),
    (dict(prefix_only=1), INVALID, "prefix_len"),                     # no prefix at all
    (dict(prefix_only=1, prefix_len=(8, 8), prefix_kv=(FAKE + 2 * GB, FAKE + 3 * GB), k=None, v=None,
          o=FAKE), INVALID, "o overlaps q"),                             # k/v NULL accepted, next check fires
    (dict(num_splits=17), INVALID, "num_splits"),
    (dict(num_splits=-1), INVALID, "num_splits"),
    (dict(num_splits=4), INVALID, "workspace"),                         # no workspace
    (dict(num_splits=4, workspace=WS + 8, workspace_bytes=1 << 30), ALIGN, "workspace"),
    (dict(num_splits=4, workspace=WS, workspace_bytes=1024), INVALID, "workspace_bytes"),
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=1 << 30), INVALID, "workspace overlaps q"),
    (dict(num_splits=4, workspace=WS, workspace_bytes=1 << 30, lse=WS + 4096), INVALID, "overlaps lse"),
])
def test_fwd_lse_split_rejects(lib, kw, code, msg):
    assert call_fwd(lib, fwd_args(**kw)) == code
    assert msg in nx.last_error()


CFG = dict(cfg_out=WS, cfg_strides=(8 * 128, 128), guidance=4.0)   # a valid guidance output


@pytest.mark.parametrize("kw,code,msg", [
    (dict(CFG, dtype=0, head_dim=64), UNSUPPORTED, "BF16 only"),
    (dict(CFG, batch=1), INVALID, "batch 2"),
    (dict(CFG, batch=3), INVALID, "batch 2"),
    (dict(CFG, num_splits=2), UNSUPPORTED, "num_splits"),
    (dict(CFG, guidance=float("inf")), INVALID, "guidance"),
    (dict(CFG, cfg_out=WS + 8), ALIGN, "cfg_out must be 16-byte aligned"),
    (dict(CFG, cfg_strides=(8 * 128, 132)), ALIGN, "cfg stride"),
    (dict(CFG, cfg_strides=(-8, 128)), INVALID, "negative cfg stride"),
    (dict(CFG, cfg_out=FAKE), INVALID, "cfg_out overlaps q"),
    (dict(CFG, cfg_out=FAKE + (1 << 32) + 4096), INVALID, "cfg_out overlaps o"),
    (dict(o=None), INVALID, "NULL q/k/v/o"),                              # o is needed without cfg_out
    (dict(CFG, o=None, lse=WS + 64), INVALID, "cfg_out overlaps lse"),   # o NULL accepted, next check fires
])
def test_fwd_cfg_out_rejects(lib, kw, code, msg):
    assert call_fwd(lib, fwd_args(**kw)) == code
    assert msg in nx.last_error()


def test_fwd_workspace_size(lib):
    n = ctypes.c_int64(-1)
    for ns in (0, 1):
        assert lib.nxattn_fwd_workspace_size(ctypes.byref(fwd_args(num_splits=ns)), ctypes.byref(n)) == OK
        assert n.value == 0
    assert lib.nxattn_fwd_workspace_size(ctypes.byref(fwd_args(num_splits=4)), ctypes.byref(n)) == OK
    rows = 4 * 2 * 64 * 8
    assert rows * (128 + 1) * 4 <= n.value <= rows * (128 + 1) * 4 + 512
    assert binding.fwd_workspace_bytes(2, 64, 8, 128, 4) == n.value
    assert lib.nxattn_fwd_workspace_size(ctypes.byref(fwd_args(num_splits=17)), ctypes.byref(n)) == INVALID
    assert lib.nxattn_fwd_workspace_size(None, ctypes.byref(n)) == INVALID


def merge_call(lib, po, pl, n=None, B=2, S=64, H=8, D=128, pst=None, dtype=1, o=FAKE + 16 * GB, ost=None,
               lse=None):
    n = len(po) if n is None else n
    st = (S * H * D, H * D, D)
    P = (ctypes.c_void_p * max(1, len(po)))(*po)
    L = (ctypes.c_void_p * max(1, len(pl)))(*pl)
    return lib.nxattn_attn_merge(P, L, n, B, S, H, D, (ctypes.c_int64 * 3)(*(pst or st)), dtype, o,
                                 (ctypes.c_int64 * 3)(*(ost or st)), lse, None)


def test_merge_rejects(lib):
    po = [FAKE, FAKE + GB]
    pl = [FAKE + 2 * GB, FAKE + 3 * GB]
    assert merge_call(lib, po, pl, dtype=5) == UNSUPPORTED
    assert merge_call(lib, po, pl, n=0) == INVALID
    assert merge_call(lib, po * 9, pl * 9) == INVALID                 # 18 parts
    assert merge_call(lib, po, pl, D=12) == UNSUPPORTED
    assert merge_call(lib, po, pl, D=264) == UNSUPPORTED
    assert merge_call(lib, po, pl, B=-1) == INVALID
    assert merge_call(lib, [FAKE, None], pl) == INVALID
    assert merge_call(lib, [FAKE + 8, FAKE + GB], pl) == ALIGN
    assert merge_call(lib, po, [FAKE + 2 * GB + 2, FAKE + 3 * GB]) == ALIGN
    assert merge_call(lib, po, pl, o=FAKE + 16 * GB + 8) == ALIGN
    assert merge_call(lib, po, pl, lse=FAKE + 17 * GB + 1) == ALIGN
    assert merge_call(lib, po, pl, pst=(64 * 8 * 128, 8 * 128 + 4, 128)) == ALIGN
    # overlaps: o partly over a part, o exactly a part but with other strides, o over an
    # lse, lse partly over a part's lse, lse over a part's output, lse over o
    assert merge_call(lib, po, pl, o=FAKE + 256) == INVALID
    assert merge_call(lib, po, pl, o=FAKE, ost=(64 * 8 * 256, 8 * 256, 256)) == INVALID
    assert merge_call(lib, po, pl, o=FAKE + 2 * GB) == INVALID
    assert merge_call(lib, po, pl, lse=FAKE + 2 * GB + 64) == INVALID
    assert merge_call(lib, po, pl, lse=FAKE + GB + 64) == INVALID
    assert merge_call(lib, po, pl, lse=FAKE + 16 * GB + 64) == INVALID
    assert "overlaps" in nx.last_error()
    # empty problems return before anything else is looked at
    assert merge_call(lib, po, pl, S=0) == OK


def test_quantize_fp8_rejects(lib):
    f = lib.nxattn_quantize_fp8
    st = (ctypes.c_int64 * 3)(64 * 4 * 128, 4 * 128, 128)
    X, C, E, W = FAKE, FAKE + GB, FAKE + 2 * GB, FAKE + 3 * GB
    ok = dict(x=X, dtype=1, B=2, S=64, H=4, D=128, st=st, c=C, e=E, w=W, wb=1 << 20)
    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["dtype"], a["B"], a["S"], a["H"], a["D"], a["st"], a["c"], a["e"], a["w"], a["wb"], None)
    assert call(dtype=7) == UNSUPPORTED
    assert call(D=12) == UNSUPPORTED
    assert call(H=5000) == UNSUPPORTED
    assert call(B=-1) == INVALID
    assert call(x=None) == INVALID
    assert call(x=X + 8) == ALIGN
    assert call(c=C + 4) == ALIGN
    assert call(wb=4) == INVALID                                 # workspace too small (4096 needed)
    assert call(wb=4095) == INVALID
    assert call(c=X + 64) == INVALID                             # codes overlap x
    assert call(e=C + 100) == INVALID                            # exps overlap codes
    assert call(S=0) == OK
    n = ctypes.c_int64(-1)
    # 32 copies of the 8 maxima, each copy padded to 32 words (one 128-byte line)
    assert lib.nxattn_quantize_fp8_workspace_size(2, 64, 4, ctypes.byref(n)) == OK and n.value == 32 * 32 * 4
    assert lib.nxattn_quantize_fp8_workspace_size(3, 64, 40, ctypes.byref(n)) == OK and n.value == 32 * 128 * 4
    assert lib.nxattn_quantize_fp8_workspace_size(-1, 64, 4, ctypes.byref(n)) == INVALID


def test_rope_quantize_fp8_rejects(lib):
    f = lib.nxattn_rope_quantize_fp8
    Q, K, CQ, CK, EQ, EK, W = (FAKE + i * GB for i in range(7))

    def desc(grid=64, pairs=64, theta=10000.0):
        d = binding.RopeDesc()
        d.n_axes, d.grid[0], d.pairs[0], d.theta = 1, grid, pairs, theta
        return d

    def tensor(x, heads, codes, exps, strides=None):
        t = binding.Fp8Tensor()
        t.x, t.heads, t.codes, t.exps = x, heads, codes, exps
        for i, v in enumerate(strides or (64 * heads * 128, heads * 128, 128)):
            t.strides[i] = v
        return t
    good = [tensor(Q, 8, CQ, EQ), tensor(K, 2, CK, EK)]
    ok = dict(t=good, n=2, dtype=1, B=2, S=64, D=128, r=[desc(), desc()], w=W, wb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        ts = (binding.Fp8Tensor * max(1, len(a["t"])))(*a["t"])
        rs = None if a["r"] is None else (binding.RopeDesc * len(a["r"]))(*a["r"])
        return f(ts, a["n"], a["dtype"], a["B"], a["S"], a["D"], rs, a["w"], a["wb"], None)
    # every rejection below comes before the first launch
    assert call(n=0) == INVALID
    assert call(n=5) == INVALID
    assert call(dtype=7) == UNSUPPORTED
    assert call(D=12) == UNSUPPORTED
    assert call(D=512) == UNSUPPORTED                            # quantizable, but beyond RoPE's 256
    assert call(t=[tensor(Q, 4000, CQ, EQ), tensor(K, 200, CK, EK)]) == UNSUPPORTED   # > 4096 heads in total
    assert call(B=9, r=[desc()] * 9) == UNSUPPORTED
    assert call(B=-1) == INVALID
    assert call(t=[tensor(Q, -1, CQ, EQ), good[1]]) == INVALID
    assert call(t=[good[0], tensor(0, 2, CK, EK)]) == INVALID    # NULL x
    assert call(t=[good[0], tensor(K, 2, 0, EK)]) == INVALID     # NULL codes
    assert call(r=None) == INVALID
    assert b"nxattn_rope_quantize_fp8" in lib.nxattn_last_error()           # errors name the entry point
    assert call(r=[desc(), desc(grid=63)]) == INVALID            # grid product != seq
    assert call(r=[desc(pairs=32), desc()]) == INVALID           # 2 * pairs != head_dim
    assert call(r=[desc(), desc(theta=1.0)]) == INVALID
    assert call(t=[tensor(Q + 8, 8, CQ, EQ), good[1]]) == ALIGN
    assert call(t=[good[0], tensor(K, 2, CK + 4, EK)]) == ALIGN
    assert call(t=[good[0], tensor(K, 2, CK, EK, (64 * 264, 264, 132))]) == ALIGN  # head stride of 264 bytes
    assert call(w=W + 2) == ALIGN
    assert call(wb=32 * 32 * 4 - 1) == INVALID                   # 20 maxima: 32 copies of 32 words
    assert call(t=[good[0], tensor(K, 2, CQ + 64, EK)]) == INVALID   # codes of k overlap codes of q
    for bad in (-1.0, float("inf"), float("nan")):                  # multipliers: 0, or finite > 0
        t = tensor(Q, 8, CQ, EQ)
        t.mult = bad
        assert call(t=[t, good[1]]) == INVALID
    for bad in (-1, 2):                                              # fold_softmax: 0 or 1
        t = tensor(Q, 8, CQ, EQ)
        t.fold_softmax = bad
        assert call(t=[t, good[1]]) == INVALID
    assert call(t=[good[0], tensor(K, 2, Q + 64, EK)]) == INVALID    # codes of k overlap q
    assert call(t=[good[0], tensor(K, 2, CK, EK)], w=K + 128) == INVALID   # workspace overlaps k
    assert call(S=0, r=None) == OK
    assert call(t=[tensor(Q, 0, 0, 0)], n=1, r=None) == OK      # no heads at all
    # block scaling: every tensor with heads has scales and no exps, head_dim % 64 == 0,
    # no workspace
    SQ, SK = FAKE + 8 * GB, FAKE + 9 * GB

    def btensor(x, heads, codes, scales):
        t = tensor(x, heads, codes, 0)
        t.scales = scales
        return t
    bgood = [btensor(Q, 8, CQ, SQ), btensor(K, 2, CK, SK)]
    assert call(t=[bgood[0], good[1]]) == INVALID                # mixed kinds of scale
    both = btensor(K, 2, CK, SK)
    both.exps = EK
    assert call(t=[bgood[0], both]) == INVALID                   # exps and scales on one tensor
    assert call(t=bgood, D=96, r=[desc(pairs=48), desc(pairs=48)]) == UNSUPPORTED   # head_dim % 64
    assert call(t=[bgood[0], btensor(K, 2, CK, CQ + 64)]) == INVALID   # scales overlap codes of q
    assert call(t=bgood, S=0, r=None, w=None, wb=0) == OK        # no workspace needed


def test_rope_quantize_fp8_noalloc_rejects(lib):
    # the variant without a workspace: its static scratch holds 2048 (branch, head) slices;
    # larger problems are refused on the host, before the scratch is looked up
    f = lib.nxattn_rope_quantize_fp8_noalloc
    t = binding.Fp8Tensor()
    t.x, t.heads, t.codes, t.exps = FAKE, 257, FAKE + GB, FAKE + 2 * GB
    for i, v in enumerate((257 * 128, 257 * 128, 128)):
        t.strides[i] = v
    d = binding.RopeDesc()
    d.n_axes, d.grid[0], d.pairs[0], d.theta = 1, 1, 64, 10000.0
    ds = (binding.RopeDesc * 8)(*([d] * 8))
    assert f(ctypes.byref(t), 1, 1, 8, 1, 128, ds, None) == UNSUPPORTED          # 8 * 257 = 2056 slices
    assert b"2048" in lib.nxattn_last_error()
    assert f(None, 1, 1, 8, 1, 128, ds, None) == INVALID
    assert f(ctypes.byref(t), 0, 1, 8, 1, 128, ds, None) == INVALID
    assert f(ctypes.byref(t), 1, 1, -1, 1, 128, ds, None) == INVALID


def test_quantize_fp8_blocks_rejects(lib):
    f = lib.nxattn_quantize_fp8_blocks
    X, C, S_ = FAKE, FAKE + GB, FAKE + 2 * GB
    st = (ctypes.c_int64 * 3)(64 * 4 * 128, 4 * 128, 128)

    def call(x=X, dtype=1, B=2, S=64, H=4, D=128, strides=st, c=C, s=S_):
        return f(x, dtype, B, S, H, D, strides, c, s, None)
    assert call(dtype=5) == UNSUPPORTED
    assert call(D=48) == UNSUPPORTED                             # runs of 32
    assert call(D=2048) == UNSUPPORTED
    assert call(B=-1) == INVALID
    assert call(strides=None) == INVALID
    assert call(c=None) == INVALID and call(s=None) == INVALID
    assert call(x=X + 8) == ALIGN
    assert call(c=C + 4) == ALIGN
    assert call(strides=(ctypes.c_int64 * 3)(64 * 4 * 128, 4 * 128, 132)) == ALIGN   # 264-byte head stride
    assert call(s=C + 100) == INVALID                            # scales overlap codes
    assert call(c=X + 64) == INVALID                             # codes overlap x
    assert call(S=0) == OK
    assert b"nxattn_quantize_fp8_blocks" in lib.nxattn_last_error() or lib.nxattn_last_error() == b""


def fp8_args(**kw):
    a = binding.FwdFp8Args()
    a.batch, a.seq_q, a.heads_q, a.heads_kv, a.head_dim = 2, 64, 8, 2, 128
    a.q8, a.k8, a.v = FAKE, FAKE + GB, FAKE + 2 * GB
    a.q_exp, a.k_exp = FAKE + 3 * GB, FAKE + 3 * GB + 4096
    a.o = FAKE + 4 * GB
    for i, s in enumerate((64 * 2 * 128, 2 * 128, 128)):
        a.v_strides[i] = s
    for i, s in enumerate((64 * 8 * 128, 8 * 128, 128)):
        a.o_strides[i] = s
    for key, val in kw.items():
        if key in ("prefix_len", "prefix_k8", "prefix_v", "v_strides", "o_strides", "prefix_k_scales", "cfg_strides"):
            for i, x in enumerate(val):
                getattr(a, key)[i] = x
        else:
            setattr(a, key, val)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), UNSUPPORTED),
    (dict(batch=9), UNSUPPORTED),
    (dict(heads_q=6, heads_kv=4), INVALID),
    (dict(q8=None), INVALID),
    (dict(q_exp=None), INVALID),
    (dict(q8=FAKE + 8), ALIGN),
    (dict(v_strides=(64 * 2 * 128, 2 * 128 + 4, 128)), ALIGN),
    (dict(prefix_len=(5, 0)), INVALID),                                   # P > 0 needs pointers
    (dict(prefix_len=(5, 0), prefix_k8=(FAKE + 5 * GB, None)), INVALID),  # ... both of them
    (dict(prefix_len=(5, 0), prefix_k8=(FAKE + 5 * GB, None), prefix_v=(FAKE + 6 * GB, None)), INVALID),  # exps
    (dict(o=FAKE + GB), INVALID),                                         # o overlaps k8
    (dict(scale=float("inf")), INVALID),
    # block scales: q_scales and k_scales instead of every exponent
    (dict(q_scales=FAKE + 7 * GB, k_scales=FAKE + 8 * GB), INVALID),      # exponents still set
    (dict(q_exp=None, k_exp=None, q_scales=FAKE + 7 * GB), INVALID),      # k_scales missing
    (dict(k_scales=FAKE + 8 * GB), INVALID),                              # k_scales without q_scales
    (dict(q_exp=None, k_exp=None, q_scales=FAKE + 7 * GB + 2, k_scales=FAKE + 8 * GB), ALIGN),
    (dict(q_exp=None, k_exp=None, q_scales=FAKE + 7 * GB, k_scales=FAKE + 8 * GB, prefix_len=(5, 0),
          prefix_k8=(FAKE + 5 * GB, None), prefix_v=(FAKE + 6 * GB, None)), INVALID),  # prefix scales missing
    (dict(prefix_k_scales=(FAKE + 9 * GB, None)), INVALID),               # prefix scales without a prefix
    (dict(q_exp=None, k_exp=None, q_scales=FAKE + 7 * GB, k_scales=FAKE + 8 * GB, o=FAKE + 8 * GB), INVALID),
    (dict(v_strides=(64 * 2 ** 24, 2 ** 24, 128)), UNSUPPORTED),          # 64 V rows span 2 GiB
])
def test_fwd_fp8_rejects(lib, kw, code):
    assert lib.nxattn_fwd_fp8(ctypes.byref(fp8_args(**kw)), None) == code
    assert nx.last_error() != ""


CFG8 = dict(cfg_out=FAKE + 10 * GB, cfg_strides=(8 * 128, 128), guidance=4.0)   # a valid guidance output


@pytest.mark.parametrize("kw,code,msg", [
    (dict(CFG8, batch=1), INVALID, "batch 2"),
    (dict(CFG8, guidance=float("nan")), INVALID, "guidance"),
    (dict(CFG8, cfg_out=FAKE + 10 * GB + 8), ALIGN, "cfg_out must be 16-byte aligned"),
    (dict(CFG8, cfg_strides=(8 * 128, 132)), ALIGN, "cfg stride"),      # 264 bytes
    (dict(CFG8, cfg_out=FAKE + 4 * GB), INVALID, "outputs overlap"),                  # cfg_out overlaps o
    (dict(o=None), INVALID, "NULL pointer"),                                         # o needed without cfg_out
    (dict(CFG8, o=None, cfg_out=FAKE + GB), INVALID, "an output overlaps an input"),  # o NULL accepted
])
def test_fwd_fp8_cfg_out_rejects(lib, kw, code, msg):
    assert lib.nxattn_fwd_fp8(ctypes.byref(fp8_args(**kw)), None) == code
    assert msg in nx.last_error()


def test_fwd_fp8_q_on_load_rejects(lib):
    # q rotated, folded and block-quantized on load: bf16 q + q_rope instead of q8 and its
    # exponents; the keys take block scales
    descs = (binding.RopeDesc * 2)(*[nx.rope_desc((64,), (64,), (b,)) for b in range(2)])
    Q = FAKE + 9 * GB

    def call(**kw):
        base = dict(q8=None, q_exp=None, k_exp=None, k_scales=FAKE + 8 * GB, q=Q)
        base.update(kw)
        a = fp8_args(**{k: v for k, v in base.items() if k not in ("q_strides", "rope")})
        for i, st in enumerate(base.get("q_strides", (64 * 8 * 128, 8 * 128, 128))):
            a.q_strides[i] = st
        a.q_rope = ctypes.cast(base.get("rope", descs), ctypes.POINTER(binding.RopeDesc))
        return lib.nxattn_fwd_fp8(ctypes.byref(a), None)
    assert call(q8=FAKE) == INVALID                                   # q8 as well
    assert call(q_scales=FAKE + 7 * GB) == INVALID                    # q's scales are formed in the kernel
    assert call(q_folded=1) == INVALID                                # the fold is implied
    assert call(k_scales=None, k_exp=FAKE + 3 * GB + 4096) == INVALID  # keys need block scales
    assert call(q=None) == INVALID
    assert call(q=Q + 8) == ALIGN
    assert call(q_strides=(64 * 8 * 128, 8 * 128 + 4, 128)) == ALIGN
    far = (binding.RopeDesc * 2)(*[nx.rope_desc((64,), (64,), ((1 << 24) - 10,)) for _ in range(2)])
    assert call(rope=far) == UNSUPPORTED                              # positions reach 2^24
    assert b"2^24" in lib.nxattn_last_error()
    bad = (binding.RopeDesc * 2)(*[nx.rope_desc((63,), (64,), (0,)) for _ in range(2)])
    assert call(rope=bad) == INVALID                                  # grid product != seq_q
    assert call(o=Q) == INVALID                                       # o overlaps q
    # the optional copies of the codes and scales formed on load: both or neither, with
    # q_rope only, aligned, overlapping nothing
    assert call(q8_out=FAKE + 10 * GB) == INVALID
    assert call(q8_out=FAKE + 10 * GB + 8, q_scales_out=FAKE + 11 * GB) == ALIGN
    assert call(q8_out=FAKE + 10 * GB, q_scales_out=FAKE + 11 * GB + 2) == ALIGN
    assert call(q8_out=Q, q_scales_out=FAKE + 11 * GB) == INVALID      # overlaps q
    assert call(q8_out=FAKE + 10 * GB, q_scales_out=FAKE + 10 * GB + 64) == INVALID   # overlap each other
    # q without q_rope; codes out without q_rope
    a = fp8_args(q=Q)
    assert lib.nxattn_fwd_fp8(ctypes.byref(a), None) == INVALID
    a = fp8_args(q8_out=FAKE + 10 * GB, q_scales_out=FAKE + 11 * GB)
    assert lib.nxattn_fwd_fp8(ctypes.byref(a), None) == INVALID


def test_fwd_null_args(lib):
    assert lib.nxattn_fwd(None, None) == INVALID


def test_fwd_zero_size_is_a_noop(lib):
    assert call_fwd(lib, fwd_args(batch=0)) == OK
    assert call_fwd(lib, fwd_args(seq_q=0)) == OK
    assert nx.last_error() == ""


# ----------------------------------------------------------------------------- relayout
def test_relayout_rejects(lib):
    f = lib.nxattn_kv_relayout
    assert f(FAKE, FAKE + (1 << 30), 1, 8, 64, 128, 7, 0, None) == UNSUPPORTED
    assert f(FAKE, FAKE + (1 << 30), 1, 8, 64, 128, 1, 2, None) == INVALID
    assert f(FAKE, FAKE + (1 << 30), -1, 8, 64, 128, 1, 0, None) == INVALID
    assert f(None, FAKE, 1, 8, 64, 128, 1, 0, None) == INVALID
    assert f(FAKE, FAKE + 1024, 1, 8, 64, 128, 1, 0, None) == INVALID     # overlap
    assert f(FAKE + 1, FAKE + (1 << 30) + 1, 1, 8, 64, 127, 1, 0, None) == ALIGN
    assert f(FAKE, FAKE, 0, 8, 64, 128, 1, 0, None) == OK                 # empty


# ----------------------------------------------------------------------------- rope
def rope_call(lib, descs, B=1, S=64, H=2, D=64, dtype=0, ptr=FAKE, strides=None):
    st = (ctypes.c_int64 * 3)(*(strides or (S * H * D, H * D, D)))
    arr = (binding.RopeDesc * max(1, len(descs)))(*descs)
    return lib.nxattn_rope_apply(ptr, B, S, H, D, st, dtype, arr, None)


def test_rope_rejects(lib):
    good = nx.rope_desc((64,), (32,), (32,))
    assert rope_call(lib, [nx.rope_desc((8, 9), (16, 16), (0, 0))]) == INVALID        # 72 != 64
    assert rope_call(lib, [nx.rope_desc((64,), (30,), (0,))]) == INVALID              # 60 != 64
    assert rope_call(lib, [nx.rope_desc((64,), (32,), (0,), theta=1.0)]) == INVALID
    bad_axes = nx.rope_desc((64,), (32,), (0,))
    bad_axes.n_axes = 4
    assert rope_call(lib, [bad_axes]) == INVALID
    assert rope_call(lib, [good], D=60) == UNSUPPORTED
    assert rope_call(lib, [good], dtype=3) == UNSUPPORTED
    assert rope_call(lib, [good], ptr=FAKE + 4) == ALIGN
    assert rope_call(lib, [good], strides=(64 * 2 * 64, 2 * 64 + 2, 64)) == ALIGN
    assert rope_call(lib, [good] * 9, B=9) == UNSUPPORTED
    assert rope_call(lib, [good], S=0) == OK


def rope_relayout_call(lib, jobs, n=None, descs=None, S=64, D=64, ptr=FAKE):
    descs = descs or [nx.rope_desc((S,), (D // 2,), (0,))] if S else [nx.rope_desc((64,), (32,), (0,))]
    st = (ctypes.c_int64 * 3)(S * 2 * D, 2 * D, D)
    arr = (binding.RopeDesc * 1)(*descs)
    arr_j = (binding.RelayoutJob * max(1, len(jobs)))()
    for i, kw in enumerate(jobs):
        j = arr_j[i]
        j.src, j.dst = kw.get("src", FAKE + GB), kw.get("dst", FAKE + 2 * GB)
        j.layers, j.kv_heads, j.seq, j.head_dim = kw.get("L", 1), kw.get("H", 2), kw.get("S", 16), kw.get("D", 64)
        j.dir = kw.get("dir", 0)
    return lib.nxattn_rope_apply_relayout(ptr, 1, S, 2, D, st, 0, arr, arr_j if jobs else None,
                                          len(jobs) if n is None else n, None)


@pytest.mark.parametrize("jobs,n,kw,code,msg", [
    ([], 9, {}, INVALID, "n_jobs"),
    ([], 1, {}, INVALID, "NULL jobs"),
    ([dict(dir=2)], None, {}, INVALID, "dir"),
    ([dict(S=-1)], None, {}, INVALID, "negative size"),
    ([dict(src=None)], None, {}, INVALID, "NULL pointer"),
    ([dict(D=62)], None, {}, UNSUPPORTED, "16-byte"),                     # 248-byte rows (f32)
    ([dict(dst=FAKE + 2 * GB + 8)], None, {}, UNSUPPORTED, "16-byte"),
    ([dict(dst=FAKE + 1024)], None, {}, INVALID, "overlaps x"),            # x is 32 KiB at FAKE
    ([dict(src=FAKE + 4096)], None, {}, INVALID, "overlaps x"),
    ([dict(), dict(src=FAKE + 3 * GB, dst=FAKE + 2 * GB + 64)], None, {}, INVALID, "dst of jobs 0 and 1 overlap"),
    ([dict(), dict(src=FAKE + 2 * GB + 64, dst=FAKE + 3 * GB)], None, {}, INVALID, "dst overlaps job 1's src"),
    ([dict()], None, dict(D=60), UNSUPPORTED, "head_dim"),                # the rotation's own checks still apply
])
def test_rope_relayout_rejects(lib, jobs, n, kw, code, msg):
    assert rope_relayout_call(lib, jobs, n, **kw) == code
    assert msg in nx.last_error()


def test_rope_relayout_empty_is_a_noop(lib):
    assert rope_relayout_call(lib, [], S=0) == OK
    assert rope_relayout_call(lib, [dict(L=0)], S=0) == OK              # zero-size job skipped


# ----------------------------------------------------------------------------- extents
BIG = 2 ** 60   # a stride (elements) whose products leave int64 at these sizes


def test_huge_sizes_and_strides_are_rejected(lib):
    """Sizes and strides far beyond any device's memory are refused as unsupported, with
    the extents formed without signed overflow (the UBSan run of this file checks that)."""
    def refused(code):
        return code == UNSUPPORTED and "2^50" in nx.last_error()
    # attention: a q, o or batch stride whose view spans more than 2^50 bytes
    assert refused(call_fwd(lib, fwd_args(q_strides=(BIG, 8 * 128, 128))))
    assert refused(call_fwd(lib, fwd_args(o_strides=(64 * 8 * 128, BIG, 128))))
    assert refused(call_fwd(lib, fwd_args(q_strides=(2 ** 62, 8 * 128, 128))))
    assert refused(lib.nxattn_fwd_fp8(ctypes.byref(fp8_args(v_strides=(BIG, 2 * 128, 128))), None))
    assert refused(lib.nxattn_fwd_fp8(ctypes.byref(fp8_args(o_strides=(64 * 8 * 128, 8 * 128, BIG))), None))
    # merge: strides, and a row count whose lse bytes leave int64
    po, pl = [FAKE, FAKE + GB], [FAKE + 2 * GB, FAKE + 3 * GB]
    assert refused(merge_call(lib, po, pl, pst=(BIG, 8 * 128, 128)))
    assert refused(merge_call(lib, po, pl, B=2 ** 40, S=2 ** 40))
    # relayout: sizes inside the per-dimension limits whose product leaves int64
    assert refused(lib.nxattn_kv_relayout(FAKE, FAKE + (1 << 30), 2 ** 20, 2 ** 20, 2 ** 31, 2 ** 20, 1, 0, None))
    # RoPE: a token stride, and a relayout job of absurd size
    assert refused(rope_call(lib, [nx.rope_desc((64,), (32,), (0,))], strides=(64 * 2 * 64, BIG, 64)))
    assert refused(rope_relayout_call(lib, [dict(L=2 ** 20, H=2 ** 20, S=2 ** 31)]))
    # quantizers
    X, C, E, W = FAKE, FAKE + GB, FAKE + 2 * GB, FAKE + 3 * GB
    st = (ctypes.c_int64 * 3)(BIG, 4 * 128, 128)
    assert refused(lib.nxattn_quantize_fp8(X, 1, 2, 64, 4, 128, st, C, E, W, 1 << 20, None))
    assert refused(lib.nxattn_quantize_fp8_blocks(X, 1, 2, 64, 4, 128, st, C, E, None))


# ----------------------------------------------------------------------------- cfg
def test_cfg_rejects(lib):
    f = lib.nxattn_cfg_combine
    a, b, c = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    assert f(a, b, c, 100, 4.0, 9, None) == UNSUPPORTED
    assert f(a, b, c, -1, 4.0, 1, None) == INVALID
    assert f(a, b, c, 100, float("inf"), 1, None) == INVALID
    assert f(None, b, c, 100, 4.0, 1, None) == INVALID
    assert f(a + 2, b, c, 100, 4.0, 1, None) == ALIGN
    assert f(a, b, a + 16, 100, 4.0, 1, None) == INVALID     # partial overlap with cond
    assert f(a, b, c, 0, 4.0, 1, None) == OK


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(nx.NxattnError):
        nx.nxattn_cfg_combine(x, x, x, 2.0)
