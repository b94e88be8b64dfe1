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
    return sorted(set(re.findall(r"\b(nxattn_[a-z_]+)\s*\(", txt)))


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
        if key in ("prefix_kv", "prefix_len", "q_strides", "kv_strides", "o_strides"):
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
])
def test_fwd_q_rope_rejects(lib, kw, descs, code):
    assert call_fwd(lib, _with_q_rope(fwd_args(**kw), descs)) == code
    assert nx.last_error() != ""


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
