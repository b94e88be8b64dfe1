"""The ctypes structures of the Python binding against the C header (CPU only).

A small C program, compiled with the host compiler against include/nxattn.h, prints the
size and the offset of every field of each argument struct; the binding's ctypes
definitions must agree field for field, so a field added on one side only (which would
shift every later field the library reads) fails here rather than on a GPU.
"""
import ctypes
import json
import os
import shutil
import subprocess

import pytest

from bidirectional_transformer_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

# C struct name -> binding class
STRUCTS = {
    "nxattn_rope_desc": binding.RopeDesc,
    "nxattn_fp8_tensor": binding.Fp8Tensor,
    "nxattn_fwd_args": binding.FwdArgs,
    "nxattn_fwd_fp8_args": binding.FwdFp8Args,
    "nxattn_relayout_job": binding.RelayoutJob,
}


def _c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("no host C compiler or HIP headers")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "nxattn.h"', "int main(void) {",
             '  printf("{");']
    first = True
    for cname, cls in STRUCTS.items():
        entries = [f'\\"size\\": %zu'] + [f'\\"{f}\\": %zu' for f, _ in cls._fields_]
        args = [f"sizeof({cname})"] + [f"offsetof({cname}, {f})" for f, _ in cls._fields_]
        sep = "" if first else ", "
        first = False
        lines.append(f'  printf("{sep}\\"{cname}\\": {{{", ".join(entries)}}}", {", ".join(args)});')
    lines += ['  printf("}\\n");', "  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                        ROCM_INCLUDE, str(src), "-o", str(exe)], capture_output=True, text=True)
    # a binding field the header lacks fails to compile (offsetof of an unknown member)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout)


def test_binding_structs_match_header(tmp_path):
    c = _c_layout(tmp_path)
    for cname, cls in STRUCTS.items():
        got = {f: getattr(cls, f).offset for f, _ in cls._fields_}
        got["size"] = ctypes.sizeof(cls)
        # a header field the binding lacks shows as a size (or later offset) mismatch
        assert got == c[cname], (cname, {k: (got[k], c[cname][k]) for k in got if got[k] != c[cname][k]})

