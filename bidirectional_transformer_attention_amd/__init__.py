"""nxattn for MI355X: non-causal GQA attention over [conditioning KV prefix ++ own tokens]
with RoPE at explicit position offsets and classifier-free guidance, as hand-written HIP
kernels for gfx950 behind a C ABI (include/nxattn.h, libnxattn.so).

The Python side only marshals torch tensors into the C ABI (``binding``) and builds the
library (``build``); ``synth`` draws seeded synthetic inputs; ``pipeline`` chains the
four calls into one attention step of a DiT layer.
"""
from .binding import (  # noqa: F401
    NxattnError,
    RopeDesc,
    fwd_workspace_bytes,
    load,
    nxattn_attn_merge,
    nxattn_cfg_combine,
    nxattn_fwd,
    nxattn_fwd_fp8,
    nxattn_quantize_fp8,
    nxattn_quantize_fp8_blocks,
    nxattn_rope_quantize_fp8,
    nxattn_rope_quantize_fp8_noalloc,
    quantize_fp8_workspace_bytes,
    nxattn_kv_relayout,
    nxattn_rope_apply,
    nxattn_rope_apply_relayout,
    rope_desc,
    status_string,
    last_error,
    version,
)
