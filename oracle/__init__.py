"""CPU fp64 oracle of the bidirectional-attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it. It shares no code with the HIP library and imports nothing
from it; both sides only read the same seeded inputs.

Every function evaluates the plain definition in float64 (numpy), with no blocking,
fusion or reordering beyond what the definition states. See ``reference.py``.
"""
from .reference import (  # noqa: F401
    relayout,
    positions,
    rope_angles,
    rope,
    attention,
    attention_weights,
    attention_lse,
    merge_partials,
    cfg_combine,
)
