"""CPU oracle for the SS1 forward, the SS1 MLP pair and the weight projection
(test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path never does.
"""
from .ss1_oracle import (  # noqa: F401
    SplitMix64,
    bf16_bits_to_f64,
    check_plan,
    dense_expand,
    dims,
    flops,
    forward,
    forward_mirror,
    gelu,
    identity_plan,
    mlp_forward,
    plan,
    plan_index,
    project,
    project_rounded,
    sketch,
    sketch_rounded,
)
