"""CPU oracle for the SS1 forward, the SS1 MLP pair and the weight projection
(test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path never does.
"""
from .ss1_oracle import (  # noqa: F401
    SplitMix64,
    backward,
    backward_dw_mirror,
    bf16_bits_to_f64,
    check_plan,
    E4M3_MAX,
    dense_expand,
    dequantize_fp8_rows,
    e4m3_decode,
    e4m3_encode,
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
    quantize_fp8_rows,
    sketch,
    sketch_rounded,
)
