"""fp64 CPU oracle for the KDA token mixer (test infrastructure only).

Importable only by the tests, the smoke check and the CPU-baseline leg of the
benchmark.  The GPU library never imports it.
"""
from .kda_oracle import (  # noqa: F401
    CONV_K,
    L2_EPS,
    RMS_EPS,
    conv_norm_reference,
    conv_tail,
    gated_delta_step,
    kda_gate,
    kda_reference,
    kda_reference_backward,
    kda_reference_backward_packed,
    kda_reference_decode_step,
    kda_reference_heads,
    kda_reference_packed,
    l2_normalize,
    output_gate_norm,
    output_gate_norm_backward,
    rms_norm,
    short_conv,
    sigmoid,
    silu,
    softplus,
)
