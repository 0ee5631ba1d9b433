"""Kimi Delta Attention (KDA) token mixer for AMD Instinct MI355X (gfx950).

The computation runs in libkda.so (hand-written HIP kernels behind a C ABI,
``include/kda.h``); this package only marshals torch tensors into that ABI.
There is no Python or CPU fallback: if the library is not built, calls raise.
"""
from ._lib import (  # noqa: F401
    KDA_BF16,
    KDA_FP32,
    KDA_OK,
    KdaError,
    LIB_PATH,
    conv_norm_args,
    decode_args,
    declared_functions,
    kda_abi_version,
    kda_conv_norm,
    kda_decode_raw,
    kda_decode_step,
    backward_args,
    kda_backward_workspace_bytes,
    kda_prefill,
    kda_prefill_backward,
    kda_prefill_backward_raw,
    kda_validate_backward,
    kda_prefill_raw,
    kda_prefill_stage,
    kda_prefill_workspace_bytes,
    kda_status_str,
    kda_validate_conv_norm,
    kda_validate_decode,
    kda_validate_prefill,
    load,
    prefill_args,
)
