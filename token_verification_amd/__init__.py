"""MI355X-native batched speculative-decoding verify step.

The computation runs in ``libspecverify.so`` (hand-written HIP for gfx950, C ABI
in ``include/spec_verify.h``). This package only marshals torch tensors into
that ABI: it checks dtypes, shapes and devices, allocates the outputs and a
cached workspace, and passes the current HIP stream. There is no fallback: if
the library is not built, importing the binding raises.
"""
from .binding import (  # noqa: F401
    CERTIFIED,
    GREEDY,
    MARGIN,
    SAMPLE,
    PackedHead,
    SpecVerifyError,
    check_args,
    lib,
    pack_lmhead,
    spec_commit,
    spec_gate,
    spec_verify,
    spec_verify_lmhead,
    spec_verify_lmhead_sample,
    workspace_size,
)
