"""MI355X (gfx950) SVDQuant W4A4 linear layer and AWQ-style W4A16 layer.

The layer runs in hand-written HIP kernels behind a C ABI (include/svdq.h,
built into ``_lib/libsvdq.so``); :mod:`.capi` is the Python binding with
the same function names, :mod:`.layer` wraps them into layer objects that
own their output buffers, and :mod:`.synth` draws seeded synthetic inputs.
"""
from .capi import (SVDQ_INT4, SVDQ_NVFP4, SvdqError, awq_gemv_w4a16, svdq_abi_version,  # noqa: F401
                   svdq_debug_group_sums, svdq_gemm_w4a4, svdq_last_error, svdq_quantize_act,
                   svdq_status_string)
