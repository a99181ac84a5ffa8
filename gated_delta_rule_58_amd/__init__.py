"""MI355X (gfx950) Kimi Delta Attention core.

Thin Python binding over the C ABI of libkda.so (include/kda.h): argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; PyTorch only provides device memory and the current stream.  There
is no fallback path: if libkda.so is missing or cannot be loaded, importing
the binding's entry points raises.
"""
from .binding import (  # noqa: F401
    KdaError,
    KDA_F32,
    KDA_BF16,
    lib,
    lib_path,
    gate,
    gate_backward,
    chunk_prefill,
    chunk_prefill_gated,
    chunk_prefill_gated_static,
    chunk_prefill_workspace_bytes,
    chunk_prefill_backward,
    chunk_prefill_backward_workspace_bytes,
    recurrent_decode,
    recurrent_decode_gated,
    shortconv_l2norm,
    exported_symbols,
)
