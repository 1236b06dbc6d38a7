"""MI355X-native (gfx950) Kimi Delta Attention hot path.

The computation lives in ``libkda.so`` (hand-written HIP kernels behind the C ABI
of ``include/kda.h``); this package is its Python binding.  Importing it does not
touch the GPU; the first call loads the library and fails loudly if it is
missing.
"""
from .kda import (  # noqa: F401
    EXPORTS,
    KDA_BF16,
    KDA_F32,
    LIB_PATH,
    KdaError,
    kda_decode_step,
    kda_device_copy,
    kda_decode_tokens,
    kda_prefill_chunked,
    kda_prefill_workspace_bytes,
    kda_prefill_workspace_bytes_batch,
    kda_short_conv_decode,
    kda_short_conv_prefill,
    kda_state_bytes,
    kda_state_init,
    load,
)
