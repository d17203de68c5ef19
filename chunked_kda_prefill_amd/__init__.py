"""MI355X-native Kimi Delta Attention (KDA) chunked prefill, forward pass.

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI of
``libkda.so`` (include/kda.h); this package only marshals arguments.  The
library is loaded on first use and its absence is an error.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    KDAError,
    LIB_PATH,
    NOALLOC_WORKSPACE_BYTES,
    chunk_fwd,
    chunk_fwd_fused,
    chunk_fwd_noalloc,
    chunk_fwd_segmented,
    chunk_intra,
    chunk_recurrence,
    chunk_table,
    decode_fwd,
    decode_fwd_fused,
    decode_step_fused,
    gate_cumsum,
    gated_rmsnorm,
    load_library,
    new_workspace,
    validate_inputs,
    workspace_layout,
    workspace_size,
)
