"""MI355X (gfx950) single-token recurrent decode for gated linear-attention
and SSM layers: the gated delta rule (GDN / DeltaNet / KDA) over a
slot-indexed fp32 (or 16-bit) state pool, its buffered and conv-fused forms,
Mamba-1's selective-scan decode, and the multi-token and chunked prefill
passes that fill the same pools.

The compute lives in libssmdec.so (hand-written HIP kernels behind the C ABI
of include/ssmdec.h); this package is its thin ctypes binding. Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built.
"""
from ._binding import (  # noqa: F401
    ACT_CODE,
    DTYPE_CODE,
    EXPORTS,
    LIB_PATH,
    SSMD_CHUNK_SCRATCH_BYTES,
    SsmdError,
    gdn_decode_step,
    gdn_decode_step_buffered,
    gdn_decode_step_conv,
    gdn_chunk_prefill,
    gdn_chunk_prefill_noalloc,
    gdn_chunk_workspace_bytes,
    gdn_fused_recurrent,
    gdn_decode_step_state16,
    kda_decode_step,
    load_library,
    mamba_decode_step,
    mamba_scan,
    mamba_scan_workspace_bytes,
    ssmd_check_slot_indices,
    ssmd_last_error,
    ssmd_stream_copy,
)

__all__ = ["gdn_decode_step", "gdn_decode_step_state16", "gdn_decode_step_buffered", "gdn_decode_step_conv",
           "gdn_fused_recurrent", "gdn_chunk_prefill", "gdn_chunk_prefill_noalloc", "gdn_chunk_workspace_bytes",
           "kda_decode_step", "mamba_decode_step", "mamba_scan", "mamba_scan_workspace_bytes", "ssmd_last_error",
           "ssmd_stream_copy", "SsmdError", "load_library"]
