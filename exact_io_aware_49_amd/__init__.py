"""MI355X (gfx950) exact attention: fused tiled forward with online softmax and a
recomputing backward, as hand-written HIP kernels behind the C ABI of
include/fa.h (libfa.so).  Python here only marshals arguments.
"""

from .fa import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    LIB_PATH,
    backward,
    decode,
    default_scale,
    fa_bwd,
    fa_bwd_gqa,
    fa_bwd_gqa_workspace_size,
    fa_bwd_noalloc,
    fa_bwd_noalloc_scratch_bytes,
    fa_bwd_workspace_size,
    fa_decode,
    fa_decode_workspace_size,
    fa_fwd,
    fa_fwd_fp8,
    fa_fwd_gqa,
    fa_status_string,
    fa_version,
    forward,
    forward_fp8,
    load_library,
)
