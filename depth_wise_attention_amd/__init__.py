"""AttnRes depth-routing hot path for AMD Instinct MI355X (gfx950).

The compute lives in libattnres.so (hand-written HIP kernels behind a C ABI,
declared in include/attnres.h).  This package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    BF16,
    F16,
    F32,
    LIB_PATH,
    AttnResError,
    attnres_block_phase1,
    attnres_block_phase2_merge,
    attnres_block_phase2_merge_update,
    attnres_block_msar_phase1,
    attnres_block_msar_phase1_workspace_size,
    attnres_block_msar_phase2,
    attnres_block_msar_phase2_workspace_size,
    attnres_bwd,
    attnres_bwd_workspace_size,
    attnres_full_bwd,
    attnres_full_bwd_workspace_size,
    attnres_full_fwd,
    attnres_full_fwd_workspace_size,
    attnres_last_error,
    attnres_msar_fwd,
    attnres_msar_fwd_workspace_size,
    attnres_set_kernel_policy,
    attnres_version,
    lib,
    mhar_fwd,
    mhar_fwd_chunked,
    mhar_fwd_workspace_size,
)
