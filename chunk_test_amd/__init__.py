"""LaCT large-chunk test-time-training layer on MI355X (gfx950).

The compute path is ``liblact.so`` (HIP kernels behind the C ABI in
``include/lact.h``); ``chunk_test_amd.lact`` is its ctypes binding.
"""

from .lact import (  # noqa: F401
    Config,
    LactError,
    alloc_workspace,
    backward_workspace_bytes,
    lact_apply,
    lact_chunked_backward,
    lact_block_forward,
    lact_chunked_forward,
    lact_chunked_forward_noalloc,
    lact_update,
    lact_window_attention,
    load_library,
    mfma_path,
    noalloc_scratch_bytes,
    profile_enable,
    profile_read,
    workspace_bytes,
)
