"""Ring Attention's per-step online-softmax fold, native on AMD MI355X (gfx950).

The computation lives in libra.so (hand-written HIP kernels behind the C ABI of
include/ra.h); this package is its thin ctypes binding:

* ``ra_state_init``  -- (m, l, o) = (-inf, 0, 0)
* ``ra_fold_block``  -- fold one visiting K/V block into the running state
* ``ra_finalize``    -- O = o / l
* ``ra_ring_forward`` -- all P virtual ring steps for the resident query blocks,
  with the double-buffered K/V hand-off on a side stream
* ``ra_ring_forward_noalloc`` -- the same in the library's static device
  scratch (``NOALLOC_SCRATCH_BYTES``), for callers that cannot allocate
* ``ra_fold_block_causal``, ``ra_ring_forward_causal`` -- the same under a
  causal mask, for contiguous, striped or zig-zag token layouts
* ``ra_ring_forward_ex`` -- the forward that also returns each row's log-sum-exp
* ``ra_ring_backward`` -- dQ, dK, dV on the same ring
* ``ra_ring_workspace_bytes``, ``ra_ring_backward_workspace_bytes``,
  ``ra_last_error``, ``ra_version``
"""

from .binding import (
    CAUSAL_LAYOUTS,
    EXPORTED,
    NOALLOC_SCRATCH_BYTES,
    RA_DTYPE_BF16,
    RA_DTYPE_F32,
    RaError,
    lib_path,
    load,
    ra_finalize,
    ra_fold_block,
    ra_fold_block_causal,
    ra_profile_folds,
    ra_profile_read,
    ra_last_error,
    ra_ring_forward,
    ra_ring_backward,
    ra_ring_backward_workspace_bytes,
    ra_ring_forward_causal,
    ra_ring_forward_ex,
    ra_ring_forward_noalloc,
    ra_ring_workspace_bytes,
    ra_state_init,
    ra_version,
)

__all__ = [
    "CAUSAL_LAYOUTS",
    "EXPORTED",
    "NOALLOC_SCRATCH_BYTES",
    "RA_DTYPE_BF16",
    "RA_DTYPE_F32",
    "RaError",
    "lib_path",
    "load",
    "ra_finalize",
    "ra_fold_block",
    "ra_fold_block_causal",
    "ra_profile_folds",
    "ra_profile_read",
    "ra_last_error",
    "ra_ring_forward",
    "ra_ring_backward",
    "ra_ring_backward_workspace_bytes",
    "ra_ring_forward_causal",
    "ra_ring_forward_ex",
    "ra_ring_forward_noalloc",
    "ra_ring_workspace_bytes",
    "ra_state_init",
    "ra_version",
]
