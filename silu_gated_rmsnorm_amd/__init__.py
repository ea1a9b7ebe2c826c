"""SiLU-gated RMSNorm training forward/backward on MI355X (gfx950).

The arithmetic runs in hand-written HIP kernels behind the C-ABI library
``libgated_rmsnorm.so`` (declared in ``include/gated_rmsnorm.h``); this
package only marshals torch tensors into that ABI.  Importing the package
does not load the library; the first call does, and raises if it is absent.
"""
from .binding import (  # noqa: F401
    GatedRMSNormError,
    gated_rmsnorm_bwd,
    gated_rmsnorm_ckpt_step,
    gated_rmsnorm_fwd,
    gated_rmsnorm_workspace_bytes,
    gated_rmsnorm_workspace_init,
    library_path,
    load_library,
    new_workspace,
)

__all__ = [
    "GatedRMSNormError",
    "gated_rmsnorm_bwd",
    "gated_rmsnorm_ckpt_step",
    "gated_rmsnorm_fwd",
    "gated_rmsnorm_workspace_bytes",
    "gated_rmsnorm_workspace_init",
    "library_path",
    "load_library",
    "new_workspace",
]
