"""MI355X-native fused relative-position attention forward (HIP, gfx950).

The compute path is the C-ABI library ``librelattn.so`` (include/relattn.h);
``binding`` marshals PyTorch tensors into it.  Importing this package does
not load the library; the first call does, and raises if it is missing.
"""

from .binding import (  # noqa: F401
    EXPORTS,
    RelattnError,
    load_library,
    make_params,
    relattn_fwd,
    relattn_fwd_noalloc,
    relattn_rel_index,
    relattn_t5_thresholds,
    relattn_workspace_bytes,
)
