"""MI355X-native FlashAttention-2 exact attention (gfx950 HIP kernels behind a C ABI).

The library itself is ``libfa2.so`` (C ABI declared in ``include/fa2.h``); this
package only marshals arguments to it.  The library is loaded on first use.
"""
from .binding import (  # noqa: F401
    Fa2Error,
    attention_backward,
    attention_forward,
    fa2_bwd,
    fa2_bwd_workspace_bytes,
    fa2_fwd,
    fa2_status_string,
    lib,
)
