"""DiT attention hot path for MI355X (gfx950).

Thin Python binding over the C-ABI library ``libdit_attn.so`` (declared in
``include/dit_attn.h``).  Calls raise if the library is not built; there is no
CPU fallback.
"""

from .binding import (  # noqa: F401
    DitError,
    attn_block_fwd,
    attn_block_fwd_merge,
    attn_block_workspace,
    attn_lse_merge,
    attn_patch_fwd,
    attn_patch_fwd_strided,
    attn_ring_fwd,
    cfg_combine,
    cfg_combine_relmae,
    default_scale,
    load,
    status_string,
)
