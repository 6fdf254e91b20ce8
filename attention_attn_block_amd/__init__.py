"""DiT attention hot path for MI355X (gfx950): thin Python binding over the
C-ABI library ``libdit_attn.so``.  See ``include/dit_attn.h`` for the calls."""
