"""fp64 CPU oracle (test infrastructure only; see ``oracle.ref``)."""

from .ref import (  # noqa: F401
    decode,
    ref_attn,
    ref_block_fold,
    ref_cfg,
    ref_cfg_relmae,
    ref_lse_merge,
    ref_patch,
    ref_patch_strided,
)
