"""RecSA tree attention on AMD Instinct MI355X (gfx950).

The compute path is librecsa.so (hand-written HIP kernels behind a C ABI,
declared in include/recsa.h); `recsa` is its thin Python binding.
"""
from . import recsa  # noqa: F401
from .recsa import (  # noqa: F401
    INT32_MAX, RECSA_DENSE_CAUSAL, RECSA_DENSE_KEYS_ROTATED, RecsaError, Shape, recsa_build_tree, recsa_decode,
    recsa_dense_ref_attn, recsa_dense_workspace_bytes, recsa_level_offset, recsa_rotate_keys,
    recsa_num_levels, recsa_prefill, recsa_sel_width, recsa_tree_bytes, recsa_workspace_bytes, tree_level_views,
)
