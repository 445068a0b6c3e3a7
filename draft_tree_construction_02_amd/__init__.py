"""MI355X (gfx950) library for DARTree's depth-wise batched draft-supertree
construction, deferred top-B pruning, the ancestor mask, one tree-attention
verification layer and an acceptance walk against a synthetic target.  Compute runs in libdartree.so (HIP); this package holds
the ctypes binding, the build script and the seeded synthetic inputs."""
from ._abi import (  # noqa: F401
    DartreeError, Head, accept_walk, accept_walk_workspace_size, build_supertree,
    build_supertree_workspace_size, build_tree_mask, build_tree_sequential,
    build_tree_sequential_workspace_size,
    corrected_topk, head_step_workspace_size, lib, prune_topB, state_update, timing_enable,
    timing_read, timing_reset, tree_attention_verify, tree_attention_workspace_size)
