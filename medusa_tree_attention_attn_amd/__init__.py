"""Medusa tree-verify step on MI355X (gfx950).

Python face of libtree_attn.so: tree attention over a paged KV cache with a
per-node ancestor mask and depth-offset RoPE, greedy longest-path acceptance,
and the KV commit of the accepted path - all in hand-written HIP kernels.
PyTorch only provides device memory and streams.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    STATUS,
    TA_BF16,
    TA_F32,
    TA_FLAG_SIMPLE_KERNEL,
    TreeAttnDesc,
    TreeAttnError,
    kv_commit_path,
    load,
    make_desc,
    tree_accept_commit,
    tree_accept_greedy,
    tree_accept_typical,
    tree_argmax_accept,
    tree_attn_plan_info,
    tree_attn_rope_table,
    tree_attn_stream_read,
    tree_attn_strerror,
    tree_attn_verify,
    tree_attn_verify_noalloc,
    tree_attn_workspace_init,
    tree_attn_workspace_size,
    tree_medusa_candidates,
    tree_medusa_tree,
    tree_vocab_argmax,
)
from .runtime import TreeVerifier  # noqa: F401
