"""Host-side runner of one Medusa tree-verify step on one GPU.

`TreeVerifier` owns what a step needs besides the caller's tensors: the
descriptor, the RoPE (cos, sin) table (filled by the library's own kernel)
and the split-KV workspace (allocated once through PyTorch and zero-filled by
the library).  Each call runs on torch's current stream; nothing here
synchronises with the device or computes anything itself.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import (TA_BF16, TA_F32, kv_commit_path, make_desc, tree_accept_commit,
                   tree_accept_greedy, tree_accept_typical, tree_argmax_accept,
                   tree_medusa_candidates, tree_medusa_tree,
                   tree_vocab_argmax,
                   tree_attn_rope_table, tree_attn_verify, tree_attn_verify_noalloc,
                   tree_attn_workspace_init,
                   tree_attn_workspace_size)

ROPE_BASE = 10000.0


class TreeVerifier:
    def __init__(self, *, batch: int, t_max: int, num_heads: int, num_kv_heads: int,
                 head_dim: int, max_blocks_per_seq: int, num_blocks: int, max_ctx_len: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", rope_base: float = ROPE_BASE,
                 scale: float = 0.0, flags: int = 0, rope_max_pos: Optional[int] = None,
                 split_tokens: int = 0):
        _lib.load()
        self.device = torch.device(device)
        self.dtype = dtype
        self.rope_max_pos = rope_max_pos or (max_ctx_len + t_max)
        stream = _lib.current_stream_handle(self.device)
        self.rope = torch.empty((self.rope_max_pos, head_dim // 2, 2), dtype=torch.float32,
                                device=self.device)
        tree_attn_rope_table(head_dim, rope_base, self.rope_max_pos, self.rope, stream)
        self.desc = make_desc(
            batch=batch, t_max=t_max, num_heads=num_heads, num_kv_heads=num_kv_heads,
            head_dim=head_dim, max_blocks_per_seq=max_blocks_per_seq, num_blocks=num_blocks,
            max_ctx_len=max_ctx_len, dtype=TA_BF16 if dtype == torch.bfloat16 else TA_F32,
            rope_table=self.rope, rope_max_pos=self.rope_max_pos, scale=scale, stream=stream,
            flags=flags, split_tokens=split_tokens)
        nbytes = tree_attn_workspace_size(self.desc)
        self.workspace_bytes_needed = nbytes
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.desc.workspace = self.workspace.data_ptr()
        self.desc.workspace_bytes = self.workspace.numel()
        tree_attn_workspace_init(self.desc)

    def _sync_stream(self):
        self.desc.stream = _lib.current_stream_handle(self.device)

    def verify(self, q, k_new, v_new, kv_pages, block_table, ctx_lens, tree_parent, tree_depth,
               out=None):
        self._sync_stream()
        if out is None:
            out = torch.empty_like(q)
        tree_attn_verify(self.desc, q, k_new, v_new, kv_pages, block_table, ctx_lens,
                         tree_parent, tree_depth, out)
        return out

    def verify_noalloc(self, q, k_new, v_new, kv_pages, block_table, ctx_lens, tree_parent,
                       tree_depth, out):
        """verify() through the allocation-free entry point: the library's
        static device workspace instead of self.workspace, `out` given by the
        caller."""
        self._sync_stream()
        tree_attn_verify_noalloc(self.desc, q, k_new, v_new, kv_pages, block_table, ctx_lens,
                                 tree_parent, tree_depth, out)
        return out

    def accept(self, node_argmax, cand_tokens, tree_parent, accept_len=None, accept_path=None):
        self._sync_stream()
        B, T = self.desc.batch, self.desc.t_max
        if accept_len is None:
            accept_len = torch.empty((B,), dtype=torch.int32, device=self.device)
        if accept_path is None:
            accept_path = torch.empty((B, T), dtype=torch.int32, device=self.device)
        tree_accept_greedy(self.desc, node_argmax, cand_tokens, tree_parent, accept_len,
                           accept_path)
        return accept_len, accept_path

    def commit(self, k_new, v_new, accept_len, accept_path, kv_pages, block_table, ctx_lens):
        self._sync_stream()
        kv_commit_path(self.desc, k_new, v_new, accept_len, accept_path, kv_pages, block_table,
                       ctx_lens)

    def accept_commit(self, node_argmax, cand_tokens, tree_parent, k_new, v_new, kv_pages,
                      block_table, ctx_lens, accept_len=None, accept_path=None):
        """accept() then commit() of its result, in one library launch."""
        self._sync_stream()
        B, T = self.desc.batch, self.desc.t_max
        if accept_len is None:
            accept_len = torch.empty((B,), dtype=torch.int32, device=self.device)
        if accept_path is None:
            accept_path = torch.empty((B, T), dtype=torch.int32, device=self.device)
        tree_accept_commit(self.desc, node_argmax, cand_tokens, tree_parent, accept_len,
                           accept_path, k_new, v_new, kv_pages, block_table, ctx_lens)
        return accept_len, accept_path

    def vocab_argmax(self, logits, node_argmax=None):
        """Greedy token after every node: argmax of logits [B][T][V] over V."""
        self._sync_stream()
        if node_argmax is None:
            node_argmax = torch.empty((self.desc.batch, self.desc.t_max), dtype=torch.int32,
                                      device=self.device)
        tree_vocab_argmax(self.desc, logits, node_argmax)
        return node_argmax

    def argmax_accept(self, logits, cand_tokens, tree_parent, node_argmax=None, accept_len=None,
                      accept_path=None):
        """vocab_argmax() then accept() of its result, in one library launch."""
        self._sync_stream()
        B, T = self.desc.batch, self.desc.t_max
        if node_argmax is None:
            node_argmax = torch.empty((B, T), dtype=torch.int32, device=self.device)
        if accept_len is None:
            accept_len = torch.empty((B,), dtype=torch.int32, device=self.device)
        if accept_path is None:
            accept_path = torch.empty((B, T), dtype=torch.int32, device=self.device)
        tree_argmax_accept(self.desc, logits, cand_tokens, tree_parent, node_argmax, accept_len,
                           accept_path)
        return node_argmax, accept_len, accept_path

    def accept_typical(self, logits, cand_tokens, tree_parent, temperature=1.0, epsilon=0.09,
                       delta=0.3, node_stats=None, node_ok=None, accept_len=None,
                       accept_path=None):
        """Typical acceptance: a child passes when its token's probability
        under softmax(logits / temperature) at the parent exceeds
        min(epsilon, delta * exp(-entropy)).  Returns (node_stats [B][T][2] =
        (log-sum-exp, entropy), node_ok, accept_len, accept_path)."""
        self._sync_stream()
        B, T = self.desc.batch, self.desc.t_max
        if node_stats is None:
            node_stats = torch.empty((B, T, 2), dtype=torch.float32, device=self.device)
        if node_ok is None:
            node_ok = torch.empty((B, T), dtype=torch.int32, device=self.device)
        if accept_len is None:
            accept_len = torch.empty((B,), dtype=torch.int32, device=self.device)
        if accept_path is None:
            accept_path = torch.empty((B, T), dtype=torch.int32, device=self.device)
        tree_accept_typical(self.desc, logits, cand_tokens, tree_parent, node_stats, node_ok,
                            accept_len, accept_path, temperature, epsilon, delta)
        return node_stats, node_ok, accept_len, accept_path

    @staticmethod
    def medusa_tree(choices, topk, num_medusa_heads):
        """Node table of a medusa choices list, built once on the host."""
        return tree_medusa_tree(choices, topk, num_medusa_heads)

    def candidates(self, choices, head_logits, topk, root_token, cand_tokens=None,
                   tree_parent=None, tree_depth=None):
        """Candidate tree from Medusa head logits [B][heads][vocab] laid out by a
        medusa-choices list: either the list itself (paths of top-k ranks,
        numbered on every call) or its node table from medusa_tree() (the
        fast path for a list used every step).  Returns (cand_tokens,
        tree_parent, tree_depth)."""
        if not hasattr(choices, "ctypes"):
            choices = tree_medusa_tree(choices, topk, head_logits.shape[1])
        self._sync_stream()
        B, T = self.desc.batch, self.desc.t_max
        mk = lambda: torch.empty((B, T), dtype=torch.int32, device=self.device)
        cand_tokens = mk() if cand_tokens is None else cand_tokens
        tree_parent = mk() if tree_parent is None else tree_parent
        tree_depth = mk() if tree_depth is None else tree_depth
        tree_medusa_candidates(self.desc, choices, head_logits, topk, root_token, cand_tokens,
                               tree_parent, tree_depth)
        return cand_tokens, tree_parent, tree_depth
