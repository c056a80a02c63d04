"""CPU oracle for the Medusa tree-verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, helpers or table generators); both sides only consume the same seeded
inputs from `synth`.

What it computes, step by step (plain definitions, no blocking or fusion):

* `rope_table`, `rope_exact`, `rope_pinned` - rotary position embedding with
  positions offset by node depth.
* `ancestors`, `verify` - tree attention over the paged KV cache plus each
  node's own ancestors (self included), fp64 explicit masked softmax.
* `accept_greedy` - longest matching root-to-node path, sequential walk.
* `commit` - write the accepted path's K/V rows into their page slots.

Pins (see tests/test_oracle_*.py): chain tree == causal attention, every node
== brute force over its own root-to-node path, T=1 == single-query decode,
invariants (block-table permutation, non-ancestor independence, V=1, one-hot V,
RoPE relative-position property), acceptance == exhaustive path enumeration on
all trees with T <= 7 and every edge-match pattern, commit == closed-form slot
arithmetic with bit-level fp32/bf16 emulation.
"""
from .tree_verify import (  # noqa: F401
    PAD_PARENT,
    ROPE_BASE,
    accept_greedy,
    ancestors,
    bf16_bits_to_f32,
    commit,
    f32_to_bf16_bits,
    gather_context,
    rope_exact,
    rope_pinned,
    rope_table,
    verify,
    verify_head,
)
