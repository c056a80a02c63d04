"""C ABI checks that need no GPU.

* The shared library loads and exports every function include/tree_attn.h
  declares.
* Every failure the host can detect returns its TA_ERR_* code before anything
  is enqueued (these calls never reach the HIP runtime, so they run on a
  machine without a GPU; no call here passes a descriptor and pointers that
  would pass validation).
"""
import ctypes
import os
import re
import subprocess

import pytest

import medusa_tree_attention_attn_amd as ta
from medusa_tree_attention_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from medusa_tree_attention_attn_amd import build
        build.build(verbose=False)
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(_lib.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def _desc(**kw):
    base = dict(batch=2, t_max=64, num_heads=4, num_kv_heads=4, head_dim=128,
                max_blocks_per_seq=20, num_blocks=40, max_ctx_len=200, dtype=ta.TA_BF16,
                rope_table=0x1000, rope_max_pos=264)
    base.update(kw)
    return ta.make_desc(**base)


def _verify_rc(lib, desc, null_arg=None):
    args = [0x2000 + 0x100 * i for i in range(9)]
    if null_arg is not None:
        args[null_arg] = None
    return lib.tree_attn_verify(ctypes.byref(desc) if desc is not None else None, *args)


def _commit_rc(lib, desc, null_arg):
    args = [0x2000 + 0x100 * i for i in range(7)]
    args[null_arg] = None
    return lib.kv_commit_path(ctypes.byref(desc), *args)


@pytest.mark.parametrize("kw, code", [
    (dict(t_max=65), -4),
    (dict(t_max=0), -2),
    (dict(batch=0), -2),
    (dict(num_heads=0), -2),
    (dict(num_blocks=0), -2),
    (dict(max_ctx_len=-1), -2),
    (dict(dtype=7), -3),
    (dict(head_dim=96), -5),
    (dict(num_heads=6, num_kv_heads=4), -6),
    (dict(block_size=32), -7),
    (dict(max_blocks_per_seq=12), -10),          # 12*16 < 200
    (dict(rope_table=None), -9),
    (dict(rope_max_pos=263), -9),
])
def test_descriptor_errors(lib, kw, code):
    desc = _desc(**kw)
    assert _verify_rc(lib, desc) == code
    assert lib.tree_attn_workspace_size(ctypes.byref(desc)) == 0
    assert _commit_rc(lib, desc, 0) == code


def test_null_descriptor(lib):
    assert lib.tree_attn_verify(None, *([None] * 9)) == -1
    assert lib.tree_accept_greedy(None, *([None] * 5)) == -1
    assert lib.kv_commit_path(None, *([None] * 7)) == -1
    assert lib.tree_accept_commit(None, *([0x3000] * 10)) == -1
    assert lib.tree_attn_workspace_size(None) == 0
    assert lib.tree_attn_workspace_init(None) == -1


@pytest.mark.parametrize("which", range(9))
def test_verify_null_tensor(lib, which):
    assert _verify_rc(lib, _desc(), null_arg=which) == -1


@pytest.mark.parametrize("which", range(7))
def test_commit_null_tensor(lib, which):
    assert _commit_rc(lib, _desc(), which) == -1


@pytest.mark.parametrize("which", range(5))
def test_accept_null_and_dims(lib, which):
    args = [0x3000 + 0x100 * i for i in range(5)]
    args[which] = None
    assert lib.tree_accept_greedy(ctypes.byref(_desc()), *args) == -1
    good = [0x3000 + 0x100 * i for i in range(5)]
    assert lib.tree_accept_greedy(ctypes.byref(_desc(t_max=65)), *good) == -4
    assert lib.tree_accept_greedy(ctypes.byref(_desc(batch=0)), *good) == -2


@pytest.mark.parametrize("which", range(10))
def test_accept_commit_null_and_checks(lib, which):
    args = [0x3000 + 0x100 * i for i in range(10)]
    args[which] = None
    assert lib.tree_accept_commit(ctypes.byref(_desc()), *args) == -1
    good = [0x3000 + 0x100 * i for i in range(10)]
    assert lib.tree_accept_commit(ctypes.byref(_desc(t_max=65)), *good) == -4
    assert lib.tree_accept_commit(ctypes.byref(_desc(batch=0)), *good) == -2
    bad = list(good)
    bad[5] += 2                                   # k_new misaligned
    assert lib.tree_accept_commit(ctypes.byref(_desc()), *bad) == -12


def test_argmax_entry_checks(lib):
    good = [0x3000, 0, 32000, 0x4000]
    d = ctypes.byref(_desc())
    assert lib.tree_vocab_argmax(None, *good) == -1
    assert lib.tree_vocab_argmax(d, None, 0, 32000, 0x4000) == -1
    assert lib.tree_vocab_argmax(d, 0x3000, 0, 32000, None) == -1
    assert lib.tree_vocab_argmax(d, 0x3000, 7, 32000, 0x4000) == -3     # dtype
    assert lib.tree_vocab_argmax(d, 0x3000, 0, 0, 0x4000) == -2         # vocab
    assert lib.tree_vocab_argmax(ctypes.byref(_desc(t_max=65)), *good) == -4
    args = [0x3000, 0, 32000] + [0x4000 + 0x100 * i for i in range(5)]
    for which in (0, 3, 4, 5, 6, 7):
        bad = list(args)
        bad[which] = None
        assert lib.tree_argmax_accept(d, *bad) == -1
    bad = list(args)
    bad[1] = 2
    assert lib.tree_argmax_accept(d, *bad) == -3
    bad = list(args)
    bad[2] = 0
    assert lib.tree_argmax_accept(d, *bad) == -2


def test_typical_entry_checks(lib):
    d = ctypes.byref(_desc())
    # logits, dtype, vocab, cand, parent, temperature, epsilon, delta, stats, ok, len, path
    args = [0x3000, 0, 32000, 0x4000, 0x4100, 1.0, 0.09, 0.3, 0x4200, 0x4300, 0x4400, 0x4500]
    assert lib.tree_accept_typical(None, *args) == -1
    for which in (0, 3, 4, 8, 9, 10, 11):
        bad = list(args)
        bad[which] = None
        assert lib.tree_accept_typical(d, *bad) == -1
    for which, value, code in ((1, 5, -3), (2, 0, -2), (5, 0.0, -2), (5, -1.0, -2),
                               (5, float("inf"), -2), (6, float("nan"), -2),
                               (7, float("inf"), -2), (8, 0x4204, -12)):
        bad = list(args)
        bad[which] = value
        assert lib.tree_accept_typical(d, *bad) == code, (which, value)
    assert lib.tree_accept_typical(ctypes.byref(_desc(t_max=65)), *args) == -4
    assert lib.tree_accept_typical(ctypes.byref(_desc(batch=0)), *args) == -2


def _tree_rc(lib, choices, topk=10, heads=4, n=None):
    import numpy as np
    from medusa_tree_attention_attn_amd._lib import choices_array
    arr = np.ascontiguousarray(choices_array(choices))
    table = np.full((3, 65), 77, dtype=np.int32)
    nn = ctypes.c_int32(-5)
    rc = lib.tree_medusa_tree(arr.ctypes.data_as(ctypes.c_void_p),
                              len(choices) if n is None else n, arr.shape[1], topk, heads,
                              table.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nn))
    return rc, table, nn.value


def test_medusa_choices_validated_on_host(lib):
    """Every rejection happens on the host; outputs stay untouched."""
    for choices, kw, code in (
            ([(0,), (0,)], {}, -13),                            # duplicate path
            ([(0,), (1, 0)], {}, -13),                          # prefix (1,) missing
            ([(0,), (10,)], {}, -13),                           # rank >= topk
            ([(0,), (0, 0), (0, 0, 0), (0, 0, 0, 0), (0, 0, 0, 0, 0)], {}, -13),  # > 4 heads
            ([(0,)], dict(topk=17), -2),                        # topk > 16
            ([(0,)], dict(heads=0), -2),
            ([(i,) for i in range(8)] + [(i, j) for i in range(8) for j in range(8)],
             dict(topk=8), -4)):                                # 73 nodes > 64
        rc, table, nn = _tree_rc(lib, choices, **kw)
        assert rc == code, choices
        assert nn == -5 and (table == 77).all()
    import numpy as np
    gap = np.array([[0, -1, 1]], dtype=np.int32)               # -1 then a rank
    out = np.zeros((3, 2), dtype=np.int32)
    nn = ctypes.c_int32(0)
    assert lib.tree_medusa_tree(gap.ctypes.data_as(ctypes.c_void_p), 1, 3, 4, 4,
                                out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nn)) == -13
    assert lib.tree_medusa_tree(None, 1, 1, 4, 4, out.ctypes.data_as(ctypes.c_void_p),
                                ctypes.byref(nn)) == -1


def test_medusa_tree_numbering_matches_oracle(lib):
    """The library's node numbering is the oracle's (root, then paths by
    length, then lexicographically), on lists given in shuffled order."""
    import numpy as np
    from oracle.candidates import choice_tree
    from synth import make_choices
    for seed, n, depth, k in ((0, 63, 4, 10), (1, 20, 5, 3), (2, 1, 1, 1), (3, 40, 2, 16)):
        choices = make_choices(seed, n=n, max_depth=depth, topk=k)
        order = np.random.default_rng(seed).permutation(len(choices))
        shuffled = [choices[i] for i in order]
        rc, table, nn = _tree_rc(lib, shuffled, topk=k, heads=depth)
        assert rc == 0 and nn == n + 1
        paths, parent, dep = choice_tree(choices)
        flat = table.reshape(-1)[:3 * nn].reshape(3, nn)   # the call writes [3][n_nodes]
        assert np.array_equal(flat[0], parent) and np.array_equal(flat[1], dep)
        assert flat[2].tolist() == [0] + [p[-1] for p in paths]
    rc, table, nn = _tree_rc(lib, [], topk=4)
    assert rc == 0 and nn == 1 and table.reshape(-1)[:3].tolist() == [-1, 0, 0]


def _cand_rc(lib, table, topk=10, heads=4, vocab=32000, t_max=64):
    import numpy as np
    table = np.ascontiguousarray(table, dtype=np.int32)
    return lib.tree_medusa_candidates(
        ctypes.byref(_desc(t_max=t_max)), table.ctypes.data_as(ctypes.c_void_p), table.shape[1],
        0x3000, 0, heads, vocab, topk, 0x4000, 0x5000, 0x6000, 0x7000)


def test_medusa_candidates_checks_the_table(lib):
    """Every rejection happens before anything is enqueued (no device here)."""
    # parent, depth, rank rows of root -> (0,) -> (0, 0)
    good = [[-1, 0, 1], [0, 1, 2], [0, 0, 0]]
    for bad in ([[0, 0, 1], [0, 1, 2], [0, 0, 0]],          # root with a parent
                [[-1, 0, 1], [1, 1, 2], [0, 0, 0]],         # root depth != 0
                [[-1, 2, 1], [0, 1, 2], [0, 0, 0]],         # parent after the child
                [[-1, 0, 1], [0, 1, 3], [0, 0, 0]],         # depth != parent's + 1
                [[-1, 0, 1], [0, 1, 2], [0, 10, 0]],        # rank >= topk
                [[-1, 0, 1], [0, 1, 2], [0, -1, 0]],        # negative rank
                [[-1, 0, 0], [0, 1, 1], [0, 3, 3]]):        # two siblings of one rank
        assert _cand_rc(lib, bad) == -13, bad
    chain = [[-1, 0, 1, 2, 3, 4], [0, 1, 2, 3, 4, 5], [0] * 6]
    assert _cand_rc(lib, chain) == -13                       # deeper than 4 heads
    assert _cand_rc(lib, good, t_max=2) == -4                # 3 nodes > t_max
    assert _cand_rc(lib, good, topk=17) == -2                # topk > 16
    assert _cand_rc(lib, good, topk=8, vocab=7) == -2        # topk > vocab
    assert _cand_rc(lib, good, heads=0) == -2
    assert lib.tree_medusa_candidates(ctypes.byref(_desc()), None, 3, 0x3000, 0, 4, 100, 4,
                                      0x4000, 0x5000, 0x6000, 0x7000) == -1


def test_plan_info_follows_flags(lib):
    """The kernel choice is a host-side rule: forced by the flags, else the
    grid kernel (the persistent kernel only when forced); splits come from
    the context bound."""
    out = [ctypes.c_int32() for _ in range(3)]
    refs = [ctypes.byref(x) for x in out]
    assert lib.tree_attn_plan_info(ctypes.byref(_desc()), *refs) == 0
    # grid kernel; a 200-token bound over 8 pairs: two splits of 128 tokens
    assert (out[0].value, out[1].value, out[2].value) == (1, 2, 128)
    assert lib.tree_attn_plan_info(ctypes.byref(_desc(max_ctx_len=128)), *refs) == 0
    assert (out[1].value, out[2].value) == (1, 128)            # fits one split
    assert lib.tree_attn_plan_info(ctypes.byref(_desc(flags=4)), *refs) == 0
    assert out[0].value == 2                                  # persistent forced
    assert lib.tree_attn_plan_info(ctypes.byref(_desc(flags=1)), *refs) == 0
    assert out[0].value == 0                                  # plain kernel
    desc = _desc(max_ctx_len=4000, max_blocks_per_seq=260, rope_max_pos=4064)
    assert lib.tree_attn_plan_info(ctypes.byref(desc), *refs) == 0
    assert out[1].value > 1 and out[1].value * out[2].value >= 4000
    assert lib.tree_attn_plan_info(ctypes.byref(desc), None, None, None) == 0
    assert lib.tree_attn_plan_info(None, *refs) == -1
    # one sequence, 32 heads, 1024 tokens: 512 / 32 = 16 splits would fit the
    # resident slots, but a split holds at least 128 tokens: 8 of 128
    desc = _desc(batch=1, num_heads=32, num_kv_heads=32, max_ctx_len=1024,
                 max_blocks_per_seq=68, num_blocks=80, rope_max_pos=1088)
    assert lib.tree_attn_plan_info(ctypes.byref(desc), *refs) == 0
    assert (out[0].value, out[1].value, out[2].value) == (1, 8, 128)


def test_one_node_trees_take_the_decode_kernel(lib):
    """t_max == 1 (bf16, head_dim 128): the decode kernel (whole contexts, no
    workspace) up to a 1024-token bound or when forced, the grid kernel
    above; the MFMA flags and the plain flag still force their kernels."""
    out = [ctypes.c_int32() for _ in range(3)]
    refs = [ctypes.byref(x) for x in out]
    desc = _desc(t_max=1, max_ctx_len=1024, max_blocks_per_seq=260, rope_max_pos=4064)
    assert lib.tree_attn_plan_info(ctypes.byref(desc), *refs) == 0
    assert out[0].value == 3 and out[1].value == 1 and out[2].value >= 1024
    assert lib.tree_attn_workspace_size(ctypes.byref(desc)) == 0
    desc = _desc(t_max=1, max_ctx_len=4000, max_blocks_per_seq=260, rope_max_pos=4064)
    assert lib.tree_attn_plan_info(ctypes.byref(desc), *refs) == 0 and out[0].value == 1
    desc = _desc(t_max=1, max_ctx_len=4000, max_blocks_per_seq=260, rope_max_pos=4064, flags=8)
    assert lib.tree_attn_plan_info(ctypes.byref(desc), *refs) == 0
    assert out[0].value == 3 and out[1].value == 1 and out[2].value >= 4000
    assert lib.tree_attn_workspace_size(ctypes.byref(desc)) == 0
    for flags, kernel in ((2, 1), (4, 2), (1, 0)):
        d = _desc(t_max=1, flags=flags)
        assert lib.tree_attn_plan_info(ctypes.byref(d), *refs) == 0
        assert out[0].value == kernel, flags
    d = _desc(t_max=1, head_dim=64)                        # not the MFMA shape
    assert lib.tree_attn_plan_info(ctypes.byref(d), *refs) == 0 and out[0].value == 0


def test_workspace_requirement(lib):
    # long contexts over few (sequence, head) pairs: the plan splits them
    desc = _desc(max_ctx_len=4000, max_blocks_per_seq=260, rope_max_pos=4064)
    need = lib.tree_attn_workspace_size(ctypes.byref(desc))
    assert need > 0
    desc.workspace = 0x5000
    desc.workspace_bytes = need - 1
    assert _verify_rc(lib, desc) == -8
    desc.workspace = None
    desc.workspace_bytes = need
    assert _verify_rc(lib, desc) == -8


def test_misaligned_tensor_pointers(lib):
    desc = _desc()
    need = lib.tree_attn_workspace_size(ctypes.byref(desc))
    desc.workspace = 0x100000
    desc.workspace_bytes = need
    for which in (0, 1, 2, 3, 8):                 # q, k_new, v_new, kv_pages, out
        args = [0x2000 + 0x100 * i for i in range(9)]
        args[which] += 8
        assert lib.tree_attn_verify(ctypes.byref(desc), *args) == -12
    args = [0x2000 + 0x100 * i for i in range(7)]
    args[0] += 2                                  # k_new
    assert lib.kv_commit_path(ctypes.byref(desc), *args) == -12
    desc2 = _desc(rope_table=0x1004)
    desc2.workspace, desc2.workspace_bytes = 0x100000, need
    assert _verify_rc(lib, desc2) == -12


def test_workspace_size_grows_with_context(lib):
    a = lib.tree_attn_workspace_size(ctypes.byref(_desc(max_ctx_len=128)))   # one split
    b = lib.tree_attn_workspace_size(ctypes.byref(_desc(max_ctx_len=4000, max_blocks_per_seq=260,
                                                        rope_max_pos=4064)))
    assert b >= a
    simple = lib.tree_attn_workspace_size(ctypes.byref(_desc(flags=ta.TA_FLAG_SIMPLE_KERNEL,
                                                               max_ctx_len=4000,
                                                               max_blocks_per_seq=260,
                                                               rope_max_pos=4064)))
    assert simple == 0                        # the plain kernel needs no workspace
    f32 = lib.tree_attn_workspace_size(ctypes.byref(_desc(dtype=ta.TA_F32)))
    assert f32 == 0
    assert a == 256 and b > 256               # MFMA: work counters, then split partials


def test_rope_table_errors(lib):
    assert lib.tree_attn_rope_table(128, 10000.0, 10, None, None) == -1
    assert lib.tree_attn_rope_table(96, 10000.0, 10, 0x1000, None) == -5
    assert lib.tree_attn_rope_table(128, 10000.0, 0, 0x1000, None) == -2
    assert lib.tree_attn_rope_table(128, 1.0, 10, 0x1000, None) == -2


def test_strerror_covers_every_code(lib):
    for code in _lib.STATUS:
        msg = _lib.strerror(code)
        assert msg and msg != "unknown status"
    assert _lib.strerror(-99) == "unknown status"


def test_binding_raises_with_code(lib):
    desc = _desc(t_max=65)
    with pytest.raises(ta.TreeAttnError) as e:
        ta.tree_attn_verify(desc, *[0x2000] * 9)
    assert e.value.code == -4


def test_noalloc_rejects_a_plan_beyond_its_static_workspace(lib):
    """The allocation-free verify keeps its split partials in a static 32 MiB
    device array; a plan that needs more is refused on the host, before any
    HIP call (no GPU is touched here)."""
    d = _desc(batch=512, num_heads=32, num_kv_heads=32, max_ctx_len=65536,
              max_blocks_per_seq=4096, num_blocks=1 << 20, rope_max_pos=65536 + 64,
              split_tokens=512)
    assert _lib.tree_attn_workspace_size(d) > 32 << 20
    args = [0x2000 + 0x100 * i for i in range(9)]
    assert lib.tree_attn_verify_noalloc(ctypes.byref(d), *args) == -8


@pytest.mark.parametrize("kw, code", [(dict(t_max=65), -4), (dict(head_dim=96), -5),
                                      (dict(block_size=8), -7)])
def test_noalloc_descriptor_errors(lib, kw, code):
    d = _desc(**kw)
    args = [0x2000 + 0x100 * i for i in range(9)]
    assert lib.tree_attn_verify_noalloc(ctypes.byref(d), *args) == code
    assert lib.tree_attn_verify_noalloc(None, *args) == -1
