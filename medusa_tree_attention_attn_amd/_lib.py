"""ctypes binding of libtree_attn.so (see include/tree_attn.h).

Argument marshalling only: every step of the verify / accept / commit path
runs in the HIP kernels of the library.  Tensors are PyTorch device tensors
(PyTorch provides device memory and streams); their data pointers and torch's
current stream are handed to the C ABI.  Before a call, the shapes, dtypes,
devices and contiguity of the tensors are checked against the descriptor, so a
kernel never sees an operand smaller than its grid assumes.

The library must be built (python -m medusa_tree_attention_attn_amd.build);
there is no fallback of any kind if it is missing.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # first: the library then binds to the HIP runtime torch loaded

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtree_attn.so")

TA_BF16 = 0
TA_F32 = 1
TA_FLAG_SIMPLE_KERNEL = 1
TA_FLAG_GRID_KERNEL = 2
TA_FLAG_PERSISTENT_KERNEL = 4
TA_FLAG_DECODE_KERNEL = 8

STATUS = {
    0: "TA_OK", -1: "TA_ERR_NULL_POINTER", -2: "TA_ERR_BAD_DIMS", -3: "TA_ERR_DTYPE",
    -4: "TA_ERR_TREE_TOO_LARGE", -5: "TA_ERR_HEAD_DIM", -6: "TA_ERR_HEADS",
    -7: "TA_ERR_BLOCK_SIZE", -8: "TA_ERR_WORKSPACE", -9: "TA_ERR_ROPE_TABLE",
    -10: "TA_ERR_CAPACITY", -11: "TA_ERR_LAUNCH", -12: "TA_ERR_ALIGNMENT",
    -13: "TA_ERR_CHOICES",
}
EXPORTED = (
    "tree_attn_verify", "tree_attn_verify_noalloc", "tree_accept_greedy", "kv_commit_path", "tree_accept_commit",
    "tree_vocab_argmax", "tree_argmax_accept", "tree_accept_typical", "tree_medusa_tree",
    "tree_medusa_candidates",
    "tree_attn_workspace_size", "tree_attn_workspace_init", "tree_attn_plan_info", "tree_attn_rope_table",
    "tree_attn_stream_read", "tree_attn_strerror",
)


class TreeAttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("t_max", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_cos_sin", ctypes.c_void_p),
        ("rope_max_pos", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
    ]


class TreeAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({strerror(code)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m medusa_tree_attention_attn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(TreeAttnDesc)
    sig = {
        "tree_attn_verify": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P]),
        "tree_attn_verify_noalloc": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P]),
        "tree_accept_greedy": (ctypes.c_int, [D, P, P, P, P, P]),
        "kv_commit_path": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "tree_accept_commit": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P]),
        "tree_vocab_argmax": (ctypes.c_int, [D, P, ctypes.c_int32, ctypes.c_int32, P]),
        "tree_argmax_accept": (ctypes.c_int, [D, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]),
        "tree_accept_typical": (ctypes.c_int, [D, P, ctypes.c_int32, ctypes.c_int32, P, P,
                                               ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                               P, P, P, P]),
        "tree_medusa_tree": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, P, P]),
        "tree_medusa_candidates": (ctypes.c_int, [D, P, ctypes.c_int32, P, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  P, P, P, P]),
        "tree_attn_workspace_size": (ctypes.c_size_t, [D]),
        "tree_attn_workspace_init": (ctypes.c_int, [D]),
        "tree_attn_plan_info": (ctypes.c_int, [D, P, P, P]),
        "tree_attn_rope_table": (ctypes.c_int, [ctypes.c_int32, ctypes.c_float,
                                                ctypes.c_int32, P, P]),
        "tree_attn_stream_read": (ctypes.c_int, [P, ctypes.c_size_t, P, P]),
        "tree_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().tree_attn_strerror(int(code)).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(code: int, what: str):
    if code != 0:
        raise TreeAttnError(code, what)


def current_stream_handle(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# ------------------------------------------------------------ descriptor --

def make_desc(*, batch, t_max, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
              num_blocks, max_ctx_len, dtype, rope_table=None, rope_max_pos=0,
              workspace=None, workspace_bytes=0, scale=0.0, stream=None, flags=0,
              block_size=16, split_tokens=0) -> TreeAttnDesc:
    d = TreeAttnDesc()
    d.batch, d.t_max = batch, t_max
    d.num_heads, d.num_kv_heads, d.head_dim = num_heads, num_kv_heads, head_dim
    d.block_size = block_size
    d.max_blocks_per_seq, d.num_blocks, d.max_ctx_len = max_blocks_per_seq, num_blocks, max_ctx_len
    d.dtype = dtype
    d.scale = scale
    d.rope_cos_sin = _ptr(rope_table)
    d.rope_max_pos = rope_max_pos
    d.workspace = _ptr(workspace)
    d.workspace_bytes = workspace_bytes
    d.stream = stream
    d.flags = flags
    d.split_tokens = split_tokens
    return d


def _dtype_of(desc):
    return torch.bfloat16 if desc.dtype == TA_BF16 else torch.float32


def _expect(t, shape, dtype, name):
    if not isinstance(t, torch.Tensor):
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, descriptor expects {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# ---------------------------------------------------------------- calls --

def tree_attn_verify(desc, q, k_new, v_new, kv_pages, block_table, ctx_lens, tree_parent,
                     tree_depth, out):
    B, T, H, Hkv, d = desc.batch, desc.t_max, desc.num_heads, desc.num_kv_heads, desc.head_dim
    dt = _dtype_of(desc)
    _expect(q, (B, T, H, d), dt, "q")
    _expect(k_new, (B, T, Hkv, d), dt, "k_new")
    _expect(v_new, (B, T, Hkv, d), dt, "v_new")
    _expect(kv_pages, (desc.num_blocks, 2, Hkv, 16, d), dt, "kv_pages")
    _expect(block_table, (B, desc.max_blocks_per_seq), torch.int32, "block_table")
    _expect(ctx_lens, (B,), torch.int32, "ctx_lens")
    _expect(tree_parent, (B, T), torch.int32, "tree_parent")
    _expect(tree_depth, (B, T), torch.int32, "tree_depth")
    _expect(out, (B, T, H, d), dt, "out")
    rc = load().tree_attn_verify(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new),
                                 _ptr(kv_pages), _ptr(block_table), _ptr(ctx_lens),
                                 _ptr(tree_parent), _ptr(tree_depth), _ptr(out))
    _check(rc, "tree_attn_verify")


def tree_attn_verify_noalloc(desc, q, k_new, v_new, kv_pages, block_table, ctx_lens,
                             tree_parent, tree_depth, out):
    """tree_attn_verify with the library's static device workspace instead of
    desc.workspace (no allocation in the call)."""
    B, T, H, Hkv, d = desc.batch, desc.t_max, desc.num_heads, desc.num_kv_heads, desc.head_dim
    dt = _dtype_of(desc)
    _expect(q, (B, T, H, d), dt, "q")
    _expect(k_new, (B, T, Hkv, d), dt, "k_new")
    _expect(v_new, (B, T, Hkv, d), dt, "v_new")
    _expect(kv_pages, (desc.num_blocks, 2, Hkv, 16, d), dt, "kv_pages")
    _expect(block_table, (B, desc.max_blocks_per_seq), torch.int32, "block_table")
    _expect(ctx_lens, (B,), torch.int32, "ctx_lens")
    _expect(tree_parent, (B, T), torch.int32, "tree_parent")
    _expect(tree_depth, (B, T), torch.int32, "tree_depth")
    _expect(out, (B, T, H, d), dt, "out")
    rc = load().tree_attn_verify_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new),
                                         _ptr(kv_pages), _ptr(block_table), _ptr(ctx_lens),
                                         _ptr(tree_parent), _ptr(tree_depth), _ptr(out))
    _check(rc, "tree_attn_verify_noalloc")


def tree_accept_greedy(desc, node_argmax, cand_tokens, tree_parent, accept_len, accept_path):
    B, T = desc.batch, desc.t_max
    for t, shp, name in ((node_argmax, (B, T), "node_argmax"), (cand_tokens, (B, T), "cand_tokens"),
                         (tree_parent, (B, T), "tree_parent"), (accept_len, (B,), "accept_len"),
                         (accept_path, (B, T), "accept_path")):
        _expect(t, shp, torch.int32, name)
    rc = load().tree_accept_greedy(ctypes.byref(desc), _ptr(node_argmax), _ptr(cand_tokens),
                                   _ptr(tree_parent), _ptr(accept_len), _ptr(accept_path))
    _check(rc, "tree_accept_greedy")


def kv_commit_path(desc, k_new, v_new, accept_len, accept_path, kv_pages, block_table, ctx_lens):
    B, T, Hkv, d = desc.batch, desc.t_max, desc.num_kv_heads, desc.head_dim
    dt = _dtype_of(desc)
    _expect(k_new, (B, T, Hkv, d), dt, "k_new")
    _expect(v_new, (B, T, Hkv, d), dt, "v_new")
    _expect(accept_len, (B,), torch.int32, "accept_len")
    _expect(accept_path, (B, T), torch.int32, "accept_path")
    _expect(kv_pages, (desc.num_blocks, 2, Hkv, 16, d), dt, "kv_pages")
    _expect(block_table, (B, desc.max_blocks_per_seq), torch.int32, "block_table")
    _expect(ctx_lens, (B,), torch.int32, "ctx_lens")
    rc = load().kv_commit_path(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(accept_len),
                               _ptr(accept_path), _ptr(kv_pages), _ptr(block_table),
                               _ptr(ctx_lens))
    _check(rc, "kv_commit_path")


def tree_accept_commit(desc, node_argmax, cand_tokens, tree_parent, accept_len, accept_path,
                       k_new, v_new, kv_pages, block_table, ctx_lens):
    B, T, Hkv, d = desc.batch, desc.t_max, desc.num_kv_heads, desc.head_dim
    dt = _dtype_of(desc)
    for t, shp, name in ((node_argmax, (B, T), "node_argmax"), (cand_tokens, (B, T), "cand_tokens"),
                         (tree_parent, (B, T), "tree_parent"), (accept_len, (B,), "accept_len"),
                         (accept_path, (B, T), "accept_path")):
        _expect(t, shp, torch.int32, name)
    _expect(k_new, (B, T, Hkv, d), dt, "k_new")
    _expect(v_new, (B, T, Hkv, d), dt, "v_new")
    _expect(kv_pages, (desc.num_blocks, 2, Hkv, 16, d), dt, "kv_pages")
    _expect(block_table, (B, desc.max_blocks_per_seq), torch.int32, "block_table")
    _expect(ctx_lens, (B,), torch.int32, "ctx_lens")
    rc = load().tree_accept_commit(ctypes.byref(desc), _ptr(node_argmax), _ptr(cand_tokens),
                                   _ptr(tree_parent), _ptr(accept_len), _ptr(accept_path),
                                   _ptr(k_new), _ptr(v_new), _ptr(kv_pages), _ptr(block_table),
                                   _ptr(ctx_lens))
    _check(rc, "tree_accept_commit")


def _logits_args(desc, logits):
    B, T = desc.batch, desc.t_max
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise TreeAttnError(-3, f"logits must be bfloat16 or float32, got {logits.dtype}")
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (B, T):
        raise TreeAttnError(-2, f"logits must be [{B}][{T}][vocab], got {tuple(logits.shape)}")
    _expect(logits, tuple(logits.shape), logits.dtype, "logits")
    return (TA_BF16 if logits.dtype == torch.bfloat16 else TA_F32), int(logits.shape[2])


def tree_vocab_argmax(desc, logits, node_argmax):
    dt, V = _logits_args(desc, logits)
    _expect(node_argmax, (desc.batch, desc.t_max), torch.int32, "node_argmax")
    rc = load().tree_vocab_argmax(ctypes.byref(desc), _ptr(logits), dt, V, _ptr(node_argmax))
    _check(rc, "tree_vocab_argmax")


def tree_argmax_accept(desc, logits, cand_tokens, tree_parent, node_argmax, accept_len,
                       accept_path):
    dt, V = _logits_args(desc, logits)
    B, T = desc.batch, desc.t_max
    for t, shp, name in ((cand_tokens, (B, T), "cand_tokens"), (tree_parent, (B, T), "tree_parent"),
                         (node_argmax, (B, T), "node_argmax"), (accept_len, (B,), "accept_len"),
                         (accept_path, (B, T), "accept_path")):
        _expect(t, shp, torch.int32, name)
    rc = load().tree_argmax_accept(ctypes.byref(desc), _ptr(logits), dt, V, _ptr(cand_tokens),
                                   _ptr(tree_parent), _ptr(node_argmax), _ptr(accept_len),
                                   _ptr(accept_path))
    _check(rc, "tree_argmax_accept")


def tree_accept_typical(desc, logits, cand_tokens, tree_parent, node_stats, node_ok,
                        accept_len, accept_path, temperature=1.0, epsilon=0.09, delta=0.3):
    dt, V = _logits_args(desc, logits)
    B, T = desc.batch, desc.t_max
    for t, shp, name in ((cand_tokens, (B, T), "cand_tokens"), (tree_parent, (B, T), "tree_parent"),
                         (node_ok, (B, T), "node_ok"), (accept_len, (B,), "accept_len"),
                         (accept_path, (B, T), "accept_path")):
        _expect(t, shp, torch.int32, name)
    _expect(node_stats, (B, T, 2), torch.float32, "node_stats")
    rc = load().tree_accept_typical(ctypes.byref(desc), _ptr(logits), dt, V, _ptr(cand_tokens),
                                    _ptr(tree_parent), float(temperature), float(epsilon),
                                    float(delta), _ptr(node_stats), _ptr(node_ok),
                                    _ptr(accept_len), _ptr(accept_path))
    _check(rc, "tree_accept_typical")


def choices_array(choices):
    """A list of rank paths -> (int32 numpy [n][max_len] padded with -1)."""
    import numpy as np
    n = len(choices)
    m = max((len(c) for c in choices), default=1)
    a = np.full((max(n, 1), m), -1, dtype=np.int32)
    for i, c in enumerate(choices):
        a[i, :len(c)] = c
    return a


def tree_medusa_tree(choices, topk, num_medusa_heads):
    """A medusa choices list (paths of top-k ranks) -> its node table, int32
    numpy [3][len(choices) + 1] (parent, depth, rank rows; root first, then
    the paths by length, then lexicographically).  Host only: build it once
    per list and pass it to every tree_medusa_candidates call."""
    import numpy as np
    arr = np.ascontiguousarray(choices_array(choices))
    n = len(choices)
    table = np.zeros((3, n + 1), dtype=np.int32)
    n_nodes = ctypes.c_int32(0)
    rc = load().tree_medusa_tree(arr.ctypes.data_as(ctypes.c_void_p), n, arr.shape[1], int(topk),
                                 int(num_medusa_heads), table.ctypes.data_as(ctypes.c_void_p),
                                 ctypes.byref(n_nodes))
    _check(rc, "tree_medusa_tree")
    return table


def tree_medusa_candidates(desc, node_table, head_logits, topk, root_token, cand_tokens,
                           tree_parent, tree_depth):
    """node_table: tree_medusa_tree's result (int32 numpy [3][n_nodes], C
    order)."""
    B, T = desc.batch, desc.t_max
    if head_logits.dtype not in (torch.bfloat16, torch.float32) or head_logits.dim() != 3 \
            or head_logits.shape[0] != B:
        raise TreeAttnError(-2, f"head_logits must be [{B}][heads][vocab] bf16/fp32")
    _expect(head_logits, tuple(head_logits.shape), head_logits.dtype, "head_logits")
    _expect(root_token, (B,), torch.int32, "root_token")
    for t, name in ((cand_tokens, "cand_tokens"), (tree_parent, "tree_parent"),
                    (tree_depth, "tree_depth")):
        _expect(t, (B, T), torch.int32, name)
    if node_table.dtype.name != "int32" or node_table.ndim != 2 or node_table.shape[0] != 3 \
            or not node_table.flags["C_CONTIGUOUS"]:
        raise TreeAttnError(-2, "node_table must be a C-contiguous int32 array [3][n_nodes]")
    rc = load().tree_medusa_candidates(
        ctypes.byref(desc), node_table.ctypes.data, int(node_table.shape[1]), _ptr(head_logits),
        TA_BF16 if head_logits.dtype == torch.bfloat16 else TA_F32, int(head_logits.shape[1]),
        int(head_logits.shape[2]), int(topk), _ptr(root_token), _ptr(cand_tokens),
        _ptr(tree_parent), _ptr(tree_depth))
    _check(rc, "tree_medusa_candidates")


KERNEL_NAMES = {0: "verify_simple_kernel", 1: "verify_mfma_kernel", 2: "verify_stream_kernel",
                3: "verify_decode_kernel"}


def tree_attn_plan_info(desc):
    """(kernel name, splits, split_tokens) tree_attn_verify will use."""
    k, sp, ch = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = load().tree_attn_plan_info(ctypes.byref(desc), ctypes.byref(k), ctypes.byref(sp),
                                    ctypes.byref(ch))
    _check(rc, "tree_attn_plan_info")
    return KERNEL_NAMES[k.value], sp.value, ch.value


def tree_attn_workspace_size(desc) -> int:
    return int(load().tree_attn_workspace_size(ctypes.byref(desc)))


def tree_attn_workspace_init(desc):
    _check(load().tree_attn_workspace_init(ctypes.byref(desc)), "tree_attn_workspace_init")


def tree_attn_rope_table(head_dim, base, max_pos, table, stream=None):
    if isinstance(table, torch.Tensor):
        _expect(table, (max_pos, head_dim // 2, 2), torch.float32, "rope table")
    rc = load().tree_attn_rope_table(int(head_dim), float(base), int(max_pos), _ptr(table), stream)
    _check(rc, "tree_attn_rope_table")


def tree_attn_stream_read(src, sink, nbytes=None):
    """Read-bandwidth probe: stream the device tensor src (its first nbytes,
    default all of it) with the KV stream's loads; sink is an int32 device
    tensor of at least one element.  Enqueued on torch's current stream."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= 1):
        raise ValueError("sink must be an int32 device tensor")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the tensor")
    rc = load().tree_attn_stream_read(_ptr(src), n, _ptr(sink),
                                      current_stream_handle(src.device))
    _check(rc, "tree_attn_stream_read")


def tree_attn_strerror(code: int) -> str:
    return strerror(code)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
