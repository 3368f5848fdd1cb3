"""ctypes loader for libtreeattn.so.

torch is imported first on purpose: torch ships its own HIP runtime, and loading
it before this library makes the library bind to that same runtime (one HIP
runtime per process, so torch streams and pointers are valid here).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load, see above)

from .build import LIB_PATH


class Shape(ctypes.Structure):
    """Mirror of ta_shape in include/tree_attn.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_tree_nodes", ctypes.c_int32),
        ("max_prefix_len", ctypes.c_int32),
        ("total_tree_nodes", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


EXPORTED = (
    "tree_attn_workspace_size",
    "tree_attn_workspace_init",
    "tree_attn_build_mask",
    "tree_attn_prefix",
    "tree_attn_suffix",
    "tree_attn_merge",
    "tree_attn_verify",
    "tree_attn_verify_noalloc",
    "tree_attn_verify_incache",
    "tree_attn_commit_incache",
    "tree_attn_accept_greedy",
    "tree_attn_commit",
    "tree_attn_get_error",
    "tree_attn_status_string",
    "tree_attn_split_tokens",
    "tree_attn_launch_info",
)

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m tree_attention_verify_attn_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, S, I32, I64, F = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64,
                         ctypes.c_float)
    SP = ctypes.POINTER(Shape)
    sig = {
        "tree_attn_workspace_size": (S, [SP]),
        "tree_attn_split_tokens": (I32, [SP]),
        "tree_attn_launch_info": (I32, [SP, P]),
        "tree_attn_workspace_init": (I32, [P, S, P]),
        "tree_attn_build_mask": (I32, [SP, P, P, P, P, S, P]),
        "tree_attn_prefix": (I32, [SP, P, P, P, P, P, P, P, P, P, S, P]),
        "tree_attn_suffix": (I32, [SP, P, P, P, P, P, P, P, P]),
        "tree_attn_merge": (I32, [I64, I32, I32, P, P, P, P, P, P, P]),
        "tree_attn_verify": (I32, [SP, P, P, P, P, P, P, P, P, P, P, P, P, S, P]),
        "tree_attn_verify_noalloc": (I32, [SP, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        "tree_attn_verify_incache": (I32, [SP, P, P, P, P, P, P, P, P, P, P, S, P]),
        "tree_attn_commit_incache": (I32, [SP, P, P, P, P, P, P, P, P, P, S, P]),
        "tree_attn_accept_greedy": (I32, [SP, P, P, P, P, P, P, P, P, S, P]),
        "tree_attn_commit": (I32, [SP, P, P, P, P, P, P, P, P, P, P, P, I32, P, P, S, P]),
        "tree_attn_get_error": (I32, [P, P]),
        "tree_attn_status_string": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
