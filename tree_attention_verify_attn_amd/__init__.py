"""MI355X (gfx950) split tree-verify attention.

A draft tree's queries attend to their sequence's committed prefix (paged KV
cache, no mask) and to the tree tokens on their root path (ancestor-or-self
mask); the two pieces are merged exactly by log-sum-exp.  After verification,
``accept_greedy`` picks the accepted root path of each tree and ``commit``
appends its K/V rows to the paged cache; ``verify_incache`` and
``commit_incache`` serve the layout with the tree rows already in the cache.  All arithmetic runs in
hand-written HIP kernels behind the C ABI of ``libtreeattn.so``
(``include/tree_attn.h``); this package only marshals arguments.
"""
from .api import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    TreeAttnError,
    accept_greedy,
    alloc_workspace,
    commit,
    commit_incache,
    build_mask,
    get_error,
    make_shape,
    merge,
    prefix,
    split_tokens,
    launch_info,
    status_string,
    suffix,
    verify,
    verify_incache,
    workspace_init,
    workspace_size,
)
from .build import LIB_PATH, build_library  # noqa: F401
