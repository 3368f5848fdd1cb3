"""Seeded synthetic inputs for the step after verification: greedy acceptance
of a tree path and committing the accepted path's K/V into the paged cache.

Input preparation only (random draws and layout); no acceptance or commit
logic lives here.

Recipe (the pages give no token statistics; these are plain readings):

* Token ids are int32 in [0, vocab).  ``target_argmax[i]`` is the target
  model's greedy next token at tree node i, drawn uniformly.
* Draft tokens: every node's children are ranked in index order.  With
  probability ``p_match`` (per parent) the rank-0 child carries the parent's
  ``target_argmax`` (it will be accepted if the parent is); every other child
  carries a different token (``argmax + rank`` or ``argmax + rank + 1``,
  modulo vocab), so siblings never share a token, as in a top-k draft tree.
  Roots carry a uniform token.
* Commit state: the verify batch is built with spare pool blocks and extra
  block-table columns; the free list is a seeded permutation of the pool
  blocks no sequence uses.
* In-cache layout ("tree padding"): each sequence's tree rows are written
  into its cache positions P .. P+T-1; blocks the region needs beyond the
  prefix's come from the free list in batch order.  The tree K/V arrays keep
  the same rows.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def make_tokens(parents: np.ndarray, tree_offsets: np.ndarray, rng: np.random.Generator,
                p_match: float = 0.7, vocab: int = 32000) -> Tuple[np.ndarray, np.ndarray]:
    """(draft_tokens int32 [N], target_argmax int32 [N]) for packed trees."""
    N = int(tree_offsets[-1])
    argmax = rng.integers(0, vocab, size=N).astype(np.int64)
    draft = np.zeros(N, dtype=np.int64)
    B = len(tree_offsets) - 1
    for b in range(B):
        lo, hi = int(tree_offsets[b]), int(tree_offsets[b + 1])
        par = parents[lo:hi]
        T = hi - lo
        match = rng.random(T) < p_match       # per parent: does its rank-0 child match?
        roots = rng.integers(0, vocab, size=T)
        rank = np.zeros(T, dtype=np.int64)
        seen = {}
        for i in range(T):
            p = int(par[i])
            if p < 0:
                draft[lo + i] = roots[i]
                continue
            rank[i] = seen.get(p, 0)
            seen[p] = rank[i] + 1
            base = int(argmax[lo + p])
            if rank[i] == 0 and match[p]:
                draft[lo + i] = base
            else:
                draft[lo + i] = (base + rank[i] + (0 if match[p] else 1)) % vocab
    return draft.astype(np.int32), argmax.astype(np.int32)


def free_list(inp, rng: np.random.Generator) -> np.ndarray:
    """int32 ids of the pool blocks no sequence's table row uses, seeded order."""
    used = np.zeros(inp.num_blocks, dtype=bool)
    t = inp.block_table
    used[t[t >= 0]] = True
    free = np.nonzero(~used)[0]
    return rng.permutation(free).astype(np.int32)


def place_tree_in_cache(inp, rng: np.random.Generator):
    """A copy of ``inp`` whose tree K/V rows also sit in the paged cache right
    after each prefix (positions P .. P+T-1), with the table rows extended as
    needed; returns (new inputs, free blocks left)."""
    import copy
    out = copy.copy(inp)
    out.k_cache = inp.k_cache.copy()
    out.v_cache = inp.v_cache.copy()
    out.block_table = inp.block_table.copy()
    free = list(free_list(inp, rng))
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        P = int(inp.prefix_lens[b])
        have = -(-P // 64)
        after = -(-(P + hi - lo) // 64)
        if after > out.block_table.shape[1]:
            raise ValueError(f"sequence {b}: table row too short for the tree region")
        for k in range(have, after):
            if out.block_table[b, k] < 0:     # a region block the row does not hold yet
                out.block_table[b, k] = free.pop(0)
        for i in range(hi - lo):
            pos = P + i
            blk = out.block_table[b, pos // 64]
            out.k_cache[blk, :, pos % 64, :] = inp.k_tree[lo + i]
            out.v_cache[blk, :, pos % 64, :] = inp.v_tree[lo + i]
    return out, np.asarray(free, dtype=np.int32)

