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
