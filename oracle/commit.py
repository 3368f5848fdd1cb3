"""Oracle for the step after verification: greedy acceptance of a tree path
and committing that path's K/V into the paged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources:

* After verification the service commits an accepted path, and the target
  cache must then reflect exactly the committed history: a rejected branch
  leaves nothing behind.  [fdeinterviews.com summary, opening paragraph and
  the paragraph on hidden correctness obligations]
* Drafting is greedy and the KV cache / hidden-state bookkeeping is rewound
  to the accepted tokens.  [pith.science verdict record, referee summary and
  minor comment on Section 3.3]

Readings taken where the pages are silent (the acceptance rule is not printed):

* Greedy acceptance: a root (parent -1) is always accepted; a node is
  accepted iff its parent is accepted and its draft token equals the target's
  greedy token at the parent.  The committed path ends at the deepest
  accepted node, the smallest index among equally deep ones; it runs root
  first.  The bonus token is the target's greedy token at that last node.
* Commit: the path's tree K/V rows are appended after the sequence's prefix,
  one token per path node in path order; the prefix length grows by the path
  length.  Blocks the new tokens need beyond the sequence's current ones come
  from the front of a free list, sequences in batch order.  A sequence whose
  path is not a root path of its tree is not committed (bad tree); when the
  free list or a block-table row is too small nothing is committed.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

BLOCK = 64


def _depths(par) -> np.ndarray:
    """Depth of every node by walking parent links (root depth 0)."""
    T = len(par)
    d = np.zeros(T, dtype=np.int64)
    for i in range(T):
        j, n = i, 0
        while par[j] != -1:
            j = int(par[j])
            n += 1
        d[i] = n
    return d


def accept_greedy(parents, tree_offsets, draft_tokens, target_argmax,
                  max_tree_nodes: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy acceptance for every sequence of a packed batch.

    Returns (accept_len int32 [B], path int32 [B, max_tree_nodes] with -1
    after the path, bonus int32 [B]).  Node indices are local to the
    sequence.  Raises ``ValueError`` on a parent that is neither -1 nor an
    earlier node.
    """
    B = len(tree_offsets) - 1
    acc_len = np.zeros(B, dtype=np.int32)
    path = np.full((B, max_tree_nodes), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(tree_offsets[b]), int(tree_offsets[b + 1])
        par = [int(p) for p in parents[lo:hi]]
        T = hi - lo
        for i, p in enumerate(par):
            if not (p == -1 or 0 <= p < i):
                raise ValueError(f"sequence {b} node {i}: bad parent {p}")
        accepted = [False] * T
        for i in range(T):          # parents come first, so one pass in order
            p = par[i]
            if p == -1:
                accepted[i] = True
            else:
                accepted[i] = accepted[p] and int(draft_tokens[lo + i]) == int(target_argmax[lo + p])
        depth = _depths(par)
        best = -1
        for i in range(T):
            if accepted[i] and (best < 0 or depth[i] > depth[best]):
                best = i
        chain = []
        j = best
        while j != -1:
            chain.append(j)
            j = par[j]
        chain.reverse()
        acc_len[b] = len(chain)
        path[b, :len(chain)] = chain
        bonus[b] = int(target_argmax[lo + best])
    return acc_len, path, bonus


def commit(inp, accept_len, path, free_blocks, free_count: int) -> Dict[str, object]:
    """Commit every sequence's accepted path into a copy of the paged cache.

    Returns a dict with the new ``k_cache``, ``v_cache``, ``block_table``,
    ``prefix_lens``, ``blocks_taken`` and ``error`` (0, ``"bad_tree"`` when
    some path was not a root path or ``"bad_prefix"`` when some prefix length
    was outside [0, 64 * table columns] -- those sequences are skipped -- or
    ``"no_blocks"`` when nothing was committed for lack of blocks).
    """
    B = inp.batch
    k_cache = inp.k_cache.copy()
    v_cache = inp.v_cache.copy()
    table = inp.block_table.copy()
    plen = inp.prefix_lens.copy()
    maxb = table.shape[1]
    ok = np.zeros(B, dtype=bool)
    need = np.zeros(B, dtype=np.int64)
    error = 0
    for b in range(B):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        par = inp.parents[lo:hi]
        A = int(accept_len[b])
        good = 0 <= A <= hi - lo
        for t in range(A if good else 0):
            node = int(path[b, t])
            want_parent = -1 if t == 0 else int(path[b, t - 1])
            if not (0 <= node < hi - lo and int(par[node]) == want_parent):
                good = False
                break
        if not good:
            error = error or "bad_tree"
            continue
        P = int(plen[b])
        if not 0 <= P <= BLOCK * maxb:
            error = error or "bad_prefix"
            continue
        have = -(-P // BLOCK)
        after = -(-(P + A) // BLOCK)
        if after > maxb:
            return dict(k_cache=inp.k_cache.copy(), v_cache=inp.v_cache.copy(),
                        block_table=inp.block_table.copy(), prefix_lens=inp.prefix_lens.copy(),
                        blocks_taken=0, error="no_blocks")
        ok[b] = True
        need[b] = after - have
    if int(need.sum()) > int(free_count):
        return dict(k_cache=inp.k_cache.copy(), v_cache=inp.v_cache.copy(),
                    block_table=inp.block_table.copy(), prefix_lens=inp.prefix_lens.copy(),
                    blocks_taken=0, error="no_blocks")
    nxt = 0
    for b in range(B):
        if not ok[b]:
            continue
        lo = int(inp.tree_offsets[b])
        P = int(plen[b])
        have = -(-P // BLOCK)
        for k in range(int(need[b])):
            table[b, have + k] = int(free_blocks[nxt])
            nxt += 1
        for t in range(int(accept_len[b])):
            pos = P + t
            blk = int(table[b, pos // BLOCK])
            row = lo + int(path[b, t])
            k_cache[blk, :, pos % BLOCK, :] = inp.k_tree[row]
            v_cache[blk, :, pos % BLOCK, :] = inp.v_tree[row]
        plen[b] = P + int(accept_len[b])
    return dict(k_cache=k_cache, v_cache=v_cache, block_table=table, prefix_lens=plen,
                blocks_taken=nxt, error=error)


def commit_incache(inp, accept_len, path) -> Dict[str, object]:
    """Commit for the in-cache layout: the tree's rows already sit at cache
    positions P .. P+T-1 of each sequence, so the accepted path is compacted
    in place -- position P + t takes the row that was at P + path[t] before
    the commit -- and the prefix length grows by the path length.  Rows past
    the new prefix are left as they are (no longer part of the history).  A
    path that is not a root path skips its sequence (``"bad_tree"``); so does
    a tree region that runs past the sequence's table row (``"bad_prefix"``).
    [pith.science verdict record: paged KV with tree padding; fdeinterviews.com
    summary: the cache must hold exactly the committed history]
    """
    B = inp.batch
    k_cache = inp.k_cache.copy()
    v_cache = inp.v_cache.copy()
    plen = inp.prefix_lens.copy()
    maxb = inp.block_table.shape[1]
    error = 0
    for b in range(B):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        par = inp.parents[lo:hi]
        T = hi - lo
        A = int(accept_len[b])
        good = 0 <= A <= T
        for t in range(A if good else 0):
            node = int(path[b, t])
            want_parent = -1 if t == 0 else int(path[b, t - 1])
            if not (0 <= node < T and int(par[node]) == want_parent):
                good = False
                break
        if not good:
            error = error or "bad_tree"
            continue
        P = int(plen[b])
        if not (0 <= P and P + T <= BLOCK * maxb):
            error = error or "bad_prefix"
            continue
        for t in range(A):
            src, dst = P + int(path[b, t]), P + t
            sb, db = int(inp.block_table[b, src // BLOCK]), int(inp.block_table[b, dst // BLOCK])
            k_cache[db, :, dst % BLOCK, :] = inp.k_cache[sb, :, src % BLOCK, :]
            v_cache[db, :, dst % BLOCK, :] = inp.v_cache[sb, :, src % BLOCK, :]
        plen[b] = P + A
    return dict(k_cache=k_cache, v_cache=v_cache, prefix_lens=plen, error=error)

