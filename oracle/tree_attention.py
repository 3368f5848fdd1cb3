"""fp64 oracle: unsplit masked softmax attention over prefix + draft tree.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources (the pages this method is described on; no formula is printed there,
so the textbook forms are written out here):

* Split tree attention: the draft tree is flattened into one token sequence;
  attention is computed as a query-to-prefix piece that needs no custom mask
  and a piece among the draft tokens that needs the tree mask; the pieces are
  combined with ``merge_attentions``.  [pith.science review of arXiv
  2508.08192, "What carries the argument"; same text in the pith.science
  verdict record, pith_extraction.key_machinery]
* ``merge_attentions`` combines attention computed over disjoint KV chunks and
  is what makes the two-pass form correct (Hydragen, Juravsky et al. 2024).
  [pith.science verdict record, pith_extraction.supporting_citations]
* Paged KV cache (PagedAttention, Kwon et al. 2023) is the memory scheme
  adapted for tree attention.  [same field; mlsanity.com index, "Builds on"]

Readings taken where the pages are silent:

* Tree mask = ancestor-or-self: node i sees tree node j iff j lies on the path
  from i to its root, i included (the SpecInfer tree-verification semantics,
  listed under "Builds on" on the mlsanity.com index).
* Every tree node sees every committed prefix token ("no custom mask").
* GQA: query head h reads KV head h // G with G = H_q / H_kv.
* Softmax: s = scale * q.k; lse in natural log; no positional encoding applied.
* A row with no visible key has o = 0 and lse = -inf.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


# ----------------------------------------------------------------- dtype upcast
def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to fp64.

    bf16 is the upper half of an IEEE fp32 word, so widening the 16-bit
    pattern into the high half of a 32-bit word gives the same real number.
    """
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------------- tree mask
def visibility(parents) -> np.ndarray:
    """Boolean [T, T]: vis[i, j] is True iff j is i or an ancestor of i.

    Built by walking parent links from each node up to its root (a different
    procedure from the GPU's, which combines parent masks).  Raises
    ``ValueError`` for a parent that is not -1 or an earlier node.
    [pith.science review, "What carries the argument": the draft-token piece
    "needs the tree mask"; ancestor-or-self reading as in SpecInfer]
    """
    par = [int(p) for p in parents]
    T = len(par)
    for i, p in enumerate(par):
        if not (p == -1 or 0 <= p < i):
            raise ValueError(f"node {i}: parent {p} is neither -1 nor an earlier node")
    vis = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j != -1:
            vis[i, j] = True
            j = par[j]
    return vis


def ancestor_or_self_mask(parents) -> np.ndarray:
    """uint64 [T]: bit j of word i is set iff j is i or an ancestor of i (T <= 64)."""
    vis = visibility(parents)
    T = vis.shape[0]
    if T > 64:
        raise ValueError(f"tree of {T} nodes does not fit one 64-bit mask word")
    out = np.zeros(T, dtype=np.uint64)
    for i in range(T):
        word = 0
        for j in range(T):
            if vis[i, j]:
                word |= 1 << j
        out[i] = np.uint64(word)
    return out


def ancestor_or_self_words(parents, words: int) -> np.ndarray:
    """uint64 [T, words]: bit j % 64 of word j // 64 in row i is set iff j is i
    or an ancestor of i -- the same mask for trees of more than 64 nodes,
    spread over several 64-bit words (T <= 64 * words)."""
    vis = visibility(parents)
    T = vis.shape[0]
    if T > 64 * words:
        raise ValueError(f"tree of {T} nodes does not fit {words} mask words")
    out = np.zeros((T, words), dtype=np.uint64)
    for i in range(T):
        for j in range(T):
            if vis[i, j]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def build_masks_words(inp, words: int) -> np.ndarray:
    """Multi-word masks of every sequence packed like the tree rows: uint64 [N, words]."""
    out = np.zeros((inp.total_tree_nodes, words), dtype=np.uint64)
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        out[lo:hi] = ancestor_or_self_words(inp.parents[lo:hi], words)
    return out


def build_masks(inp) -> np.ndarray:
    """Masks of every sequence packed like the tree rows: uint64 [N]."""
    out = np.zeros(inp.total_tree_nodes, dtype=np.uint64)
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        out[lo:hi] = ancestor_or_self_mask(inp.parents[lo:hi])
    return out


# ---------------------------------------------------------- attention pieces
def _attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
            visible: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of ``qrows`` [R, D] over keys K [L, D] / values V [L, D].

    ``visible`` [R, L] selects the keys each row may attend to.  Returns
    o [R, D] and lse [R] (natural log), both fp64.
    """
    R, D = qrows.shape
    o = np.zeros((R, V.shape[1] if V.ndim == 2 else D), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if K.shape[0] == 0 or R == 0:
        return o, lse
    s = scale * (qrows @ K.T)                 # [R, L]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)                         # [R]
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    p = np.exp(s - m_safe[:, None])           # exp(-inf) = 0 for hidden keys
    l = p.sum(axis=1)
    o[has] = (p[has] @ V) / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def _prefix_kv(inp, b: int, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """Committed prefix keys/values of sequence b, KV head g, read through the
    block table: token t is slot t % 64 of pool block block_table[b][t // 64]."""
    P = int(inp.prefix_lens[b])
    bs = inp.block_size
    D = inp.head_dim
    K = np.empty((P, D), dtype=np.float64)
    V = np.empty((P, D), dtype=np.float64)
    for t in range(0, P, bs):
        blk = int(inp.block_table[b, t // bs])
        n = min(bs, P - t)
        K[t:t + n] = to_f64(inp.k_cache[blk, g, :n, :], inp.dtype)
        V[t:t + n] = to_f64(inp.v_cache[blk, g, :n, :], inp.dtype)
    return K, V


def _rows_of(inp, b: int, g: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Query rows of (sequence b, KV head g): node-major, grouped head minor.

    Returns (q [T*G, D] fp64, node index of each row, query head of each row).
    """
    G = inp.num_q_heads // inp.num_kv_heads
    lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
    heads = np.arange(g * G, (g + 1) * G)
    q = to_f64(inp.q[lo:hi][:, heads, :], inp.dtype).reshape(-1, inp.head_dim)
    nodes = np.repeat(np.arange(hi - lo), G)
    return q, nodes, np.tile(heads, hi - lo)


def _check_shape(inp) -> None:
    if inp.num_q_heads % inp.num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")


def verify(inp) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Unsplit tree-verify attention.

    For every sequence b, tree node i and query head h: softmax attention of
    q[i, h] over the P_b prefix keys of KV head h // G followed by the tree keys
    of the nodes on i's root path.  Returns (o [N, Hq, D], lse [N, Hq], masks
    [N] uint64 -- [N, W] words when some tree has more than 64 nodes), all
    computed in fp64 without splitting.
    [pith.science review, "What carries the argument"]
    """
    _check_shape(inp)
    N, Hq, D = inp.total_tree_nodes, inp.num_q_heads, inp.head_dim
    o = np.zeros((N, Hq, D), dtype=np.float64)
    lse = np.full((N, Hq), -np.inf, dtype=np.float64)
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        if hi == lo:
            continue
        vis_tree = visibility(inp.parents[lo:hi])
        P = int(inp.prefix_lens[b])
        for g in range(inp.num_kv_heads):
            Kp, Vp = _prefix_kv(inp, b, g)
            Kt = to_f64(inp.k_tree[lo:hi, g, :], inp.dtype)
            Vt = to_f64(inp.v_tree[lo:hi, g, :], inp.dtype)
            K = np.concatenate([Kp, Kt], axis=0)
            V = np.concatenate([Vp, Vt], axis=0)
            q, nodes, heads = _rows_of(inp, b, g)
            visible = np.concatenate(
                [np.ones((len(nodes), P), dtype=bool), vis_tree[nodes]], axis=1)
            ob, lb = _attend(q, K, V, inp.softmax_scale, visible)
            o[lo + nodes, heads] = ob
            lse[lo + nodes, heads] = lb
    T_max = int(np.diff(inp.tree_offsets).max()) if inp.batch else 0
    if T_max <= 64:
        return o, lse, build_masks(inp)
    return o, lse, build_masks_words(inp, -(-T_max // 64))


def tree_rows_from_cache(inp) -> Tuple[np.ndarray, np.ndarray]:
    """The tree K/V rows of an in-cache batch: node i of sequence b is cache
    position prefix_lens[b] + i, read through the block table (slot
    (P + i) % 64 of block block_table[b][(P + i) // 64]).  Returns
    (k_tree, v_tree) [N, Hkv, D] in the storage dtype (a plain gather).
    [pith.science verdict record: paged KV with tree padding, and
    paged/persistent KV-cache handling for tree attention]"""
    N = inp.total_tree_nodes
    kt = np.empty((N,) + inp.k_cache.shape[1:2] + inp.k_cache.shape[3:], dtype=inp.k_cache.dtype)
    vt = np.empty_like(kt)
    bs = inp.block_size
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        P = int(inp.prefix_lens[b])
        for i in range(hi - lo):
            pos = P + i
            blk = int(inp.block_table[b, pos // bs])
            kt[lo + i] = inp.k_cache[blk, :, pos % bs, :]
            vt[lo + i] = inp.v_cache[blk, :, pos % bs, :]
    return kt, vt


def verify_incache(inp) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """:func:`verify` for a batch whose tree K/V rows sit in the paged cache
    right after each prefix (``inp.k_tree`` / ``inp.v_tree`` are ignored):
    the rows are gathered (:func:`tree_rows_from_cache`) and the definition
    is the same.  The prefix piece still covers positions [0, P) only."""
    import copy
    kt, vt = tree_rows_from_cache(inp)
    view = copy.copy(inp)
    view.k_tree, view.v_tree = kt, vt
    return verify(view)


def verify_rows(inp, rows) -> Tuple[np.ndarray, np.ndarray]:
    """Same definition as :func:`verify`, evaluated only for the listed
    (node row n, query head h) pairs.  Returns (o [k, D], lse [k])."""
    _check_shape(inp)
    G = inp.num_q_heads // inp.num_kv_heads
    seq_of = np.searchsorted(inp.tree_offsets, np.arange(inp.total_tree_nodes),
                             side="right") - 1
    out_o = np.zeros((len(rows), inp.head_dim), dtype=np.float64)
    out_l = np.zeros(len(rows), dtype=np.float64)
    for k, (n, h) in enumerate(rows):
        b = int(seq_of[n])
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        g = h // G
        vis = visibility(inp.parents[lo:hi])[n - lo]
        Kp, Vp = _prefix_kv(inp, b, g)
        Kt = to_f64(inp.k_tree[lo:hi, g, :], inp.dtype)
        Vt = to_f64(inp.v_tree[lo:hi, g, :], inp.dtype)
        K = np.concatenate([Kp, Kt], axis=0)
        V = np.concatenate([Vp, Vt], axis=0)
        visible = np.concatenate([np.ones(Kp.shape[0], dtype=bool), vis])[None, :]
        q = to_f64(inp.q[n, h, :], inp.dtype)[None, :]
        ob, lb = _attend(q, K, V, inp.softmax_scale, visible)
        out_o[k], out_l[k] = ob[0], lb[0]
    return out_o, out_l


def prefix_only(inp) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every tree query over the committed prefix alone, no mask
    (the "large, but no custom mask needed" piece).  (o [N,Hq,D], lse [N,Hq]).
    A sequence with an empty prefix gives o = 0, lse = -inf.
    [pith.science review, "What carries the argument"]"""
    _check_shape(inp)
    N, Hq, D = inp.total_tree_nodes, inp.num_q_heads, inp.head_dim
    o = np.zeros((N, Hq, D), dtype=np.float64)
    lse = np.full((N, Hq), -np.inf, dtype=np.float64)
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        if hi == lo:
            continue
        for g in range(inp.num_kv_heads):
            Kp, Vp = _prefix_kv(inp, b, g)
            q, nodes, heads = _rows_of(inp, b, g)
            visible = np.ones((len(nodes), Kp.shape[0]), dtype=bool)
            ob, lb = _attend(q, Kp, Vp, inp.softmax_scale, visible)
            o[lo + nodes, heads] = ob
            lse[lo + nodes, heads] = lb
    return o, lse


def suffix_only(inp) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every tree query over the tree keys on its root path only
    (the "small, but needs the tree mask" piece).  (o [N,Hq,D], lse [N,Hq]).
    [pith.science review, "What carries the argument"]"""
    _check_shape(inp)
    N, Hq, D = inp.total_tree_nodes, inp.num_q_heads, inp.head_dim
    o = np.zeros((N, Hq, D), dtype=np.float64)
    lse = np.full((N, Hq), -np.inf, dtype=np.float64)
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        if hi == lo:
            continue
        vis_tree = visibility(inp.parents[lo:hi])
        for g in range(inp.num_kv_heads):
            Kt = to_f64(inp.k_tree[lo:hi, g, :], inp.dtype)
            Vt = to_f64(inp.v_tree[lo:hi, g, :], inp.dtype)
            q, nodes, heads = _rows_of(inp, b, g)
            ob, lb = _attend(q, Kt, Vt, inp.softmax_scale, vis_tree[nodes])
            o[lo + nodes, heads] = ob
            lse[lo + nodes, heads] = lb
    return o, lse


def merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray,
          lse_b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Combine two attention results computed over disjoint key sets.

    Each piece's softmax denominator is exp(lse); the combined denominator is
    their sum, so lse = log(exp(lse_a) + exp(lse_b)) and the combined output is
    the denominator-weighted average of the two outputs.  Both -inf gives
    o = 0, lse = -inf.  [merge_attentions: pith.science verdict record,
    pith_extraction.supporting_citations (Juravsky et al. 2024)]
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    both_empty = ~np.isfinite(m)
    m_safe = np.where(both_empty, 0.0, m)
    wa = np.exp(lse_a - m_safe)   # exp(-inf) = 0 for an empty piece
    wb = np.exp(lse_b - m_safe)
    tot = wa + wb
    tot_safe = np.where(both_empty, 1.0, tot)
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / tot_safe[..., None]
    o = np.where(both_empty[..., None], 0.0, o)
    lse = np.where(both_empty, -np.inf, m_safe + np.log(tot_safe))
    return o, lse
