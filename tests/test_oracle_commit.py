"""Pins for the acceptance / commit oracle (CPU only).

Each check compares the oracle with something other than itself: a
hand-derived fixture, a closed form for chains, a brute-force search over all
root paths, and the attention oracle (itself pinned elsewhere) evaluated on
the committed cache.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from workloads import TREE_12, TREE_CHAIN4, free_list, make_inputs, make_tokens

HERE = os.path.dirname(os.path.abspath(__file__))


def _read_accept_fixture():
    cases, cur = [], {}
    with open(os.path.join(HERE, "golden", "accept_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            cur[key] = [int(v) for v in vals]
            if key == "bonus":
                cases.append(cur)
                cur = {}
    return cases


def test_accept_hand_fixture():
    cases = _read_accept_fixture()
    assert len(cases) == 2
    for c in cases:
        par = np.array(c["parents"], dtype=np.int32)
        off = np.array([0, len(par)], dtype=np.int32)
        n, path, bonus = oracle.accept_greedy(par, off, np.array(c["draft"]), np.array(c["argmax"]), 12)
        assert n[0] == len(c["path"])
        assert list(path[0, :n[0]]) == c["path"]
        assert np.all(path[0, n[0]:] == -1)
        assert bonus[0] == c["bonus"][0]


def test_accept_chain_closed_form():
    # on a chain the accepted length is 1 + the number of leading matches
    rng = np.random.default_rng(7)
    for T in (1, 2, 4, 9, 64):
        par = np.arange(-1, T - 1, dtype=np.int32)
        for _ in range(20):
            argmax = rng.integers(0, 3, size=T)
            draft = rng.integers(0, 3, size=T)
            match = draft[1:] == argmax[:-1]
            lead = int(np.argmin(np.append(match, False)))
            n, path, bonus = oracle.accept_greedy(par, np.array([0, T]), draft, argmax, 64)
            assert n[0] == 1 + lead
            assert list(path[0, :n[0]]) == list(range(1 + lead))
            assert bonus[0] == argmax[lead]


def _brute_force(par, draft, argmax):
    """Every root path; keep those whose every step matches; longest wins,
    then the smaller last node."""
    T = len(par)
    best = None
    for last in range(T):
        chain = []
        j = last
        while j != -1:
            chain.append(j)
            j = int(par[j])
        chain.reverse()
        if all(draft[chain[k]] == argmax[chain[k - 1]] for k in range(1, len(chain))):
            key = (-len(chain), last)
            if best is None or key < best[0]:
                best = (key, chain)
    return best[1]


def test_accept_brute_force_random_trees():
    rng = np.random.default_rng(11)
    for _ in range(300):
        T = int(rng.integers(1, 11))
        par = [-1] + [int(rng.integers(-1, i)) for i in range(1, T)]   # forests too
        draft = rng.integers(0, 2, size=T)
        argmax = rng.integers(0, 2, size=T)
        n, path, bonus = oracle.accept_greedy(np.array(par), np.array([0, T]), draft, argmax, 10)
        want = _brute_force(par, draft, argmax)
        assert list(path[0, :n[0]]) == want
        assert bonus[0] == argmax[want[-1]]


def test_accept_brute_force_large_trees():
    # trees of 65..256 nodes (forests too) with matching rates high enough for
    # long accepted paths, against the brute force over every root path
    from helpers import random_tree
    rng = np.random.default_rng(12)
    for k in range(12):
        T = int(rng.integers(65, 257))
        par = random_tree(rng, T, forest_p=0.05 if k % 3 == 0 else 0.0)
        draft = rng.integers(0, 2, size=T)
        argmax = rng.integers(0, 2, size=T)
        if k % 2:   # mostly matching steps: paths run deep
            par_arr = np.array(par)
            draft = np.where(rng.random(T) < 0.9, argmax[np.maximum(par_arr, 0)], draft)
        n, path, bonus = oracle.accept_greedy(np.array(par), np.array([0, T]), draft, argmax, 256)
        want = _brute_force(par, draft, argmax)
        assert list(path[0, :n[0]]) == want
        assert np.all(path[0, n[0]:] == -1)
        assert bonus[0] == argmax[want[-1]]


def test_accept_chain_closed_form_256():
    rng = np.random.default_rng(13)
    T = 256
    par = np.arange(-1, T - 1, dtype=np.int32)
    for lead in (0, 63, 64, 200, 255):
        argmax = rng.integers(0, 5, size=T)
        draft = np.empty(T, dtype=np.int64)
        draft[0] = 0
        draft[1:] = argmax[:-1]                       # every step matches ...
        if lead + 1 < T:
            draft[lead + 1] = argmax[lead] + 1        # ... until step lead + 1
        n, path, bonus = oracle.accept_greedy(par, np.array([0, T]), draft, argmax, T)
        assert n[0] == 1 + lead
        assert list(path[0, :n[0]]) == list(range(1 + lead))
        assert bonus[0] == argmax[lead]


def test_accept_packed_batch_matches_per_sequence():
    rng = np.random.default_rng(3)
    trees = [TREE_12, [-1], TREE_CHAIN4, TREE_12]
    par = np.concatenate([np.array(t, dtype=np.int32) for t in trees])
    off = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    draft, argmax = make_tokens(par, off, rng, p_match=0.8, vocab=50)
    n, path, bonus = oracle.accept_greedy(par, off, draft, argmax, 12)
    for b, t in enumerate(trees):
        lo, hi = off[b], off[b + 1]
        n1, p1, b1 = oracle.accept_greedy(np.array(t), np.array([0, len(t)]), draft[lo:hi], argmax[lo:hi], 12)
        assert n[b] == n1[0] and list(path[b]) == list(p1[0]) and bonus[b] == b1[0]


def test_accept_rejects_bad_parent():
    with pytest.raises(ValueError):
        oracle.accept_greedy(np.array([-1, 2, 0]), np.array([0, 3]), np.zeros(3), np.zeros(3), 3)


# ------------------------------------------------------------------- commit
def _commit_case(seed, prefix_lens, trees, spare=6, extra_cols=2, p_match=0.9):
    rng = np.random.default_rng(seed)
    inp = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                      prefix_lens=prefix_lens, trees=trees, rng=rng, spare_blocks=spare,
                      extra_table_cols=extra_cols)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=40)
    n, path, bonus = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax,
                                          inp.max_tree_nodes)
    free = free_list(inp, rng)
    return inp, n, path, free


def _gather(cache, table_row, length):
    out = []
    for t in range(length):
        out.append(cache[table_row[t // 64], :, t % 64, :])
    return np.stack(out) if out else np.zeros((0,) + cache.shape[1:2] + cache.shape[3:], cache.dtype)


def test_commit_appends_path_and_leaves_the_rest():
    inp, n, path, free = _commit_case(21, [63, 64, 130, 0], [TREE_12, TREE_CHAIN4, TREE_12, TREE_CHAIN4])
    r = oracle.commit(inp, n, path, free, len(free))
    assert r["error"] == 0
    written = set()
    for b in range(inp.batch):
        P, A = int(inp.prefix_lens[b]), int(n[b])
        assert r["prefix_lens"][b] == P + A
        lo = int(inp.tree_offsets[b])
        kc = _gather(r["k_cache"], r["block_table"][b], P + A)
        vc = _gather(r["v_cache"], r["block_table"][b], P + A)
        assert np.array_equal(kc[:P], _gather(inp.k_cache, inp.block_table[b], P))
        assert np.array_equal(kc[P:], inp.k_tree[lo + path[b, :A]])
        assert np.array_equal(vc[P:], inp.v_tree[lo + path[b, :A]])
        for t in range(P, P + A):
            written.add((int(r["block_table"][b][t // 64]), t % 64))
    # every other slot of the pool keeps its bits (NaN poison included)
    mask = np.ones(inp.k_cache.shape[0:1] + inp.k_cache.shape[2:3], dtype=bool)
    for blk, slot in written:
        mask[blk, slot] = False
    a = inp.k_cache.transpose(0, 2, 1, 3)[mask]
    bb = r["k_cache"].transpose(0, 2, 1, 3)[mask]
    assert np.array_equal(a.view(np.uint16), bb.view(np.uint16))


def test_commit_takes_free_blocks_in_order():
    inp, n, path, free = _commit_case(22, [63, 64, 128, 10], [TREE_CHAIN4] * 4, p_match=1.0)
    assert list(n) == [4, 4, 4, 4]
    r = oracle.commit(inp, n, path, free, len(free))
    # new blocks: seq 0 (63 -> 67) 1, seq 1 (64 -> 68) 1, seq 2 (128 -> 132) 1, seq 3 none
    assert r["blocks_taken"] == 3
    assert r["block_table"][0][1] == free[0]
    assert r["block_table"][1][1] == free[1]
    assert r["block_table"][2][2] == free[2]
    r2 = oracle.commit(inp, n, path, free, 2)          # one block short
    assert r2["error"] == "no_blocks" and r2["blocks_taken"] == 0
    assert np.array_equal(r2["block_table"], inp.block_table)
    assert np.array_equal(r2["prefix_lens"], inp.prefix_lens)


def test_commit_bad_path_skips_that_sequence_only():
    inp, n, path, free = _commit_case(23, [10, 20], [TREE_12, TREE_12], p_match=1.0)
    bad = path.copy()
    bad[0, 1] = 3 if bad[0, 1] != 3 else 1      # still a child of 0 ...
    bad[0, 2] = 5 if bad[0, 2] not in (5,) else 4   # ... but no longer a child of bad[0, 1]
    r = oracle.commit(inp, n, bad, free, len(free))
    assert r["error"] == "bad_tree"
    assert r["prefix_lens"][0] == inp.prefix_lens[0]
    assert r["prefix_lens"][1] == inp.prefix_lens[1] + n[1]


def test_commit_then_prefix_attention_equals_verify_of_last_node():
    # the committed history seen by the last accepted node is exactly what it
    # saw during verification: prefix + its ancestors-or-self
    inp, n, path, free = _commit_case(24, [70, 5, 200], [TREE_12, TREE_CHAIN4, TREE_12], p_match=0.8)
    o_ver, lse_ver, _ = oracle.verify(inp)
    r = oracle.commit(inp, n, path, free, len(free))
    assert r["error"] == 0
    for b in range(inp.batch):
        lo = int(inp.tree_offsets[b])
        last = lo + int(path[b, n[b] - 1])
        one = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                          prefix_lens=[0], trees=[[-1]], rng=np.random.default_rng(0))
        one.k_cache, one.v_cache = r["k_cache"], r["v_cache"]
        one.block_table = r["block_table"][b:b + 1]
        one.prefix_lens = r["prefix_lens"][b:b + 1].copy()
        one.q = inp.q[last:last + 1]
        o_pre, lse_pre = oracle.prefix_only(one)
        assert np.allclose(o_pre[0], o_ver[last], atol=1e-12, rtol=0)
        assert np.allclose(lse_pre[0], lse_ver[last], atol=1e-12, rtol=0)


def test_commit_nothing_when_table_row_full():
    inp, n, path, free = _commit_case(25, [127, 3], [TREE_CHAIN4, TREE_CHAIN4], extra_cols=0, p_match=1.0)
    # sequence 0 holds 2 blocks, its row has 2 columns: 127 + 4 tokens need 3
    assert inp.block_table.shape[1] == 2
    r = oracle.commit(inp, n, path, free, len(free))
    assert r["error"] == "no_blocks"
    assert np.array_equal(r["prefix_lens"], inp.prefix_lens)


# ------------------------------------------------------- in-cache tree rows
def test_incache_verify_equals_separate_tree_rows():
    from workloads import place_tree_in_cache
    rng = np.random.default_rng(31)
    inp = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                      prefix_lens=[63, 0, 130], trees=[TREE_12, TREE_CHAIN4, TREE_12], rng=rng,
                      spare_blocks=6, extra_table_cols=1)
    ic, _ = place_tree_in_cache(inp, rng)
    # the gathered rows are the tree rows, bit for bit
    kt, vt = oracle.tree_rows_from_cache(ic)
    assert np.array_equal(kt.view(np.uint16), inp.k_tree.view(np.uint16))
    assert np.array_equal(vt.view(np.uint16), inp.v_tree.view(np.uint16))
    # so the verify outputs agree exactly; the prefix piece still ends at P
    o1, l1, _ = oracle.verify(inp)
    ic.k_tree = np.zeros_like(inp.k_tree)          # must not be read
    o2, l2, _ = oracle.verify_incache(ic)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_incache_commit_matches_separate_commit_and_attention():
    from workloads import place_tree_in_cache
    rng = np.random.default_rng(32)
    inp = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                      prefix_lens=[63, 5, 190], trees=[TREE_12, TREE_CHAIN4, TREE_12], rng=rng,
                      spare_blocks=8, extra_table_cols=1)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.8, vocab=30)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    ic, _ = place_tree_in_cache(inp, rng)
    o_ver, l_ver, _ = oracle.verify_incache(ic)
    r = oracle.commit_incache(ic, n, path)
    assert r["error"] == 0
    for b in range(inp.batch):
        P, A = int(inp.prefix_lens[b]), int(n[b])
        assert r["prefix_lens"][b] == P + A
        lo = int(inp.tree_offsets[b])
        got = _gather(r["k_cache"], ic.block_table[b], P + A)
        # the committed history: the old prefix, then the accepted rows in path order
        assert np.array_equal(got[:P], _gather(inp.k_cache, inp.block_table[b], P))
        assert np.array_equal(got[P:], inp.k_tree[lo + path[b, :A]])
        # and the last accepted node sees exactly that history
        last = lo + int(path[b, n[b] - 1])
        one = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                          prefix_lens=[0], trees=[[-1]], rng=np.random.default_rng(0))
        one.k_cache, one.v_cache = r["k_cache"], r["v_cache"]
        one.block_table = ic.block_table[b:b + 1]
        one.prefix_lens = r["prefix_lens"][b:b + 1].copy()
        one.q = inp.q[last:last + 1]
        o_pre, l_pre = oracle.prefix_only(one)
        assert np.allclose(o_pre[0], o_ver[last], atol=1e-12, rtol=0)
        assert np.allclose(l_pre[0], l_ver[last], atol=1e-12, rtol=0)


def test_incache_commit_bad_path_skips_sequence():
    from workloads import place_tree_in_cache
    rng = np.random.default_rng(33)
    inp = make_inputs(dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=64,
                      prefix_lens=[10, 70], trees=[TREE_12, TREE_12], rng=rng,
                      spare_blocks=4, extra_table_cols=1)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=1.0, vocab=30)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    ic, _ = place_tree_in_cache(inp, rng)
    bad = path.copy()
    bad[1, 1] = 2 if bad[1, 1] != 2 else 3
    bad[1, 2] = 4 if bad[1, 1] != 1 else 5   # 4 and 5 are children of 1 only
    r = oracle.commit_incache(ic, n, bad)
    assert r["error"] == "bad_tree"
    assert r["prefix_lens"][1] == inp.prefix_lens[1]
    assert r["prefix_lens"][0] == inp.prefix_lens[0] + n[0]
