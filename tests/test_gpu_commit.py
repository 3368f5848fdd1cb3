"""GPU parity for the step after verification: greedy acceptance and the
commit of the accepted path into the paged cache, against the oracle.

Both are integer / byte work, so the bar is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import say, to_device
from helpers import random_tree
from workloads import TREE_12, TREE_CHAIN4, TREE_SINGLE, free_list, make_inputs, make_tokens

pytestmark = pytest.mark.gpu


def _i32(x, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a device tensor (bf16 -> uint16, f32 -> uint32)."""
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else \
        a.numpy().view(np.uint32)


def _host_bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint16) if x.dtype == np.uint16 else x.view(np.uint32)


def _batch(seed, trees, prefix_lens, *, dtype="bf16", Hkv=2, D=64, spare=8, extra_cols=2,
           p_match=0.7, vocab=50):
    rng = np.random.default_rng(seed)
    inp = make_inputs(dtype=dtype, num_q_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=D,
                      prefix_lens=prefix_lens, trees=trees, rng=rng, spare_blocks=spare,
                      extra_table_cols=extra_cols)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=vocab)
    free = free_list(inp, rng)
    return inp, draft, argmax, free


def _accept_gpu(d, draft, argmax):
    import tree_attention_verify_attn_amd as ta
    n, path, bonus = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                      d.workspace)
    torch.cuda.synchronize()
    return n.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy()


def _check_accept(inp, d, draft, argmax, what):
    n, path, bonus = _accept_gpu(d, draft, argmax)
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax,
                                             d.shape.max_tree_nodes)
    np.testing.assert_array_equal(n, wn, err_msg=f"{what} accept_len")
    np.testing.assert_array_equal(path, wpath, err_msg=f"{what} path")
    np.testing.assert_array_equal(bonus, wbonus, err_msg=f"{what} bonus")


# ------------------------------------------------------------- acceptance
def test_accept_mixed_batch_bit_exact():
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(5)
    kinds = rng.choice(3, size=256, p=[0.2, 0.5, 0.3])
    trees = [(TREE_SINGLE, TREE_CHAIN4, TREE_12)[k] for k in kinds]
    inp, draft, argmax, _ = _batch(61, trees, [1] * 256, spare=0, extra_cols=0)
    d = to_device(inp)
    say("accept: 256 sequences, tree mix 1/chain-4/12")
    _check_accept(inp, d, draft, argmax, "mix")
    assert ta.get_error(d.workspace) == 0


@pytest.mark.parametrize("p_match", [0.0, 0.5, 1.0])
def test_accept_random_trees_and_forests(p_match):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(62)
    trees = [random_tree(rng, int(rng.integers(1, 65)), forest_p=0.1 if i % 3 == 0 else 0.0)
             for i in range(40)]
    trees.append(list(range(-1, 63)))             # a 64-node chain
    trees.append([-1] + [0] * 63)                 # 64-node star
    inp, draft, argmax, _ = _batch(63, trees, [1] * len(trees), spare=0, extra_cols=0,
                                   p_match=p_match, vocab=3)
    d = to_device(inp, max_tree_nodes=64)
    say(f"accept: random trees and forests up to 64 nodes, p_match {p_match}")
    _check_accept(inp, d, draft, argmax, f"random p={p_match}")
    assert ta.get_error(d.workspace) == 0


def test_accept_padded_path_width():
    # max_tree_nodes above every tree: the path rows are padded with -1
    inp, draft, argmax, _ = _batch(64, [TREE_CHAIN4, TREE_SINGLE], [1, 1], spare=0, extra_cols=0,
                                   p_match=1.0)
    d = to_device(inp, max_tree_nodes=20)
    say("accept: path width 20 for trees of 4 and 1 nodes")
    _check_accept(inp, d, draft, argmax, "padded")


def test_accept_bad_tree_flagged():
    import tree_attention_verify_attn_amd as ta
    inp, draft, argmax, _ = _batch(65, [TREE_12, TREE_CHAIN4], [1, 1], spare=0, extra_cols=0)
    d = to_device(inp)
    d.parents[3] = 7                               # a later node as parent
    say("accept: bad parent flagged")
    n, path, bonus = _accept_gpu(d, draft, argmax)
    assert ta.get_error(d.workspace) == 3
    assert n[0] == 0 and bonus[0] == -1 and (path[0] == -1).all()
    # the other sequence is unaffected
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents[12:], np.array([0, 4]), draft[12:],
                                             argmax[12:], 12)
    assert n[1] == wn[0] and (path[1] == wpath[0]).all() and bonus[1] == wbonus[0]


# ----------------------------------------------------------------- commit
def _commit_gpu(inp, d, n, path, free, free_count):
    import tree_attention_verify_attn_amd as ta
    taken = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta.commit(d.shape, d.k_tree, d.v_tree, d.parents, d.tree_offsets, _i32(n), _i32(path),
              d.k_cache, d.v_cache, d.block_table, d.prefix_lens, _i32(free) if len(free) else None,
              free_count, d.workspace, blocks_taken=taken)
    torch.cuda.synchronize()
    return int(taken.item())


def _check_commit(inp, d, want, taken, what):
    assert taken == want["blocks_taken"], what
    np.testing.assert_array_equal(d.block_table.cpu().numpy(), want["block_table"], err_msg=what)
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"], err_msg=what)
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]), err_msg=what)
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]), err_msg=what)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_commit_bit_exact(dtype, D):
    import tree_attention_verify_attn_amd as ta
    trees = [TREE_12, TREE_CHAIN4, TREE_12, TREE_SINGLE, TREE_CHAIN4, TREE_12]
    inp, draft, argmax, free = _batch(71, trees, [63, 64, 130, 0, 1, 250], dtype=dtype, D=D,
                                      p_match=0.9)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    want = oracle.commit(inp, n, path, free, len(free))
    assert want["error"] == 0
    d = to_device(inp)
    say(f"commit {dtype} D={D}: 6 sequences across block boundaries")
    taken = _commit_gpu(inp, d, n, path, free, len(free))
    assert ta.get_error(d.workspace) == 0
    _check_commit(inp, d, want, taken, "commit")


def test_accept_then_commit_on_device():
    import tree_attention_verify_attn_amd as ta
    trees = [TREE_12] * 8 + [TREE_CHAIN4] * 8
    lens = [int(x) for x in np.random.default_rng(3).integers(0, 300, size=16)]
    inp, draft, argmax, free = _batch(72, trees, lens, D=128, p_match=0.8)
    d = to_device(inp)
    say("accept then commit, both on the device")
    n, path, _ = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                  d.workspace)
    taken_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta.commit(d.shape, d.k_tree, d.v_tree, d.parents, d.tree_offsets, n, path, d.k_cache,
              d.v_cache, d.block_table, d.prefix_lens, _i32(free), len(free), d.workspace,
              blocks_taken=taken_t)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wn, wpath, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    want = oracle.commit(inp, wn, wpath, free, len(free))
    _check_commit(inp, d, want, int(taken_t.item()), "accept+commit")


def test_commit_no_blocks_changes_nothing():
    import tree_attention_verify_attn_amd as ta
    inp, draft, argmax, free = _batch(73, [TREE_CHAIN4] * 4, [63, 64, 128, 10], p_match=1.0)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 4)
    want = oracle.commit(inp, n, path, free, 2)
    assert want["error"] == "no_blocks"
    d = to_device(inp)
    say("commit: free list one block short")
    taken = _commit_gpu(inp, d, n, path, free, 2)
    assert ta.get_error(d.workspace) == 8
    _check_commit(inp, d, want, taken, "no blocks")


def test_commit_bad_path_skips_only_that_sequence():
    import tree_attention_verify_attn_amd as ta
    inp, draft, argmax, free = _batch(74, [TREE_12, TREE_12, TREE_CHAIN4], [10, 64, 5], p_match=1.0)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    bad = path.copy()
    bad[0, 2] = 5 if bad[0, 1] != 1 else 6          # not a child of bad[0, 1]
    want = oracle.commit(inp, n, bad, free, len(free))
    assert want["error"] == "bad_tree"
    d = to_device(inp)
    say("commit: one bad path")
    taken = _commit_gpu(inp, d, n, bad, free, len(free))
    assert ta.get_error(d.workspace) == 3
    _check_commit(inp, d, want, taken, "bad path")


def test_commit_twice_in_a_row():
    # the second commit appends after the first (prefix lengths were advanced
    # on the device); the oracle applies the same two steps
    import tree_attention_verify_attn_amd as ta
    inp, draft, argmax, free = _batch(75, [TREE_CHAIN4, TREE_12], [60, 127], spare=10, extra_cols=3,
                                      p_match=1.0)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    first = oracle.commit(inp, n, path, free, len(free))
    second_in = make_inputs(dtype=inp.dtype, num_q_heads=inp.num_q_heads,
                            num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                            prefix_lens=[1, 1], trees=[TREE_CHAIN4, TREE_12],
                            rng=np.random.default_rng(0))
    for k in ("k_tree", "v_tree", "parents", "tree_offsets"):
        setattr(second_in, k, getattr(inp, k))
    second_in.k_cache, second_in.v_cache = first["k_cache"], first["v_cache"]
    second_in.block_table, second_in.prefix_lens = first["block_table"], first["prefix_lens"]
    rest = free[first["blocks_taken"]:]
    second = oracle.commit(second_in, n, path, rest, len(rest))
    d = to_device(inp)
    say("commit twice in a row")
    t1 = _commit_gpu(inp, d, n, path, free, len(free))
    t2 = _commit_gpu(inp, d, n, path, rest, len(rest))
    assert ta.get_error(d.workspace) == 0
    assert t1 == first["blocks_taken"]
    _check_commit(inp, d, second, t2, "second commit")


def test_commit_full_size_ragged_batch_properties():
    # 256 sequences drawn like the ragged large-batch workload (log-normal
    # prefixes, tree mix), checked through properties at full size: the
    # appended rows are the accepted tree rows, tables and lengths advance as
    # the allocation rule says, and untouched sample slots keep their bits.
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(1005)
    B = 256
    z = rng.standard_normal(B)
    lens = np.clip(np.rint(np.exp(np.log(2048.0) + z)), 16, 32768).astype(np.int64)
    kinds = rng.choice(3, size=B, p=[0.2, 0.5, 0.3])
    trees = [(TREE_SINGLE, TREE_CHAIN4, TREE_12)[k] for k in kinds]
    inp = make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                      prefix_lens=lens, trees=trees, rng=rng, spare_blocks=300, extra_table_cols=1)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.7, vocab=32000)
    free = free_list(inp, rng)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    d = to_device(inp)
    say("commit: 256 ragged sequences, full size, property checks")
    taken = _commit_gpu(inp, d, n, path, free, len(free))
    assert ta.get_error(d.workspace) == 0
    table = d.block_table.cpu().numpy()
    plen = d.prefix_lens.cpu().numpy()
    kc = _bits(d.k_cache)
    vc = _bits(d.v_cache)
    kt = _host_bits(inp.k_tree)
    vt = _host_bits(inp.v_tree)
    nxt = 0
    for b in range(B):
        P, A = int(inp.prefix_lens[b]), int(n[b])
        assert plen[b] == P + A
        have, after = -(-P // 64), -(-(P + A) // 64)
        assert list(table[b, :have]) == list(inp.block_table[b, :have])
        assert list(table[b, have:after]) == list(free[nxt:nxt + after - have])
        nxt += after - have
        lo = int(inp.tree_offsets[b])
        for t in range(A):
            pos = P + t
            blk = table[b, pos // 64]
            assert np.array_equal(kc[blk, :, pos % 64], kt[lo + path[b, t]])
            assert np.array_equal(vc[blk, :, pos % 64], vt[lo + path[b, t]])
        # the slot right after the new rows, when in an existing block, is untouched
        pos = P + A
        if pos % 64 and pos // 64 < have:
            blk = table[b, pos // 64]
            assert np.array_equal(kc[blk, :, pos % 64], _host_bits(inp.k_cache)[blk, :, pos % 64])
    assert taken == nxt


def test_commit_bad_prefix_length_skips_only_that_sequence():
    import tree_attention_verify_attn_amd as ta
    inp, draft, argmax, free = _batch(76, [TREE_CHAIN4, TREE_12, TREE_CHAIN4], [10, 64, 5],
                                      p_match=1.0)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    inp.prefix_lens[1] = 64 * inp.max_blocks_per_seq + 1    # beyond the table row
    want = oracle.commit(inp, n, path, free, len(free))
    assert want["error"] == "bad_prefix"
    d = to_device(inp, max_prefix_len=0)
    say("commit: one prefix length beyond its table row")
    taken = _commit_gpu(inp, d, n, path, free, len(free))
    assert ta.get_error(d.workspace) == 6
    _check_commit(inp, d, want, taken, "bad prefix")
