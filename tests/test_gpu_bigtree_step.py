"""GPU parity of the verify step's other half for trees of 65..256 nodes: the
in-cache verify (tree rows in the paged cache after each prefix, a region of
up to 5 blocks) against the fp64 oracle, greedy acceptance and both commits
bit for bit, and a whole step (verify, accept, commit) on the device.
Tolerances as in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_lse, host, run_verify, say, to_device, tolerances
from helpers import random_tree
from workloads import free_list, make_inputs, make_tokens, place_tree_in_cache

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _bits(t):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else \
        a.numpy().view(np.uint32)


def _host_bits(x):
    return x.view(np.uint16) if x.dtype == np.uint16 else x.view(np.uint32)


def _large_trees(seed):
    # the last one, a 256-node chain, is the deepest tree: its ancestor sets
    # take all eight pointer-jumping rounds and its whole-path commit moves
    # 256 rows
    rng = np.random.default_rng(seed)
    return [random_tree(rng, 200), list(range(-1, 99)), [-1] + [0] * 64,
            random_tree(rng, 256, forest_p=0.05), random_tree(rng, 70), list(range(-1, 255))]


def _incache(seed, trees, lens, *, dtype="bf16", Hq=8, Hkv=2, D=128):
    rng = np.random.default_rng(seed)
    inp = make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_lens=lens,
                      trees=trees, rng=rng, spare_blocks=6 * len(lens) + 2, extra_table_cols=5)
    ic, _ = place_tree_in_cache(inp, rng)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    ic.k_tree = np.full_like(inp.k_tree, nan)      # the in-cache path must not read these
    ic.v_tree = np.full_like(inp.v_tree, nan)
    return inp, ic


def _verify_incache(d):
    import tree_attention_verify_attn_amd as ta
    out, lse = ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                                 d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------ in-cache verify
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_verify_incache_large_trees_matches_oracle(dtype, D):
    import tree_attention_verify_attn_amd as ta
    # P = 63 under the 256-node tree: its region touches 5 blocks
    inp, ic = _incache(401, _large_trees(4), [130, 1, 0, 63, 64, 100], dtype=dtype, D=D)
    d = to_device(ic, max_tree_nodes=256)
    say(f"verify_incache large trees {dtype} D={D}: {ta.launch_info(d.shape)}")
    out, lse = _verify_incache(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    tol_o, tol_l = tolerances(ic)
    assert_close(host(out), o_want, tol_o, "large in-cache o")
    assert_close_lse(host(lse), l_want, tol_l, "large in-cache lse")


@pytest.mark.parametrize("split", [0, 4096])
def test_verify_incache_large_tree_one_sequence(split):
    # one 8190-token sequence, 256-node tree across 5 blocks; split 0: items
    # numbered without a table (the region's ids ride spare lanes of the
    # block-id load); 4096: 64-block chunks leave no spare lanes (table mode)
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(402)
    inp, ic = _incache(402, [random_tree(rng, 256)], [8190], Hq=16, Hkv=4)
    d = to_device(ic, split_tokens=split, max_tree_nodes=256)
    say(f"verify_incache one sequence, 256 nodes at 8190: {ta.launch_info(d.shape)}")
    out, lse = _verify_incache(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    assert_close(host(out), o_want, 2e-2, "one sequence o")
    assert_close_lse(host(lse), l_want, 1e-3, "one sequence lse")


def test_verify_incache_large_equals_separate_buffers():
    inp, ic = _incache(403, _large_trees(5), [700, 63, 5, 128, 1, 64])
    say("verify_incache vs separate tree rows, large trees")
    out_ic, lse_ic = _verify_incache(to_device(ic, max_tree_nodes=256))
    out_sep, lse_sep = run_verify(to_device(inp, max_tree_nodes=256))
    assert torch.equal(out_ic, out_sep) and torch.equal(lse_ic, lse_sep)


def test_verify_incache_large_bad_region_block_flagged():
    import tree_attention_verify_attn_amd as ta
    inp, ic = _incache(404, [random_tree(np.random.default_rng(1), 200), [-1, 0]], [63, 10])
    d = to_device(ic, max_tree_nodes=256)
    d.block_table[0, 3] = ic.num_blocks + 7       # a block of the first tree's region
    say("verify_incache large tree: bad region block")
    _verify_incache(d)
    assert ta.get_error(d.workspace) == 6


# ---------------------------------------------------------------- acceptance
def _accept(d, draft, argmax):
    import tree_attention_verify_attn_amd as ta
    n, path, bonus = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                      d.workspace)
    torch.cuda.synchronize()
    return n.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy()


@pytest.mark.parametrize("p_match", [0.0, 0.5, 0.9, 1.0])
def test_accept_large_trees_bit_exact(p_match):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(410)
    trees = [random_tree(rng, int(rng.integers(65, 257)), forest_p=0.05 if i % 4 == 0 else 0.0)
             for i in range(24)]
    trees += [list(range(-1, 255)), [-1] + [0] * 255, random_tree(rng, 30)]
    inp = make_inputs(dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=64,
                      prefix_lens=[1] * len(trees), trees=trees, rng=rng)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=3)
    d = to_device(inp, max_tree_nodes=256)
    say(f"accept: {len(trees)} trees of up to 256 nodes, p_match {p_match}")
    n, path, bonus = _accept(d, draft, argmax)
    assert ta.get_error(d.workspace) == 0
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 256)
    np.testing.assert_array_equal(n, wn)
    np.testing.assert_array_equal(path, wpath)
    np.testing.assert_array_equal(bonus, wbonus)


def test_accept_large_bad_tree_flagged():
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(411)
    trees = [random_tree(rng, 150), random_tree(rng, 90)]
    inp = make_inputs(dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=64,
                      prefix_lens=[1, 1], trees=trees, rng=rng)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.9, vocab=5)
    d = to_device(inp, max_tree_nodes=256)
    d.parents[100] = 120                          # a later node as parent
    say("accept: bad parent in a 150-node tree")
    n, path, bonus = _accept(d, draft, argmax)
    assert ta.get_error(d.workspace) == 3
    assert n[0] == 0 and bonus[0] == -1 and (path[0] == -1).all()
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents[150:], np.array([0, 90]), draft[150:],
                                             argmax[150:], 256)
    assert n[1] == wn[0] and (path[1] == wpath[0]).all() and bonus[1] == wbonus[0]


# -------------------------------------------------------------------- commit
@pytest.mark.parametrize("p_match", [0.5, 1.0])
def test_commit_large_trees_bit_exact(p_match):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(420)
    trees = _large_trees(6)
    inp = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=128,
                      prefix_lens=[63, 0, 200, 64, 1, 20], trees=trees, rng=rng, spare_blocks=40,
                      extra_table_cols=5)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=5)
    free = free_list(inp, rng)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 256)
    want = oracle.commit(inp, n, path, free, len(free))
    assert want["error"] == 0
    d = to_device(inp, max_tree_nodes=256)
    taken = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"commit: large trees, p_match {p_match}, paths of {list(n)} nodes")
    ta.commit(d.shape, d.k_tree, d.v_tree, d.parents, d.tree_offsets, _i32(n), _i32(path),
              d.k_cache, d.v_cache, d.block_table, d.prefix_lens, _i32(free), len(free),
              d.workspace, blocks_taken=taken)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    assert int(taken.item()) == want["blocks_taken"]
    np.testing.assert_array_equal(d.block_table.cpu().numpy(), want["block_table"])
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))


@pytest.mark.parametrize("p_match", [0.0, 0.8, 1.0])
def test_commit_incache_large_trees_bit_exact(p_match):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(430)
    trees = _large_trees(7)
    inp = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=4, head_dim=128,
                      prefix_lens=[63, 64, 0, 63, 130, 1], trees=trees, rng=rng, spare_blocks=40,
                      extra_table_cols=5)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=4)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 256)
    ic, _ = place_tree_in_cache(inp, rng)
    want = oracle.commit_incache(ic, n, path)
    assert want["error"] == 0
    d = to_device(ic, max_tree_nodes=256)
    say(f"commit_incache: large trees, p_match {p_match}, paths of {list(n)} nodes")
    ta.commit_incache(d.shape, d.parents, d.tree_offsets, _i32(n), _i32(path), d.k_cache,
                      d.v_cache, d.block_table, d.prefix_lens, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))


def test_large_tree_incache_step_on_device():
    # verify, accept and commit of 65..256-node trees on the device, in the
    # in-cache layout, against the oracle applied to the same operations
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(440)
    trees = [random_tree(rng, 256), random_tree(rng, 120), list(range(-1, 79))]
    inp = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                      prefix_lens=[63, 1000, 5], trees=trees, rng=rng, spare_blocks=20,
                      extra_table_cols=5)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.95, vocab=3)
    ic, _ = place_tree_in_cache(inp, rng)
    d = to_device(ic, max_tree_nodes=256)
    say("large-tree in-cache step: verify, accept, commit")
    out, lse = ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                                 d.parents, d.tree_offsets, d.workspace)
    n, path, bonus = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                      d.workspace)
    ta.commit_incache(d.shape, d.parents, d.tree_offsets, n, path, d.k_cache, d.v_cache,
                      d.block_table, d.prefix_lens, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    assert_close(host(out), o_want, 2e-2, "step o")
    assert_close_lse(host(lse), l_want, 1e-3, "step lse")
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 256)
    np.testing.assert_array_equal(n.cpu().numpy(), wn)
    np.testing.assert_array_equal(path.cpu().numpy(), wpath)
    np.testing.assert_array_equal(bonus.cpu().numpy(), wbonus)
    want = oracle.commit_incache(ic, wn, wpath)
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))
