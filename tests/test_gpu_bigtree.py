"""GPU parity for trees of more than 64 nodes (up to 256): multi-word masks
bit for bit; mask + prefix + suffix + merge (split path) and the fused verify
against the fp64 oracle.  Also the draft-side shape: short prefixes under
large trees (multi-round drafting attends with the same kernels)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close, assert_close_lse, host, run_split, run_verify, say,
                      to_device, tolerances)
from helpers import random_tree
from workloads import make_config, make_inputs

pytestmark = pytest.mark.gpu


def _big(seed, trees, lens, *, dtype="bf16", Hq=8, Hkv=2, D=128):
    rng = np.random.default_rng(seed)
    return make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       prefix_lens=lens, trees=trees, rng=rng, spare_blocks=2)


def _trees(seed):
    rng = np.random.default_rng(seed)
    return [random_tree(rng, 200), list(range(-1, 99)), [-1] + [0] * 64,
            random_tree(rng, 256, forest_p=0.05), random_tree(rng, 70)]


def test_multiword_masks_bit_exact():
    import tree_attention_verify_attn_amd as ta
    trees = _trees(1)
    inp = _big(91, trees, [1] * len(trees))
    d = to_device(inp, max_tree_nodes=256)
    say("multi-word masks: trees of 200, 99, 65, 256, 70 nodes")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    got = mask.cpu().numpy().view(np.uint64)
    want = oracle.build_masks_words(inp, 4)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_split_path_large_trees_matches_oracle(dtype, D):
    import tree_attention_verify_attn_amd as ta
    trees = _trees(2)
    inp = _big(92, trees, [300, 0, 1000, 65, 7], dtype=dtype, D=D)
    d = to_device(inp, max_tree_nodes=256)
    say(f"split path, trees up to 256 nodes, {dtype} D={D}")
    out, lse, _ = run_split(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, "big-tree o")
    assert_close_lse(host(lse), l_want, tol_l, "big-tree lse")


def test_draft_side_short_prefixes_under_large_trees():
    # multi-round drafting: the draft model's queries see a short context and a
    # large tree; 8 sequences, prefixes 16..100, 128-node trees, GQA 32/8
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(93)
    trees = [random_tree(rng, 128) for _ in range(8)]
    lens = [int(x) for x in rng.integers(16, 101, size=8)]
    inp = make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                      prefix_lens=lens, trees=trees, rng=rng)
    d = to_device(inp, max_tree_nodes=128)
    say("draft-side shape: 8 x 128-node trees over 16..100-token prefixes")
    out, lse, _ = run_split(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    assert_close(host(out), o_want, 2e-2, "draft-side o")
    assert_close_lse(host(lse), l_want, 1e-3, "draft-side lse")


def test_large_tree_bad_parent_flagged():
    import tree_attention_verify_attn_amd as ta
    trees = _trees(3)
    inp = _big(94, trees, [10] * len(trees))
    d = to_device(inp, max_tree_nodes=256)
    d.parents[150] = 170       # a later node of the 200-node tree
    say("multi-word mask: bad parent flagged")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 3
    got = mask.cpu().numpy().view(np.uint64)
    assert not got[:200].any()          # the bad tree's words are zero
    want = oracle.build_masks_words(inp, 4)
    np.testing.assert_array_equal(got[200:], want[200:])   # the others are intact


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_fused_verify_large_trees_matches_oracle(dtype, D):
    # trees of 65..256 nodes in one launch: the last chunk of each group runs
    # the tree's 64-node segments after its KV blocks
    import tree_attention_verify_attn_amd as ta
    trees = _trees(5)
    inp = _big(95, trees, [300, 0, 1000, 65, 7], dtype=dtype, D=D)
    d = to_device(inp, max_tree_nodes=256)
    say(f"fused verify, trees up to 256 nodes, {dtype} D={D}")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, "fused big-tree o")
    assert_close_lse(host(lse), l_want, tol_l, "fused big-tree lse")


def test_deep_chains_every_pointer_jumping_round():
    # Chains are the deepest trees: a 256-node chain needs all eight
    # pointer-jumping rounds (a link reaches 2^k ancestors after round k), a
    # 129-node chain exactly eight, a 128-node chain seven.  The rounds stop
    # early once no node has a link left, so these pin the last round in the
    # mask kernel, the split path and the fused verify (one launch with all
    # three, and one sequence with the 256-node chain alone).
    import tree_attention_verify_attn_amd as ta
    chains = [list(range(-1, 255)), list(range(-1, 128)), list(range(-1, 127))]
    inp = _big(97, chains, [130, 0, 700])
    d = to_device(inp, max_tree_nodes=256)
    say("deep chains of 256, 129 and 128 nodes: masks, split path, fused verify")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint64), oracle.build_masks_words(inp, 4))
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    out, lse, _ = run_split(d)
    assert ta.get_error(d.workspace) == 0
    assert_close(host(out), o_want, tol_o, "deep chains, split path o")
    assert_close_lse(host(lse), l_want, tol_l, "deep chains, split path lse")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    assert_close(host(out), o_want, tol_o, "deep chains, fused o")
    assert_close_lse(host(lse), l_want, tol_l, "deep chains, fused lse")
    one = _big(98, [chains[0]], [2000], Hq=8, Hkv=2)
    d1 = to_device(one, max_tree_nodes=256, split_tokens=512)
    say("deep chain of 256 nodes, one sequence in 4 chunks")
    out, lse = run_verify(d1)
    assert ta.get_error(d1.workspace) == 0
    o_want, l_want, _ = oracle.verify(one)
    assert_close(host(out), o_want, tol_o, "deep chain one sequence o")
    assert_close_lse(host(lse), l_want, tol_l, "deep chain one sequence lse")


def test_fused_verify_large_tree_one_sequence_split_chunks():
    # one sequence (numbered without a table), a 256-node tree over a
    # 4000-token prefix cut into many chunks; small trees mixed in are covered
    # by the test above
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(96)
    inp = _big(96, [random_tree(rng, 256)], [4000], Hq=8, Hkv=2)
    d = to_device(inp, max_tree_nodes=256, split_tokens=256)
    say("fused verify, one sequence, 256-node tree, 16 chunks")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    assert_close(host(out), o_want, 2e-2, "one-sequence big-tree o")
    assert_close_lse(host(lse), l_want, 1e-3, "one-sequence big-tree lse")


@pytest.mark.parametrize("dtype,D,mode", [("bf16", 128, "two_launch"), ("f32", 64, "two_launch"),
                                          ("bf16", 64, "first_round")])
def test_fused_verify_large_tree_one_sequence_first_round(dtype, D, mode):
    # one sequence, a 256-node tree, 16 chunks a group and every item in the
    # first round: two launches (partials, then the combine kernel), except
    # bf16 at head dim 64, whose large-tree kernel meets in the launch
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(97)
    inp = _big(97, [random_tree(rng, 256)], [4000], Hq=2, Hkv=2, dtype=dtype, D=D)
    d = to_device(inp, max_tree_nodes=256, split_tokens=256)
    info = ta.launch_info(d.shape)
    say(f"fused verify, one sequence, 256-node tree, {dtype} D={D}: {info}")
    assert info["mode"] == mode, info
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, f"one-sequence big-tree {dtype} D={D} o")
    assert_close_lse(host(lse), l_want, tol_l, f"one-sequence big-tree {dtype} D={D} lse")


def test_fused_verify_draft_side_matches_split():
    # the draft-side shape through the fused verify, against the oracle and
    # the split path
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(97)
    trees = [random_tree(rng, 128) for _ in range(8)]
    lens = [int(x) for x in rng.integers(16, 101, size=8)]
    inp = make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                      prefix_lens=lens, trees=trees, rng=rng)
    d = to_device(inp, max_tree_nodes=128)
    say("fused verify, draft-side shape")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    assert_close(host(out), o_want, 2e-2, "fused draft-side o")
    assert_close_lse(host(lse), l_want, 1e-3, "fused draft-side lse")
    out2, lse2, _ = run_split(d)
    assert_close(host(out), host(out2), 2e-2, "fused vs split o")


def test_fused_verify_large_tree_bad_parent_flagged():
    import tree_attention_verify_attn_amd as ta
    trees = _trees(6)
    inp = _big(98, trees, [100] * len(trees))
    d = to_device(inp, max_tree_nodes=256)
    d.parents[150] = 170       # a later node of the 200-node tree
    say("fused verify, large tree with a bad parent")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 3
    # every other sequence is still right
    o_want, l_want, _ = oracle.verify(inp)
    off = inp.tree_offsets
    rows = slice(int(off[1]), int(off[-1]))
    assert_close(host(out)[rows], o_want[rows], 2e-2, "other sequences o")


def test_fused_verify_full_size_256_node_tree():
    # the 8k-prefix, 256-node workload at full size in the benchmark's launch
    # configuration (library chunking; one-sequence numbering, row passes of
    # a KV head placed together), fused and split: every row against the oracle
    import tree_attention_verify_attn_amd as ta
    inp = make_config(6)
    d = to_device(inp)
    say(f"fused verify, 256-node tree over 8192 tokens, split_tokens {ta.split_tokens(d.shape)}")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    assert_close(host(out), o_want, 2e-2, "256-node full o")
    assert_close_lse(host(lse), l_want, 1e-3, "256-node full lse")
    say("split path, same workload")
    out2, lse2, _ = run_split(d)
    assert ta.get_error(d.workspace) == 0
    assert_close(host(out2), o_want, 2e-2, "256-node split o")
    assert_close_lse(host(lse2), l_want, 1e-3, "256-node split lse")


def test_fused_verify_full_size_draft_side():
    # the draft-side workload at full size (8 sequences, 128-node trees,
    # 16..100-token prefixes): every row against the oracle
    import tree_attention_verify_attn_amd as ta
    inp = make_config(7)
    d = to_device(inp)
    say("fused verify, draft-side workload at full size")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    assert_close(host(out), o_want, 2e-2, "draft-side full o")
    assert_close_lse(host(lse), l_want, 1e-3, "draft-side full lse")
