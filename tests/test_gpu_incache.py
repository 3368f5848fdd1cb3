"""GPU parity for the in-cache tree layout: the tree K/V rows sit in the paged
cache right after each prefix.  Verify against the fp64 oracle (same
tolerances as the separate-buffer verify); the in-place commit bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_lse, host, say, to_device, tolerances
from helpers import random_tree
from workloads import (TREE_12, TREE_CHAIN4, TREE_SINGLE, make_inputs, make_tokens,
                       place_tree_in_cache)

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _bits(t):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else \
        a.numpy().view(np.uint32)


def _host_bits(x):
    return x.view(np.uint16) if x.dtype == np.uint16 else x.view(np.uint32)


def _incache(seed, trees, lens, *, dtype="bf16", Hq=8, Hkv=2, D=128, poison_tree=True):
    rng = np.random.default_rng(seed)
    inp = make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_lens=lens,
                      trees=trees, rng=rng, spare_blocks=2 * len(lens) + 2, extra_table_cols=2)
    ic, _ = place_tree_in_cache(inp, rng)
    if poison_tree:   # the in-cache path must not read the separate tree rows
        nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
        ic.k_tree = np.full_like(inp.k_tree, nan)
        ic.v_tree = np.full_like(inp.v_tree, nan)
    return inp, ic


def _run_incache(ic, **kw):
    import tree_attention_verify_attn_amd as ta
    d = to_device(ic, **kw)
    out, lse = ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                                 d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    return d, out, lse


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_verify_incache_matches_oracle(dtype, D):
    import tree_attention_verify_attn_amd as ta
    trees = [TREE_12, TREE_CHAIN4, TREE_SINGLE, TREE_12, [-1, 0, 0, 1, 1, 2, 2]]
    inp, ic = _incache(81, trees, [700, 63, 0, 64, 130], dtype=dtype, D=D)
    say(f"verify_incache {dtype} D={D}: 5 sequences, tree regions across block boundaries")
    d, out, lse = _run_incache(ic)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    tol_o, tol_l = tolerances(ic)
    assert_close(host(out), o_want, tol_o, "incache o")
    assert_close_lse(host(lse), l_want, tol_l, "incache lse")


def test_verify_incache_one_sequence_8k():
    import tree_attention_verify_attn_amd as ta
    inp, ic = _incache(82, [TREE_12], [8190], Hq=32, Hkv=8)   # tree spans two blocks
    say("verify_incache: one sequence, 8190-token prefix, 12-node tree over a block boundary")
    d, out, lse = _run_incache(ic)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    assert_close(host(out), o_want, 2e-2, "incache 8k o")
    assert_close_lse(host(lse), l_want, 1e-3, "incache 8k lse")


def test_verify_incache_equals_separate_buffers():
    # same rows, two layouts: the fused kernel gives the same output bits
    import tree_attention_verify_attn_amd as ta
    trees = [random_tree(np.random.default_rng(i), 9) for i in range(6)]
    inp, ic = _incache(83, trees, [300, 64, 65, 1, 129, 1000])
    say("verify_incache vs verify on the same rows")
    d, out_ic, lse_ic = _run_incache(ic)
    d2 = to_device(inp)
    out_sep, lse_sep = ta.verify(d2.shape, d2.q, d2.k_cache, d2.v_cache, d2.block_table,
                                 d2.prefix_lens, d2.k_tree, d2.v_tree, d2.parents, d2.tree_offsets,
                                 d2.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0 and ta.get_error(d2.workspace) == 0
    assert torch.equal(out_ic.view(torch.int16), out_sep.view(torch.int16))
    assert torch.equal(lse_ic, lse_sep)


def test_verify_incache_bad_region_block_flagged():
    import tree_attention_verify_attn_amd as ta
    inp, ic = _incache(84, [TREE_12, TREE_CHAIN4], [60, 10])
    d = to_device(ic)
    d.block_table[0, 1] = ic.num_blocks + 3      # second block of sequence 0's tree region
    say("verify_incache: bad region block id")
    ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens, d.parents,
                      d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 6


def _commit_case(seed, trees, lens, p_match=0.8):
    rng = np.random.default_rng(seed)
    inp = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=4, head_dim=128, prefix_lens=lens,
                      trees=trees, rng=rng, spare_blocks=2 * len(lens) + 2, extra_table_cols=2)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=20)
    n, path, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax,
                                      inp.max_tree_nodes)
    ic, _ = place_tree_in_cache(inp, rng)
    return inp, ic, n, path


def _commit_gpu(ic, n, path):
    import tree_attention_verify_attn_amd as ta
    d = to_device(ic)
    ta.commit_incache(d.shape, d.parents, d.tree_offsets, _i32(n), _i32(path), d.k_cache, d.v_cache,
                      d.block_table, d.prefix_lens, d.workspace)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("p_match", [0.0, 0.8, 1.0])
def test_commit_incache_bit_exact(p_match):
    import tree_attention_verify_attn_amd as ta
    trees = [TREE_12, TREE_CHAIN4, TREE_SINGLE, TREE_12, list(range(-1, 63))]
    inp, ic, n, path = _commit_case(85, trees, [63, 64, 0, 120, 70], p_match=p_match)
    want = oracle.commit_incache(ic, n, path)
    assert want["error"] == 0
    say(f"commit_incache p_match {p_match}")
    d = _commit_gpu(ic, n, path)
    assert ta.get_error(d.workspace) == 0
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))


def test_commit_incache_bad_path_skips_sequence():
    import tree_attention_verify_attn_amd as ta
    inp, ic, n, path = _commit_case(86, [TREE_12, TREE_12], [10, 70], p_match=1.0)
    bad = path.copy()
    bad[1, 1] = 2 if bad[1, 1] != 2 else 3
    bad[1, 2] = 4 if bad[1, 1] != 1 else 5
    want = oracle.commit_incache(ic, n, bad)
    assert want["error"] == "bad_tree"
    say("commit_incache: one bad path")
    d = _commit_gpu(ic, n, bad)
    assert ta.get_error(d.workspace) == 3
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))


def test_incache_step_then_verify_again():
    # a full in-cache step on the device: verify, accept, commit; then the next
    # step's tree rows go after the new prefix and verify again -- against the
    # oracle applied to the same sequence of operations
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(87)
    trees = [TREE_12, TREE_CHAIN4, TREE_12]
    inp = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                      prefix_lens=[100, 63, 250], trees=trees, rng=rng, spare_blocks=10,
                      extra_table_cols=2)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.8, vocab=20)
    ic, free = place_tree_in_cache(inp, rng)
    d = to_device(ic, max_prefix_len=ic.max_prefix_len + 64)   # room for the grown prefixes
    say("in-cache step: verify, accept, commit, verify again")
    ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens, d.parents,
                      d.tree_offsets, d.workspace)
    n, path, _ = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                  d.workspace)
    ta.commit_incache(d.shape, d.parents, d.tree_offsets, n, path, d.k_cache, d.v_cache,
                      d.block_table, d.prefix_lens, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wn, wpath, _ = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax, 12)
    committed = oracle.commit_incache(ic, wn, wpath)
    # next step: new tree rows at the new prefix ends (written on host and device alike)
    nxt = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                      prefix_lens=[1, 1, 1], trees=trees, rng=rng)
    step2 = make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                        prefix_lens=[1, 1, 1], trees=trees, rng=np.random.default_rng(0))
    step2.q, step2.k_tree, step2.v_tree = nxt.q, nxt.k_tree, nxt.v_tree
    step2.k_cache, step2.v_cache = committed["k_cache"], committed["v_cache"]
    step2.block_table, step2.prefix_lens = ic.block_table, committed["prefix_lens"]
    ic2, _ = place_tree_in_cache(step2, np.random.default_rng(1))
    assert np.array_equal(ic2.block_table, ic.block_table)   # the regions fit the existing blocks
    d.q = torch.from_numpy(nxt.q.view(np.int16)).cuda().view(torch.bfloat16)
    d.k_cache.copy_(torch.from_numpy(ic2.k_cache.view(np.int16)).cuda().view(torch.bfloat16))
    d.v_cache.copy_(torch.from_numpy(ic2.v_cache.view(np.int16)).cuda().view(torch.bfloat16))
    out, lse = ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                                 d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    assert np.array_equal(d.prefix_lens.cpu().numpy(), committed["prefix_lens"])
    o_want, l_want, _ = oracle.verify_incache(ic2)
    assert_close(host(out), o_want, 2e-2, "second step o")
    assert_close_lse(host(lse), l_want, 1e-3, "second step lse")
