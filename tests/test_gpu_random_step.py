"""A seeded sweep of random batches through the step after verification:
greedy acceptance on the device, then the commit of the accepted paths into
the paged cache (separate tree buffers) or the in-place compaction (tree rows
in the cache), each bit for bit against the oracle.  Trees and forests of 1-256
nodes, batches of 1-64 sequences, prefixes that end anywhere in a block, match
rates 0-1, bf16 and fp32, D 64 and 128.  The case's parameters are printed
before its GPU step."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import say, to_device
from helpers import random_tree
from workloads import free_list, make_inputs, make_tokens, place_tree_in_cache

pytestmark = pytest.mark.gpu

N_CASES = 24


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _bits(t):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else \
        a.numpy().view(np.uint32)


def _host_bits(x):
    return x.view(np.uint16) if x.dtype == np.uint16 else x.view(np.uint32)


def _case(k, incache):
    rng = np.random.default_rng((11000 if incache else 10000) + k)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = 1 if rng.random() < 0.25 else int(rng.integers(2, 65))
    tmax = int(rng.choice([4, 12, 64, 100, 256], p=[0.25, 0.35, 0.2, 0.1, 0.1]))
    trees = [random_tree(rng, int(rng.integers(1, tmax + 1)), forest_p=0.1 if rng.random() < 0.2 else 0.0)
             for _ in range(B)]
    lens = [int(rng.integers(0, 600)) for _ in range(B)]
    p_match = float(rng.choice([0.0, 0.5, 0.8, 1.0]))
    inp = make_inputs(dtype=dtype, num_q_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=D, prefix_lens=lens,
                      trees=trees, rng=rng, seed=10000 + k, spare_blocks=5 * B + 4, extra_table_cols=5)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=p_match, vocab=8)
    return rng, inp, draft, argmax, p_match


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_accept_then_commit_bit_exact(k):
    import tree_attention_verify_attn_amd as ta
    rng, inp, draft, argmax, p_match = _case(k, incache=False)
    free = free_list(inp, rng)
    d = to_device(inp)
    say(f"random step {k}: {inp.dtype} D={inp.head_dim} B={inp.batch} trees<={inp.max_tree_nodes} "
        f"P<={inp.max_prefix_len} p_match={p_match} free={len(free)}")
    n, path, bonus = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                      d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wn, wpath, wbonus = oracle.accept_greedy(inp.parents, inp.tree_offsets, draft, argmax,
                                             d.shape.max_tree_nodes)
    np.testing.assert_array_equal(n.cpu().numpy(), wn)
    np.testing.assert_array_equal(path.cpu().numpy(), wpath)
    np.testing.assert_array_equal(bonus.cpu().numpy(), wbonus)
    want = oracle.commit(inp, wn, wpath, free, len(free))
    assert want["error"] == 0
    taken = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta.commit(d.shape, d.k_tree, d.v_tree, d.parents, d.tree_offsets, n, path, d.k_cache, d.v_cache,
              d.block_table, d.prefix_lens, _i32(free) if len(free) else None, len(free), d.workspace,
              blocks_taken=taken)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    assert int(taken.item()) == want["blocks_taken"]
    np.testing.assert_array_equal(d.block_table.cpu().numpy(), want["block_table"])
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_accept_then_commit_incache_bit_exact(k):
    import tree_attention_verify_attn_amd as ta
    rng, inp, draft, argmax, p_match = _case(k, incache=True)
    ic, _ = place_tree_in_cache(inp, rng)
    d = to_device(ic)
    say(f"random in-cache step {k}: {ic.dtype} D={ic.head_dim} B={ic.batch} "
        f"trees<={ic.max_tree_nodes} P<={ic.max_prefix_len} p_match={p_match}")
    n, path, _ = ta.accept_greedy(d.shape, d.parents, d.tree_offsets, _i32(draft), _i32(argmax),
                                  d.workspace)
    ta.commit_incache(d.shape, d.parents, d.tree_offsets, n, path, d.k_cache, d.v_cache,
                      d.block_table, d.prefix_lens, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wn, wpath, _ = oracle.accept_greedy(ic.parents, ic.tree_offsets, draft, argmax,
                                        d.shape.max_tree_nodes)
    want = oracle.commit_incache(ic, wn, wpath)
    assert want["error"] == 0
    np.testing.assert_array_equal(d.prefix_lens.cpu().numpy(), want["prefix_lens"])
    np.testing.assert_array_equal(_bits(d.k_cache), _host_bits(want["k_cache"]))
    np.testing.assert_array_equal(_bits(d.v_cache), _host_bits(want["v_cache"]))
