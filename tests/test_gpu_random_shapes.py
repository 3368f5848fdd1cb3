"""A seeded sweep of random shapes through the fused verify and the split
path (mask words bit for bit, prefix pass, suffix pass, merge), each against
the fp64 oracle: batch sizes, GQA groupings, head dims,
dtypes, ragged prefix lengths (empty ones included), trees of 1-256 nodes
and forests, caller chunk sizes and a max_prefix_len above the actual
lengths.  Together they reach every launch mode (first round with the
meeting, two launches, the device-chosen chunk, tickets with the solo
combine) in combinations the hand-picked cases do not.  The case's
parameters are printed before its GPU step."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close, assert_close_lse, host, run_split, run_verify, say, to_device,
                      tolerances)
from helpers import random_tree
from workloads import make_inputs, place_tree_in_cache

pytestmark = pytest.mark.gpu

N_CASES = 64
MAX_MACS = 6e8  # oracle work per case: sum over sequences of T x Hq x (P + T) x D


def _case(k, incache=False, short=False):
    rng = np.random.default_rng((9000 if incache else 11000 if short else 7000) + k)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8]))
    while Hkv * G > 64:
        G //= 2
    Hq = Hkv * G
    B = 1 if rng.random() < 0.4 else int(rng.integers(2, 49))
    tmax = int(rng.choice([4, 12, 12, 64, 100, 256], p=[0.2, 0.3, 0.2, 0.1, 0.1, 0.1]))
    trees = [random_tree(rng, int(rng.integers(1, tmax + 1)), forest_p=0.05 if rng.random() < 0.2 else 0.0)
             for _ in range(B)]
    lens = []
    # short: up to 3, 6 or 7 blocks (one chunk per sequence, and past the bounds)
    ub = int(rng.choice([192, 384, 448])) if short else 0
    for _ in range(B):
        u = rng.random()
        if short:
            lens.append(0 if u < 0.1 else int(rng.integers(1, ub + 1)))
        else:
            lens.append(0 if u < 0.08 else int(rng.integers(1, 64)) if u < 0.2 else int(rng.integers(64, 6000)))
    # keep the oracle's work bounded: shorten prefixes until it fits
    def macs():
        return sum(len(t) * Hq * (p + len(t)) * D for t, p in zip(trees, lens))
    while macs() > MAX_MACS and any(lens):
        lens = [p // 2 for p in lens]
    while macs() > MAX_MACS and len(trees) > 1:  # large trees alone: fewer sequences
        trees, lens = trees[:-1], lens[:-1]
    B = len(trees)
    split = 0 if short else int(rng.choice([0, 0, 0, 64, 128, 320, 1024]))
    extra = int(rng.integers(5, 40)) if rng.random() < (0.4 if short else 0.2) else 0
    spare = int(rng.integers(0, 5))
    if incache:   # room in every table row and in the pool for a tree region
        extra, spare = max(extra, 5), spare + 5 * B + 2
    inp = make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_lens=lens,
                      trees=trees, rng=rng, seed=(11000 if short else 7000) + k,
                      name=f"random{k}", permute_blocks=True,
                      spare_blocks=spare, extra_table_cols=extra)
    max_p = None
    if extra and not incache:
        max_p = min(inp.max_blocks_per_seq * 64, max(inp.max_prefix_len, 1) + 64 * extra // 2)
    elif extra > 5:   # in-cache: the bound leaves room for the tree region
        max_p = min(inp.max_blocks_per_seq * 64 - 64 * 5, max(inp.max_prefix_len, 1) + 64 * extra // 2)
        max_p = max(max_p, inp.max_prefix_len)
    if incache:
        inp, _ = place_tree_in_cache(inp, rng)
    return inp, split, max_p


def _split(d):
    import tree_attention_verify_attn_amd as ta
    out, lse, (po, pl, so, sl, mask) = run_split(d)
    return so, sl, out, lse, mask


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape_against_oracle(k):
    inp, split, max_p = _case(k)
    _check_case(f"random {k}", inp, split, max_p)


N_SHORT = 24


@pytest.mark.parametrize("k", range(N_SHORT))
def test_random_short_prefixes_against_oracle(k):
    """Prefixes of at most 7 blocks and the library's own chunk: one chunk per
    sequence (chosen by the host from max_prefix_len, or by the kernel from
    the actual lengths when max_prefix_len is larger) or, past the bounds,
    split as before."""
    inp, split, max_p = _case(k, short=True)
    _check_case(f"random short {k}", inp, split, max_p)


def _check_case(k, inp, split, max_p):
    import tree_attention_verify_attn_amd as ta
    d = to_device(inp, split_tokens=split, max_prefix_len=max_p)
    info = ta.launch_info(d.shape)
    say(f"{k}: {inp.dtype} B={inp.batch} Hq={inp.num_q_heads} Hkv={inp.num_kv_heads} "
        f"D={inp.head_dim} trees<={inp.max_tree_nodes} P<={inp.max_prefix_len} "
        f"max_prefix_len={d.shape.max_prefix_len} split={split}: {info}")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, f"{k} o")
    assert_close_lse(host(lse), l_want, tol_l, f"{k} lse")
    po, pl = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                       d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wpo, wpl = oracle.prefix_only(inp)
    assert_close(host(po), wpo, tol_o, f"{k} prefix o")
    assert_close_lse(host(pl), wpl, tol_l, f"{k} prefix lse")
    # the split path: mask words bit for bit, the suffix pass and the merged result
    so_, sl_, mo, ml, mask = _split(d)
    W = -(-d.shape.max_tree_nodes // 64)
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint64).reshape(-1, W),
                                  oracle.build_masks_words(inp, W).reshape(-1, W))
    wso, wsl = oracle.suffix_only(inp)
    assert_close(host(so_), wso, tol_o, f"{k} suffix o")
    assert_close_lse(host(sl_), wsl, tol_l, f"{k} suffix lse")
    assert_close(host(mo), o_want, tol_o, f"{k} split o")
    assert_close_lse(host(ml), l_want, tol_l, f"{k} split lse")


N_INCACHE = 24


@pytest.mark.parametrize("k", range(N_INCACHE))
def test_random_incache_against_oracle(k):
    """The same kind of sweep with each tree's K/V rows in the paged cache
    right after its prefix (tree_attn_verify_incache)."""
    import tree_attention_verify_attn_amd as ta
    ic, split, max_p = _case(k, incache=True)
    d = to_device(ic, split_tokens=split, max_prefix_len=max_p)
    say(f"random in-cache shape {k}: {ic.dtype} B={ic.batch} Hq={ic.num_q_heads} Hkv={ic.num_kv_heads} "
        f"D={ic.head_dim} trees<={ic.max_tree_nodes} P<={ic.max_prefix_len} "
        f"max_prefix_len={d.shape.max_prefix_len} split={split}")
    out, lse = ta.verify_incache(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                                 d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    o_want, l_want, _ = oracle.verify_incache(ic)
    tol_o, tol_l = tolerances(ic)
    assert_close(host(out), o_want, tol_o, f"random in-cache {k} o")
    assert_close_lse(host(lse), l_want, tol_l, f"random in-cache {k} lse")
