"""Pins for the oracle's attention (CPU only).

Each check ties the oracle to something other than itself: a hand-derived
closed form, a library attention routine (torch SDPA in fp64 with an explicit
mask built here), algebraic invariants of softmax attention, and brute-force
perturbation.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (dp_masks, f64, manual_inputs, random_tree, read_hand_example,
                     small_inputs)
from workloads import TREE_12, TREE_CHAIN4, make_config, make_inputs


# ------------------------------------------------------------ closed forms
def _hand_inputs():
    ln = np.log
    q = np.array([[[ln(3.0), 0.0]], [[ln(2.0), ln(5.0)]]])
    k_tree = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v_tree = np.array([[[0.0, 1.0]], [[1.0, 1.0]]])
    return manual_inputs(q=q, k_prefix=[np.array([[[0.0, 0.0]]])],
                         v_prefix=[np.array([[[1.0, 0.0]]])], k_tree=k_tree,
                         v_tree=v_tree, trees=[[-1, 0]], scale=1.0)


def test_hand_example():
    want = read_hand_example()
    inp = _hand_inputs()
    o, lse, _ = oracle.verify(inp)
    po, pl = oracle.prefix_only(inp)
    so, sl = oracle.suffix_only(inp)
    for piece, (oo, ll) in {"verify": (o, lse), "prefix": (po, pl), "suffix": (so, sl)}.items():
        for node, (w0, w1, wl) in want[piece].items():
            # inputs are fp32 roundings of ln 2, ln 3, ln 5: error ~1e-7
            np.testing.assert_allclose(oo[node, 0], [w0, w1], atol=2e-7, err_msg=piece)
            np.testing.assert_allclose(ll[node, 0], wl, atol=2e-7, err_msg=piece)


def test_single_node_empty_prefix():
    # T = 1 and P = 0: the only visible key is the root itself, so o = v_root
    # exactly and lse = scale * q.k_root.
    rng = np.random.default_rng(3)
    inp = make_inputs(dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=8,
                      prefix_lens=[0], trees=[[-1]], rng=rng)
    o, lse, _ = oracle.verify(inp)
    G = 2
    for h in range(4):
        g = h // G
        np.testing.assert_array_equal(o[0, h], f64(inp.v_tree[0, g], "f32"))
        want = inp.softmax_scale * float(f64(inp.q[0, h], "f32") @ f64(inp.k_tree[0, g], "f32"))
        assert abs(lse[0, h] - want) < 1e-12


def test_identical_keys_give_mean_of_values():
    # all keys equal -> all scores equal -> o is the plain mean over visible values
    rng = np.random.default_rng(4)
    P, D = 37, 8
    k = rng.standard_normal(D)
    kp = np.tile(k, (P, 1, 1))
    vp = rng.standard_normal((P, 1, D))
    tree = [-1, 0, 1, 0]
    kt = np.tile(k, (4, 1, 1))
    vt = rng.standard_normal((4, 1, D))
    q = rng.standard_normal((4, 1, D))
    inp = manual_inputs(q=q, k_prefix=[kp], v_prefix=[vp], k_tree=kt, v_tree=vt,
                        trees=[tree], scale=0.3)
    o, lse, _ = oracle.verify(inp)
    kp32, vp32 = f64(inp.k_prefix_logical[0], "f32"), f64(inp.v_prefix_logical[0], "f32")
    vt32 = f64(inp.v_tree, "f32")
    anc = {0: [0], 1: [0, 1], 2: [0, 1, 2], 3: [0, 3]}
    for i, a in anc.items():
        vis = np.concatenate([vp32[:, 0], vt32[a, 0]], axis=0)
        np.testing.assert_allclose(o[i, 0], vis.mean(axis=0), atol=1e-12)
        s = 0.3 * float(f64(inp.q[i, 0], "f32") @ kp32[0, 0])
        np.testing.assert_allclose(lse[i, 0], s + np.log(P + len(a)), atol=1e-12)


def test_merge_closed_forms():
    rng = np.random.default_rng(5)
    oa, ob = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    la = np.array([0.5, -np.inf, 2.0])
    lb = np.array([-np.inf, -1.0, 2.0])
    o, l = oracle.merge(oa, la, ob, lb)
    np.testing.assert_array_equal(o[0], oa[0])        # empty b -> a exactly
    assert l[0] == 0.5
    np.testing.assert_array_equal(o[1], ob[1])        # empty a -> b exactly
    assert l[1] == -1.0
    np.testing.assert_allclose(o[2], 0.5 * (oa[2] + ob[2]), atol=1e-15)  # equal weights
    np.testing.assert_allclose(l[2], 2.0 + np.log(2.0), atol=1e-15)
    o, l = oracle.merge(oa[:1], np.array([-np.inf]), ob[:1], np.array([-np.inf]))
    assert np.all(o == 0) and l[0] == -np.inf


# ------------------------------------------------ library routine (SDPA)
def sdpa_reference(inp):
    """Independent reference: torch SDPA (fp64, CPU) on the logically contiguous
    sequence [prefix ; tree] with an explicit boolean mask built from dp_masks,
    KV heads expanded with repeat_interleave (head h reads KV head h // G).
    lse from torch.logsumexp of the masked scaled scores."""
    G = inp.num_q_heads // inp.num_kv_heads
    N, Hq, D = inp.total_tree_nodes, inp.num_q_heads, inp.head_dim
    o = np.zeros((N, Hq, D))
    lse = np.zeros((N, Hq))
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        T, P = hi - lo, int(inp.prefix_lens[b])
        if T == 0:
            continue
        kp = f64(inp.k_prefix_logical[b], inp.dtype)
        vp = f64(inp.v_prefix_logical[b], inp.dtype)
        kt = f64(inp.k_tree[lo:hi], inp.dtype)
        vt = f64(inp.v_tree[lo:hi], inp.dtype)
        K = torch.from_numpy(np.concatenate([kp, kt], 0)).permute(1, 0, 2)   # [Hkv, L, D]
        V = torch.from_numpy(np.concatenate([vp, vt], 0)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        Q = torch.from_numpy(f64(inp.q[lo:hi], inp.dtype)).permute(1, 0, 2).contiguous()
        words = dp_masks([int(x) for x in inp.parents[lo:hi]])
        mask = torch.zeros(T, P + T, dtype=torch.bool)
        mask[:, :P] = True
        for i in range(T):
            for j in range(T):
                mask[i, P + j] = bool(words[i] >> j & 1)
        out = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=mask[None, None],
            scale=inp.softmax_scale)[0]
        s = inp.softmax_scale * (Q @ K.transpose(1, 2))
        s = s.masked_fill(~mask[None], float("-inf"))
        o[lo:hi] = out.permute(1, 0, 2).numpy()
        lse[lo:hi] = torch.logsumexp(s, dim=-1).permute(1, 0).numpy()
    return o, lse


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_vs_sdpa_random(seed, dtype):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    lens = [int(rng.integers(0, 200)) for _ in range(B)]
    trees = [random_tree(rng, int(rng.integers(1, 10)), forest_p=0.1) for _ in range(B)]
    inp = small_inputs(seed, dtype=dtype, B=B, Hq=Hkv * G, Hkv=Hkv, D=16,
                       prefix_lens=lens, trees=trees)
    o, lse, _ = oracle.verify(inp)
    ro, rl = sdpa_reference(inp)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


@pytest.mark.parametrize("idx", [1, 4])
def test_oracle_vs_sdpa_configs(idx):
    inp = make_config(idx, keep_logical=True)
    o, lse, _ = oracle.verify(inp)
    ro, rl = sdpa_reference(inp)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-11)


def test_chain_equals_causal_attention():
    # A chain tree makes tree query k see the whole prefix plus chain[0..k]: plain
    # causal attention over [prefix ; chain] whose last T queries are the chain
    # (bottom-right aligned).  Reference: SDPA with that triangular mask.
    for seed in range(3):
        rng = np.random.default_rng(200 + seed)
        P, T, D, Hq, Hkv = int(rng.integers(1, 150)), 4, 16, 6, 2
        inp = small_inputs(seed, dtype="bf16", B=1, Hq=Hq, Hkv=Hkv, D=D,
                           prefix_lens=[P], trees=[TREE_CHAIN4])
        o, lse, _ = oracle.verify(inp)
        kp, vp = f64(inp.k_prefix_logical[0], "bf16"), f64(inp.v_prefix_logical[0], "bf16")
        K = torch.from_numpy(np.concatenate([kp, f64(inp.k_tree, "bf16")])).permute(1, 0, 2)
        V = torch.from_numpy(np.concatenate([vp, f64(inp.v_tree, "bf16")])).permute(1, 0, 2)
        K = K.repeat_interleave(Hq // Hkv, 0).contiguous()
        V = V.repeat_interleave(Hq // Hkv, 0).contiguous()
        Q = torch.from_numpy(f64(inp.q, "bf16")).permute(1, 0, 2).contiguous()
        causal = torch.ones(T, P + T, dtype=torch.bool).tril(diagonal=P)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=causal[None, None],
            scale=inp.softmax_scale)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12)


# ----------------------------------------------------------- invariants
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_split_merge_equals_unsplit(idx):
    # merge(prefix piece, tree piece) == attention over the union of the two
    # disjoint key sets (exact in real arithmetic).  Configs 3 and 5 use their
    # first draws at a reduced batch to keep the CPU suite short.
    inp = make_config(idx, batch_override={3: 6, 5: 12}.get(idx))
    o, lse, _ = oracle.verify(inp)
    po, pl = oracle.prefix_only(inp)
    so, sl = oracle.suffix_only(inp)
    mo, ml = oracle.merge(po, pl, so, sl)
    assert np.max(np.abs(mo - o)) <= 1e-12
    assert np.max(np.abs(ml - lse)) <= 1e-12


def test_split_merge_with_empty_prefix():
    inp = small_inputs(11, prefix_lens=(0, 0), B=2)
    o, lse, _ = oracle.verify(inp)
    so, sl = oracle.suffix_only(inp)
    po, pl = oracle.prefix_only(inp)
    assert np.all(pl == -np.inf) and np.all(po == 0)
    mo, ml = oracle.merge(po, pl, so, sl)
    np.testing.assert_array_equal(mo, so)
    np.testing.assert_array_equal(o, so)
    np.testing.assert_array_equal(lse, sl)


@pytest.mark.parametrize("seed", range(4))
def test_ancestor_only_dependence(seed):
    # Brute-force perturbation: change tree node j's key/value (or its query) and
    # check that outputs of nodes not below j are bit-identical, while every node
    # that has j as an ancestor-or-self changes.
    rng = np.random.default_rng(300 + seed)
    T = int(rng.integers(2, 9))
    tree = random_tree(rng, T)
    base = small_inputs(seed, dtype="bf16", B=1, Hq=4, Hkv=2, D=8,
                        prefix_lens=[int(rng.integers(0, 90))], trees=[tree])
    o0, l0, _ = oracle.verify(base)
    words = dp_masks(tree)
    for j in range(T):
        for which in ("kv", "q"):
            pert = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=8,
                               prefix_lens=[int(base.prefix_lens[0])], trees=[tree],
                               rng=np.random.default_rng(seed), seed=seed)
            # reuse base values, then overwrite node j
            for name in ("q", "k_cache", "v_cache", "k_tree", "v_tree", "block_table"):
                setattr(pert, name, getattr(base, name).copy())
            if which == "kv":
                pert.k_tree[j] = pert.k_tree[j] ^ np.uint16(0x0040)   # finite change
                pert.v_tree[j] = pert.v_tree[j] ^ np.uint16(0x0040)
            else:
                pert.q[j] = pert.q[j] ^ np.uint16(0x0040)
            o1, l1, _ = oracle.verify(pert)
            for i in range(T):
                affected = (words[i] >> j & 1) if which == "kv" else (i == j)
                if affected:
                    assert not np.array_equal(o1[i], o0[i]), (tree, i, j, which)
                else:
                    np.testing.assert_array_equal(o1[i], o0[i])
                    np.testing.assert_array_equal(l1[i], l0[i])


def test_score_shift_moves_lse_only():
    # Give every key (prefix and tree) last feature 1.  Setting every query's
    # last feature to c instead of 0 moves every score by scale*c, so o is
    # unchanged and lse moves by scale*c.
    c = 0.75
    a = small_inputs(21, B=2, Hq=4, Hkv=2, D=8, prefix_lens=(90, 3))
    b = small_inputs(21, B=2, Hq=4, Hkv=2, D=8, prefix_lens=(90, 3))
    for inp in (a, b):
        inp.k_cache[..., -1] = 1.0
        inp.k_tree[..., -1] = 1.0
    a.q[..., -1] = 0.0
    b.q[..., -1] = c
    o0, l0, _ = oracle.verify(a)
    o1, l1, _ = oracle.verify(b)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + a.softmax_scale * c, atol=1e-12)


def test_gqa_equals_replicated_heads():
    # Grouped heads == the same computation with KV replicated to every q head.
    g = small_inputs(31, dtype="bf16", B=2, Hq=6, Hkv=2, D=8, prefix_lens=(65, 130))
    r = small_inputs(31, dtype="bf16", B=2, Hq=6, Hkv=2, D=8, prefix_lens=(65, 130))
    r.num_kv_heads = 6
    r.k_cache = np.repeat(g.k_cache, 3, axis=1)
    r.v_cache = np.repeat(g.v_cache, 3, axis=1)
    r.k_tree = np.repeat(g.k_tree, 3, axis=1)
    r.v_tree = np.repeat(g.v_tree, 3, axis=1)
    og, lg, _ = oracle.verify(g)
    orr, lr, _ = oracle.verify(r)
    np.testing.assert_array_equal(og, orr)
    np.testing.assert_array_equal(lg, lr)


def test_output_is_convex_combination():
    inp = make_config(1)
    o, _, _ = oracle.verify(inp)
    V = np.concatenate([f64(inp.v_cache[:2, 0].reshape(-1, 64), "f32"),
                        f64(inp.v_tree[:, 0], "f32")])
    assert np.all(o <= V.max(axis=0) + 1e-12) and np.all(o >= V.min(axis=0) - 1e-12)


def test_paging_invariance():
    # Moving blocks around the pool (and updating the table) changes nothing.
    inp = small_inputs(41, dtype="bf16", B=3, Hq=4, Hkv=2, D=8,
                       prefix_lens=(200, 64, 129), spare_blocks=5)
    o0, l0, _ = oracle.verify(inp)
    rng = np.random.default_rng(9)
    perm = rng.permutation(inp.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    inp.k_cache = inp.k_cache[perm]
    inp.v_cache = inp.v_cache[perm]
    tab = inp.block_table.copy()
    tab[tab >= 0] = inv[tab[tab >= 0]]
    inp.block_table = tab
    o1, l1, _ = oracle.verify(inp)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_poisoned_slots_never_read():
    inp = make_config(3, batch_override=4)
    o, lse, _ = oracle.verify(inp)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_verify_rows_matches_verify():
    inp = make_config(5, batch_override=6)
    o, lse, _ = oracle.verify(inp)
    rows = [(0, 0), (inp.total_tree_nodes - 1, 31), (3, 17)]
    ro, rl = oracle.verify_rows(inp, rows)
    for k, (n, h) in enumerate(rows):
        np.testing.assert_allclose(ro[k], o[n, h], atol=1e-13)
        np.testing.assert_allclose(rl[k], lse[n, h], atol=1e-13)


def test_tree12_config_structure():
    # the 12-node tree has 33 ancestor-or-self pairs (sum of depths + 12)
    assert sum(bin(w).count("1") for w in dp_masks(TREE_12)) == 33
