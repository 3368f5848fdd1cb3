"""GPU parity: every entry point of the HIP library against the fp64 oracle.

Tolerances (from the numerics of the path): fp32 inputs max |o err| 1e-5; bf16
inputs max |o err| 2e-2 and max |lse err| 1e-3; mask words bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_close, assert_close_lse, host, run_split, run_verify, say,
                      to_device, tolerances)
from helpers import random_tree, read_mask_table, small_inputs
from workloads import TREE_12, make_config, make_inputs

pytestmark = pytest.mark.gpu


def _check_verify(inp, out, lse, what):
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    err = assert_close(host(out), o_want, tol_o, f"{what} o")
    assert_close_lse(host(lse), l_want, tol_l, f"{what} lse")
    return err


# ------------------------------------------------------------------ mask
def test_mask_golden_tables_bit_exact():
    import tree_attention_verify_attn_amd as ta
    table = read_mask_table()
    trees = [par for _, par, _ in table]
    inp = small_inputs(1, B=len(trees), D=64, trees=trees, prefix_lens=[1] * len(trees))
    d = to_device(inp)
    say("mask golden tables")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    got = mask.cpu().numpy().view(np.uint64)
    want = np.concatenate([np.array(w, dtype=np.uint64) for _, _, w in table])
    np.testing.assert_array_equal(got, want)
    assert ta.get_error(d.workspace) == 0


@pytest.mark.parametrize("seed", range(3))
def test_mask_random_trees_bit_exact(seed):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(50 + seed)
    trees = [random_tree(rng, int(rng.integers(1, 65)), forest_p=0.05) for _ in range(40)]
    trees.append([-1] + list(range(63)))  # 64-node chain
    inp = small_inputs(seed, B=len(trees), D=64, trees=trees, prefix_lens=[0] * len(trees))
    d = to_device(inp)
    say(f"mask random trees seed {seed}")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint64), oracle.build_masks(inp))


def test_mask_flags_bad_parents():
    import tree_attention_verify_attn_amd as ta
    trees = [[-1, 0, 1], [-1, 2, 0], [-1, 0]]   # the middle tree has a forward parent
    inp = small_inputs(2, B=3, D=64, trees=trees, prefix_lens=[0, 0, 0])
    d = to_device(inp)
    say("mask bad parents")
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 3          # TA_ERR_BAD_TREE
    got = mask.cpu().numpy().view(np.uint64)
    np.testing.assert_array_equal(got[:3], oracle.ancestor_or_self_mask([-1, 0, 1]))
    np.testing.assert_array_equal(got[3:6], 0)     # bad tree -> zero words
    np.testing.assert_array_equal(got[6:], oracle.ancestor_or_self_mask([-1, 0]))
    assert ta.get_error(d.workspace) == 0          # flag cleared by the read


# ----------------------------------------------------------------- merge
@pytest.mark.parametrize("out_dtype", [0, 1])
def test_merge_vs_oracle(out_dtype):
    import tree_attention_verify_attn_amd as ta
    rng = np.random.default_rng(60)
    rows, D = 777, 128
    oa, ob = rng.standard_normal((rows, D)), rng.standard_normal((rows, D))
    la, lb = rng.standard_normal(rows) * 5, rng.standard_normal(rows) * 5
    la[::7] = -np.inf
    lb[::11] = -np.inf
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")
    say(f"merge out_dtype {out_dtype}")
    out, lse = ta.merge(t(oa), t(la), t(ob), t(lb), out_dtype=out_dtype)
    torch.cuda.synchronize()
    # the oracle merges the fp32-rounded inputs
    r32 = lambda x: x.astype(np.float32).astype(np.float64)
    wo, wl = oracle.merge(r32(oa), r32(la), r32(ob), r32(lb))
    assert_close(host(out), wo, 1e-5 if out_dtype == 0 else 2e-2, "merge o")
    assert_close_lse(host(lse), wl, 1e-5, "merge lse")


# --------------------------------------------------------- prefix, suffix
PIECE_CASES = [
    ("cfg1", lambda: make_config(1)),
    ("cfg2", lambda: make_config(2)),
    ("cfg3", lambda: make_config(3)),
    ("cfg4", lambda: make_config(4)),
    ("cfg5-b24", lambda: make_config(5, batch_override=24)),
    ("small-f32", lambda: small_inputs(70, dtype="f32", B=3, Hq=6, Hkv=2, D=64,
                                       prefix_lens=(0, 200, 63))),
    ("small-bf16", lambda: small_inputs(71, dtype="bf16", B=3, Hq=8, Hkv=1, D=128,
                                        prefix_lens=(1, 129, 640))),
]


@pytest.mark.parametrize("name,make", PIECE_CASES, ids=[c[0] for c in PIECE_CASES])
def test_split_path_pieces(name, make):
    inp = make()
    d = to_device(inp)
    say(f"split path {name}")
    out, lse, (po, pl, so, sl, mask) = run_split(d)
    tol_o, tol_l = tolerances(inp)
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint64), oracle.build_masks(inp))
    wpo, wpl = oracle.prefix_only(inp)
    wso, wsl = oracle.suffix_only(inp)
    # partial outputs are fp32; their error budget is the same as the final one
    assert_close(host(po), wpo, tol_o, f"{name} prefix o")
    assert_close_lse(host(pl), wpl, tol_l, f"{name} prefix lse")
    assert_close(host(so), wso, tol_o, f"{name} suffix o")
    assert_close_lse(host(sl), wsl, tol_l, f"{name} suffix lse")
    _check_verify(inp, out, lse, f"{name} split")


# ----------------------------------------------------------------- verify
@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_verify_configs(idx):
    inp = make_config(idx)
    d = to_device(inp)
    say(f"verify cfg{idx} split_tokens={d.shape.split_tokens}")
    out, lse = run_verify(d)
    import tree_attention_verify_attn_amd as ta
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, f"cfg{idx}")


def test_verify_cfg5_full_size():
    """The ragged batch-256 workload at full size, in the benchmark's launch
    configuration (library chunking, items handed out by ticket, the last
    chunk of a group combining alone): every row and head against the oracle."""
    import tree_attention_verify_attn_amd as ta
    inp = make_config(5)
    d = to_device(inp)
    say(f"verify cfg5 full size, split_tokens {ta.split_tokens(d.shape)}")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, "cfg5 full size")


def _ticket_inputs(seed, *, B, lens, D=128, Hq=8, Hkv=2, trees=None):
    return small_inputs(seed, dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, D=D,
                        prefix_lens=tuple(int(x) for x in lens),
                        trees=trees or [TREE_12] * B)


# Many groups of many chunks: more items than workgroups, so items are handed
# out by ticket and the chunk that arrives last combines its group alone; with
# more than 4 chunks per group (2 at D = 64) that combine loads several chunk
# partials per lane and folds several rows per pass.
TICKET_CASES = [
    # 64-token chunks, 5..64 chunks per group
    ("split64-d128", lambda: _ticket_inputs(
        400, B=40, lens=np.random.default_rng(400).integers(321, 4097, 40)), 64),
    ("split64-d64", lambda: _ticket_inputs(
        401, B=40, D=64, lens=np.random.default_rng(401).integers(321, 4097, 40)), 64),
    # 300 sequences of mixed length, 1024-token chunks (1..6 chunks per group)
    ("300seq-split1024", lambda: _ticket_inputs(
        402, B=300, Hq=8, Hkv=1, trees=[[-1, 0, 1, 2]] * 300,
        lens=np.random.default_rng(402).integers(16, 6001, 300)), 1024),
]


@pytest.mark.parametrize("name,make,split", TICKET_CASES, ids=[c[0] for c in TICKET_CASES])
def test_verify_ticket_many_chunks(name, make, split):
    import tree_attention_verify_attn_amd as ta
    inp = make()
    d = to_device(inp, split_tokens=split)
    S = [max(1, -(-int(p) // split)) for p in inp.prefix_lens]
    say(f"verify ticket mode {name}: {sum(S) * inp.num_kv_heads} items, "
        f"chunks per group {min(S)}..{max(S)}")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, f"ticket {name}")
    # the same call again on the same workspace: the counters reset themselves
    out2, lse2 = run_verify(d)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def _one_seq(seed, *, dtype, Hq, Hkv, D, P, tree=None, extra_cols=0):
    rng = np.random.default_rng(seed)
    return make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       prefix_lens=[P], trees=[tree or TREE_12], rng=rng, seed=seed,
                       name=f"one-seq{seed}", permute_blocks=True, spare_blocks=3,
                       extra_table_cols=extra_cols)


# One sequence whose groups have several chunks, all in the first round: the
# attention kernel stores every chunk's partial and a second launch
# (combine_kernel) folds them.  One case per combine instantiation (output
# type, head dim), the largest chunk count at each head dim, two chunks, a
# tree of more than 64 nodes (the large-tree attention kernel, several row
# passes), and a prefix far shorter than max_prefix_len (chunks with no key
# at all).
TWO_LAUNCH_CASES = [
    ("bf16-d64-s12", lambda: _one_seq(500, dtype="bf16", Hq=8, Hkv=2, D=64, P=3000), 256, None),
    ("bf16-d128-s2", lambda: _one_seq(506, dtype="bf16", Hq=8, Hkv=2, D=128, P=1500), 1024, None),
    ("f32-d128-s40", lambda: _one_seq(501, dtype="f32", Hq=4, Hkv=1, D=128, P=5000), 128, None),
    ("f32-d64-s64", lambda: _one_seq(502, dtype="f32", Hq=6, Hkv=2, D=64, P=4096), 64, None),
    ("bf16-d128-s64", lambda: _one_seq(503, dtype="bf16", Hq=5, Hkv=1, D=128, P=8100), 128, None),
    ("bf16-200-node-tree", lambda: _one_seq(504, dtype="bf16", Hq=2, Hkv=1, D=128, P=2048,
                                            tree=[-1] + [i // 2 for i in range(199)]), 256, None),
    ("empty-chunks", lambda: _one_seq(505, dtype="bf16", Hq=8, Hkv=2, D=128, P=900,
                                      extra_cols=60), 256, 4096),
]


@pytest.mark.parametrize("name,make,split,max_p", TWO_LAUNCH_CASES,
                         ids=[c[0] for c in TWO_LAUNCH_CASES])
def test_verify_two_launch(name, make, split, max_p):
    import tree_attention_verify_attn_amd as ta
    inp = make()
    d = to_device(inp, split_tokens=split, max_prefix_len=max_p)
    info = ta.launch_info(d.shape)
    say(f"two-launch verify {name}: {info}")
    assert info["mode"] == "two_launch", info
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, f"two-launch {name}")
    # the prefix pass alone takes the same two launches (fp32 output)
    po, pl = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                       d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wpo, wpl = oracle.prefix_only(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(po), wpo, tol_o, f"two-launch {name} prefix o")
    assert_close_lse(host(pl), wpl, tol_l, f"two-launch {name} prefix lse")
    # and again on the same workspace: nothing to reset, the same result
    out2, lse2 = run_verify(d)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_verify_two_launch_prefix_shorter_than_before():
    """One workspace, one shape (max_prefix_len 4096, 16 chunks a group), the
    actual prefix length shrinking from call to call: the chunks past it store
    nothing, so the combine must not fold what earlier calls left in their
    slots; with one chunk left the attention kernel writes the rows itself and
    the combine must leave them; with none, every row is the tree alone."""
    import dataclasses

    import tree_attention_verify_attn_amd as ta
    base = _one_seq(507, dtype="bf16", Hq=8, Hkv=2, D=128, P=4000)
    d = to_device(base, split_tokens=256)
    assert ta.launch_info(d.shape)["mode"] == "two_launch"
    for P in (4000, 900, 4000, 200, 0, 3100):
        say(f"two-launch verify, prefix {P} of at most 4000")
        inp = dataclasses.replace(base, prefix_lens=np.array([P], dtype=np.int32))
        d.prefix_lens.fill_(P)
        out, lse = run_verify(d)
        assert ta.get_error(d.workspace) == 0
        _check_verify(inp, out, lse, f"two-launch prefix {P}")
        po, pl = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                           d.tree_offsets, d.workspace)
        torch.cuda.synchronize()
        wpo, wpl = oracle.prefix_only(inp)
        tol_o, tol_l = tolerances(inp)
        assert_close(host(po), wpo, tol_o, f"two-launch prefix pass {P} o")
        assert_close_lse(host(pl), wpl, tol_l, f"two-launch prefix pass {P} lse")


@pytest.mark.parametrize("split", [64, 128, 256, 1024, 2048, 4096])
def test_verify_split_sizes(split):
    inp = make_config(4)
    d = to_device(inp, split_tokens=split)
    say(f"verify cfg4 split_tokens={split}")
    out, lse = run_verify(d)
    _check_verify(inp, out, lse, f"cfg4 split {split}")


def _batch(seed, *, dtype, Hq, Hkv, D, lens, extra_cols=0, trees=None):
    rng = np.random.default_rng(seed)
    return make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       prefix_lens=list(lens), trees=trees or [TREE_12] * len(lens), rng=rng,
                       seed=seed, name=f"batch{seed}", permute_blocks=True, spare_blocks=3,
                       extra_table_cols=extra_cols)


# Short prefixes stream in one chunk per sequence (no exchange): one sequence
# up to 3 blocks, a batch whose max_prefix_len is up to 6 blocks, or 8 with
# 32 groups or more (the host's chunk), a batch whose longest actual prefix
# is that short (the kernel picks that chunk even when max_prefix_len would
# allow more), and the first lengths past each bound, which split again.
SHORT_CASES = [
    ("one-seq-150", lambda: _one_seq(520, dtype="bf16", Hq=8, Hkv=2, D=128, P=150), None,
     "first_round"),
    ("one-seq-192-f32-d64", lambda: _one_seq(521, dtype="f32", Hq=4, Hkv=1, D=64, P=192), None,
     "first_round"),
    ("one-seq-193", lambda: _one_seq(522, dtype="bf16", Hq=5, Hkv=1, D=128, P=193), None,
     "two_launch"),
    ("batch8-up-to-384", lambda: _batch(523, dtype="bf16", Hq=8, Hkv=2, D=128,
                                        lens=(384, 1, 0, 200, 321, 64, 65, 383), extra_cols=58),
     4096, "device"),
    ("batch4-host-chunk", lambda: _batch(526, dtype="bf16", Hq=32, Hkv=8, D=128,
                                         lens=(300, 5, 384, 0)), None, "first_round"),
    ("batch8-wide-8-blocks", lambda: _batch(527, dtype="bf16", Hq=32, Hkv=8, D=128,
                                            lens=(512, 449, 300, 0, 65, 500, 480, 1)),
     None, "first_round"),
    ("batch8-wide-kernel", lambda: _batch(528, dtype="bf16", Hq=32, Hkv=8, D=64,
                                          lens=(450, 10, 511, 200, 0, 64, 300, 129), extra_cols=56),
     4096, "device"),
    ("batch6-385", lambda: small_inputs(524, dtype="bf16", B=6, Hq=8, Hkv=1, D=128,
                                        prefix_lens=(385, 17, 130, 384, 0, 256),
                                        trees=[[-1, 0, 1, 2]] * 6), None, "device"),
    ("batch5-d64-f32", lambda: _batch(525, dtype="f32", Hq=4, Hkv=2, D=64,
                                      lens=(100, 300, 5, 64, 250), extra_cols=27), 2048, "device"),
]


@pytest.mark.parametrize("name,make,max_p,mode", SHORT_CASES, ids=[c[0] for c in SHORT_CASES])
def test_verify_short_prefixes_one_chunk(name, make, max_p, mode):
    import tree_attention_verify_attn_amd as ta
    inp = make()
    d = to_device(inp, max_prefix_len=max_p)
    info = ta.launch_info(d.shape)
    say(f"verify short prefixes {name}: {info}")
    assert info["mode"] == mode, info
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, f"short {name}")
    out2, lse2 = run_verify(d)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # the prefix pass alone makes the same chunk choice
    po, pl = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                       d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert ta.get_error(d.workspace) == 0
    wpo, wpl = oracle.prefix_only(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(po), wpo, tol_o, f"short {name} o_prefix")
    assert_close_lse(host(pl), wpl, tol_l, f"short {name} lse_prefix")


# The log-sum-exp output is optional (lse_out = NULL): every way a row's
# output is written -- by the one chunk of its group, by a chunk after the
# meeting in the launch, by the last arrival in ticket mode, by the combine
# kernel of a two-launch call -- must then write o alone, the same bits.
NO_LSE_CASES = [
    ("one-chunk", lambda: make_config(1), 0),
    ("two-launch", lambda: _one_seq(530, dtype="bf16", Hq=8, Hkv=2, D=128, P=1500), 256),
    ("meeting", lambda: small_inputs(531, dtype="bf16", B=6, Hq=8, Hkv=2, D=128,
                                     prefix_lens=(900, 64, 1500, 0, 700, 1200)), 256),
    ("ticket", lambda: _ticket_inputs(532, B=40, lens=np.random.default_rng(532).integers(321, 2049, 40)),
     64),
]


@pytest.mark.parametrize("name,make,split", NO_LSE_CASES, ids=[c[0] for c in NO_LSE_CASES])
def test_verify_without_lse_output(name, make, split):
    import tree_attention_verify_attn_amd as ta
    inp = make()
    d = to_device(inp, split_tokens=split)
    say(f"verify without lse {name}: {ta.launch_info(d.shape)}")
    out, lse = run_verify(d)
    out2, lse2 = run_verify(d, want_lse=False)
    assert lse2 is None and ta.get_error(d.workspace) == 0
    assert torch.equal(out, out2)
    _check_verify(inp, out2, lse, f"no lse {name}")


EDGE_CASES = [
    ("empty-prefix", lambda: small_inputs(80, dtype="bf16", B=3, Hq=4, Hkv=2, D=128,
                                          prefix_lens=(0, 0, 0))),
    ("mixed-empty", lambda: small_inputs(81, dtype="bf16", B=4, Hq=8, Hkv=2, D=128,
                                         prefix_lens=(0, 65, 1, 3000))),
    ("single-node", lambda: small_inputs(82, dtype="bf16", B=2, Hq=4, Hkv=4, D=128,
                                         prefix_lens=(100, 7), trees=[[-1], [-1]])),
    ("chain64-G1", lambda: small_inputs(83, dtype="bf16", B=1, Hq=2, Hkv=2, D=128,
                                        prefix_lens=(333,), trees=[[-1] + list(range(63))])),
    ("rows>64-G8", lambda: small_inputs(84, dtype="bf16", B=2, Hq=8, Hkv=1, D=128,
                                        prefix_lens=(513, 77), trees=[TREE_12, [-1, 0, 0]])),
    ("rows=512", lambda: small_inputs(85, dtype="bf16", B=1, Hq=8, Hkv=1, D=128,
                                      prefix_lens=(200,), trees=[[-1] + list(range(63))])),
    ("d64-bf16", lambda: small_inputs(86, dtype="bf16", B=2, Hq=4, Hkv=2, D=64,
                                      prefix_lens=(190, 64))),
    ("d128-f32", lambda: small_inputs(87, dtype="f32", B=2, Hq=4, Hkv=1, D=128,
                                      prefix_lens=(190, 1000))),
    ("forest", lambda: small_inputs(88, dtype="bf16", B=1, Hq=4, Hkv=1, D=128,
                                    prefix_lens=(90,), trees=[[-1, -1, 0, 1, -1]])),
    ("keys-x4", lambda: small_inputs(89, dtype="bf16", B=2, Hq=5, Hkv=1, D=128,
                                     prefix_lens=(700, 2), key_scale=4.0)),
]


@pytest.mark.parametrize("name,make", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_verify_edge_cases(name, make):
    inp = make()
    d = to_device(inp)
    say(f"verify edge {name}")
    out, lse = run_verify(d)
    import tree_attention_verify_attn_amd as ta
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, name)


def test_verify_workspace_reuse_and_determinism():
    import tree_attention_verify_attn_amd as ta
    inp = make_config(2)
    d = to_device(inp)
    say("verify cfg2 repeated calls")
    out1, lse1 = run_verify(d)
    out2, lse2 = run_verify(d)
    out3, lse3 = run_verify(d)
    assert torch.equal(out1, out2) and torch.equal(out2, out3)
    assert torch.equal(lse1, lse2) and torch.equal(lse2, lse3)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out3, lse3, "cfg2 third call")


def test_verify_shared_workspace_changing_inputs():
    """One workspace across calls whose data, batch, chunk counts and dtype
    change from call to call (and with a device error in between): every call
    combines its own chunk partials, never those a previous call left."""
    import tree_attention_verify_attn_amd as ta
    specs = [
        ("two-long", dict(B=2, prefix_lens=(3000, 1500))),
        ("two-long-new-data", dict(B=2, prefix_lens=(3000, 1500))),
        ("three-mixed", dict(B=3, prefix_lens=(4000, 200, 2500))),
        ("one-seq", dict(B=1, prefix_lens=(6000,))),
        ("f32", dict(B=2, prefix_lens=(2000, 900), dtype="f32")),
        ("two-long-again", dict(B=2, prefix_lens=(3000, 1500))),
        ("one-seq-new-data", dict(B=1, prefix_lens=(6000,))),
        # more groups than workgroups: items handed out by ticket
        ("tickets", dict(B=160, prefix_lens=tuple(100 + (37 * i) % 1400 for i in range(160)))),
        ("two-long-after-tickets", dict(B=2, prefix_lens=(3000, 1500))),
    ]
    cases = []
    for k, (name, kw) in enumerate(specs):
        kw = dict(kw)
        dtype = kw.pop("dtype", "bf16")
        inp = small_inputs(300 + k, dtype=dtype, Hq=8, Hkv=2, D=128,
                           trees=[TREE_12] * kw["B"], **kw)
        cases.append((name, inp, to_device(inp)))
    ws = max((c[2].workspace for c in cases), key=lambda t: t.numel())
    for name, inp, d in cases:
        d.workspace = ws
    for rep in range(2):
        for name, inp, d in cases:
            say(f"shared workspace: {name} pass {rep}")
            out, lse = run_verify(d)
            assert ta.get_error(ws) == 0, name
            _check_verify(inp, out, lse, f"shared workspace {name}")
        # a call that flags a bad prefix length, then clean calls again
        name, inp, d = cases[2]
        d.prefix_lens[1] = inp.max_prefix_len + 1
        say("shared workspace: bad prefix length")
        run_verify(d)
        assert ta.get_error(ws) == 6
        d.prefix_lens[1] = int(inp.prefix_lens[1])


def test_verify_block_permutation_bit_identical():
    inp = make_config(3, batch_override=8)
    d = to_device(inp)
    say("verify block permutation A")
    out_a, lse_a = run_verify(d)
    rng = np.random.default_rng(11)
    perm = rng.permutation(inp.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    inp.k_cache = np.ascontiguousarray(inp.k_cache[perm])
    inp.v_cache = np.ascontiguousarray(inp.v_cache[perm])
    tab = inp.block_table.copy()
    tab[tab >= 0] = inv[tab[tab >= 0]]
    inp.block_table = tab
    d2 = to_device(inp)
    say("verify block permutation B")
    out_b, lse_b = run_verify(d2)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)


def test_verify_ancestor_only_dependence():
    # perturb tree node j's key/value: rows of nodes without j on their root path
    # must be bit-identical, the others must change
    base = make_config(2)
    d = to_device(base)
    say("perturbation base")
    out0, _ = run_verify(d)
    o0 = out0.float().cpu().numpy()
    words = [int(w) for w in oracle.build_masks(base)]
    for j in (1, 4, 11):
        pert = make_config(2)
        pert.k_tree[j] ^= np.uint16(0x0040)
        pert.v_tree[j] ^= np.uint16(0x0040)
        dp = to_device(pert)
        say(f"perturbation node {j}")
        out1, _ = run_verify(dp)
        o1 = out1.float().cpu().numpy()
        for i in range(12):
            if words[i] >> j & 1:
                assert not np.array_equal(o0[i], o1[i]), (i, j)
            else:
                np.testing.assert_array_equal(o0[i], o1[i])


def test_verify_device_errors_flagged():
    import tree_attention_verify_attn_amd as ta
    inp = small_inputs(90, dtype="bf16", B=2, Hq=4, Hkv=2, D=128, prefix_lens=(300, 20))
    d = to_device(inp, max_prefix_len=300)
    # prefix length beyond the declared bound -> BAD_PREFIX, no out-of-bounds read
    d.prefix_lens[1] = 301
    say("device error: prefix beyond bound")
    run_verify(d)
    assert ta.get_error(d.workspace) == 6
    d.prefix_lens[1] = int(inp.prefix_lens[1])
    # block id out of range
    good = int(inp.block_table[0, 1])
    d.block_table[0, 1] = inp.num_blocks + 5
    say("device error: block id out of range")
    run_verify(d)
    assert ta.get_error(d.workspace) == 6
    d.block_table[0, 1] = good
    # bad parent array
    root1 = int(inp.tree_offsets[1])
    d.parents[root1] = 5
    say("device error: bad parent")
    run_verify(d)
    assert ta.get_error(d.workspace) == 3
    d.parents[root1] = -1
    # the same workspace still works for a clean call afterwards
    say("device error: clean call after errors")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, "after errors")


@pytest.mark.gpu
def test_verify_device_errors_flagged_single_sequence():
    """One-sequence launches read the prefix length inside each item; bad data
    is still flagged and never read out of bounds."""
    import tree_attention_verify_attn_amd as ta
    inp = small_inputs(91, dtype="bf16", B=1, Hq=8, Hkv=2, D=128, prefix_lens=(700,),
                       trees=[[-1, 0, 0, 1, 2]])
    d = to_device(inp, max_prefix_len=704, split_tokens=128)
    d.prefix_lens[0] = 705
    say("single-sequence device error: prefix beyond bound")
    run_verify(d)
    assert ta.get_error(d.workspace) == 6
    d.prefix_lens[0] = int(inp.prefix_lens[0])
    good = int(inp.block_table[0, 3])
    d.block_table[0, 3] = inp.num_blocks + 1
    say("single-sequence device error: block id out of range")
    run_verify(d)
    assert ta.get_error(d.workspace) == 6
    d.block_table[0, 3] = good
    d.parents[1] = 7
    say("single-sequence device error: bad parent")
    run_verify(d)
    assert ta.get_error(d.workspace) == 3
    d.parents[1] = int(inp.parents[1])
    d.tree_offsets[1] = int(inp.tree_offsets[1]) - 1
    say("single-sequence device error: bad tree offsets")
    run_verify(d)
    assert ta.get_error(d.workspace) == 3
    d.tree_offsets[1] = int(inp.tree_offsets[1])
    say("single-sequence device error: clean call after errors")
    out, lse = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    _check_verify(inp, out, lse, "single after errors")
