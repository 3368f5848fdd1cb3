"""GPU tests of the verify call under HIP-graph capture, under concurrent
launches on two streams, and of the group meeting's leave path.

The chunks of a first-round group meet after writing their partials.  A
chunk waits there only when every chunk of its group has started; otherwise
it leaves and the last arrival combines its rows.  TREE_ATTN_TEST_FORCE_LEAVE
makes the odd chunks of every group leave (as they would if the launch did not
hold the whole GPU): the output must be bit-identical to the normal meeting.
Tolerances as in test_gpu_parity.py.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_lse, host, run_verify, say, to_device, tolerances
from helpers import small_inputs
from workloads import TREE_12, make_config, make_inputs

pytestmark = pytest.mark.gpu


def _check(inp, out, lse, what):
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, f"{what} o")
    assert_close_lse(host(lse), l_want, tol_l, f"{what} lse")


class _ForceLeave:
    def __enter__(self):
        os.environ["TREE_ATTN_TEST_FORCE_LEAVE"] = "1"

    def __exit__(self, *exc):
        os.environ.pop("TREE_ATTN_TEST_FORCE_LEAVE", None)


LEAVE_CASES = [
    # one sequence: bf16 at head dim 64 with a tree of more than 64 nodes is
    # the one-sequence shape that still meets in the launch (others take two
    # launches and have no meeting: the forced leave must change nothing)
    ("one-seq-d64-big", lambda: make_inputs(
        dtype="bf16", num_q_heads=2, num_kv_heads=2, head_dim=64, prefix_lens=[3000],
        trees=[[-1] + [i // 3 for i in range(99)]], rng=np.random.default_rng(60), seed=60), 256),
    ("cfg2", lambda: make_config(2), 0),                       # two launches, 26 chunks a group
    ("cfg3", lambda: make_config(3), 0),                       # 32 sequences, device-chosen chunk
    ("d64-f32", lambda: small_inputs(120, dtype="f32", B=2, Hq=4, Hkv=2, D=64,
                                     prefix_lens=(2000, 700)), 128),
]


@pytest.mark.parametrize("name,make,split", LEAVE_CASES, ids=[c[0] for c in LEAVE_CASES])
def test_verify_leave_path_bit_identical(name, make, split):
    import tree_attention_verify_attn_amd as ta
    inp = make()
    d = to_device(inp, split_tokens=split)
    info = ta.launch_info(d.shape)
    say(f"leave path {name}: {info}")
    out0, lse0 = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    with _ForceLeave():
        say(f"leave path {name}: odd chunks leave")
        out1, lse1 = run_verify(d)
        assert ta.get_error(d.workspace) == 0
        # and the prefix pass alone, through the same meeting
        po1, pl1 = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                             d.tree_offsets, d.workspace)
        torch.cuda.synchronize()
        assert ta.get_error(d.workspace) == 0
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    po0, pl0 = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                         d.tree_offsets, d.workspace)
    torch.cuda.synchronize()
    assert torch.equal(po0, po1) and torch.equal(pl0, pl1)
    _check(inp, out1, lse1, f"leave path {name}")
    # the counters were left ready: a normal call after the forced leaves
    out2, lse2 = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    assert torch.equal(out0, out2) and torch.equal(lse0, lse2)


def test_verify_two_streams_concurrent():
    """Two first-round verify calls on two streams, each with its own
    workspace, launched back to back several times: neither waits for
    chunks of a group that the other launch keeps off the GPU, and every
    result matches the oracle."""
    import tree_attention_verify_attn_amd as ta
    inps = [make_config(2), make_config(3), make_config(4)]
    devs = [to_device(x) for x in inps]
    for x, d in zip(inps, devs):
        say(f"two streams: {x.name} launch {ta.launch_info(d.shape)}")
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [(torch.empty_like(d.q), torch.empty(d.q.shape[:2], dtype=torch.float32,
                                                device="cuda")) for d in devs]
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"two streams: round {rep}")
        for k in range(6):
            i = (k + rep) % len(devs)
            s = streams[k % 2]
            d = devs[i]
            with torch.cuda.stream(s):
                ta.verify(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                          d.k_tree, d.v_tree, d.parents, d.tree_offsets, d.workspace,
                          out=outs[i][0], lse=outs[i][1], stream=s)
        torch.cuda.synchronize()
        for x, d in zip(inps, devs):
            assert ta.get_error(d.workspace) == 0, x.name
    for x, d, (o, l) in zip(inps, devs, outs):
        _check(x, o, l, f"two streams {x.name}")


def _same_shape_inputs(seed):
    # two sequences of one shape; each seed draws new data, tables and trees
    return small_inputs(seed, dtype="bf16", B=2, Hq=8, Hkv=2, D=128,
                        prefix_lens=(3000, 1100), trees=[TREE_12, TREE_12])


_TICKET_LENS = tuple(int(x) for x in np.random.default_rng(209).integers(300, 2000, 40))


def _ticket_inputs(seed):
    # one shape for every seed (the lengths are fixed); the data, block
    # tables and pool placement change with the seed
    return small_inputs(seed, dtype="bf16", B=40, Hq=8, Hkv=2, D=128,
                        prefix_lens=_TICKET_LENS, trees=[[-1, 0, 1]] * 40)


def _copy_inputs(dst, src):
    for name in ("q", "k_cache", "v_cache", "block_table", "prefix_lens", "k_tree", "v_tree",
                 "parents", "tree_offsets"):
        getattr(dst, name).copy_(getattr(src, name))


def _one_seq_inputs(seed):
    # one sequence, 12 chunks a group: two launches (attention, then combine)
    return small_inputs(seed, dtype="bf16", B=1, Hq=8, Hkv=2, D=128, prefix_lens=(3000,),
                        trees=[TREE_12])


def test_verify_graph_capture_replay():
    """workspace_init and four verify calls (first-round, ticket mode, first-
    round again, and a one-sequence call in two launches, on one workspace)
    captured in a HIP graph and replayed with new inputs: every replay matches
    the oracle for its inputs, also with eager work between replays."""
    import tree_attention_verify_attn_amd as ta
    a0, t0, s0 = _same_shape_inputs(200), _ticket_inputs(210), _one_seq_inputs(220)
    da, dt, ds = to_device(a0), to_device(t0, split_tokens=128), to_device(s0, split_tokens=256)
    assert ta.launch_info(ds.shape)["mode"] == "two_launch"
    ws = torch.zeros(max(ta.workspace_size(d.shape) for d in (da, dt, ds)),
                     dtype=torch.uint8, device="cuda")
    da.workspace = dt.workspace = ds.workspace = ws
    oa1, la1 = torch.empty_like(da.q), torch.empty(da.q.shape[:2], device="cuda")
    oa2, la2 = torch.empty_like(da.q), torch.empty(da.q.shape[:2], device="cuda")
    ot, lt = torch.empty_like(dt.q), torch.empty(dt.q.shape[:2], device="cuda")
    os_, ls_ = torch.empty_like(ds.q), torch.empty(ds.q.shape[:2], device="cuda")

    def calls(stream):
        ta.workspace_init(ws, stream=stream)
        for d, o, l in ((da, oa1, la1), (dt, ot, lt), (da, oa2, la2), (ds, os_, ls_)):
            ta.verify(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                      d.k_tree, d.v_tree, d.parents, d.tree_offsets, ws, out=o, lse=l,
                      stream=stream)

    say("graph: eager warm-up")
    calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert ta.get_error(ws) == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g, stream=side):
        calls(side)
    torch.cuda.synchronize()
    for rep, (sa, st) in enumerate(((201, 211), (202, 212), (203, 213))):
        a, t, o1 = _same_shape_inputs(sa), _ticket_inputs(st), _one_seq_inputs(221 + rep)
        _copy_inputs(da, to_device(a))
        _copy_inputs(dt, to_device(t, split_tokens=128))
        _copy_inputs(ds, to_device(o1, split_tokens=256))
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert ta.get_error(ws) == 0
        _check(a, oa1, la1, f"replay {rep} first call")
        _check(t, ot, lt, f"replay {rep} ticket call")
        _check(o1, os_, ls_, f"replay {rep} two-launch call")
        assert torch.equal(oa1, oa2) and torch.equal(la1, la2)
        # eager work on the same workspace between replays
        oe, le = run_verify(dt)
        assert torch.equal(oe, ot) and torch.equal(le, lt)
