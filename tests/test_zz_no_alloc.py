"""GPU test of tree_attn_verify_noalloc, called through the C ABI: its output
equals tree_attn_verify's on the same inputs (same kernels, same chunking:
bit for bit) and the oracle's within the bf16 tolerances, on two calls in a
row (the second smaller), with a device error reported through its status
word and cleared for the next call."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, assert_close_lse, host, run_verify, say, to_device, tolerances
from helpers import small_inputs
from workloads import TREE_12, make_config

pytestmark = pytest.mark.gpu


def _noalloc(d, out, lse, status):
    from tree_attention_verify_attn_amd._lib import load
    lib = load()
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.tree_attn_verify_noalloc(
        ctypes.byref(d.shape), d.q.data_ptr(), d.k_cache.data_ptr(), d.v_cache.data_ptr(),
        d.block_table.data_ptr(), d.prefix_lens.data_ptr(), d.k_tree.data_ptr(),
        d.v_tree.data_ptr(), d.parents.data_ptr(), d.tree_offsets.data_ptr(), out.data_ptr(),
        lse.data_ptr(), None if status is None else status.data_ptr(), sh)


def _check_against_verify(inp, d, what):
    import tree_attention_verify_attn_amd as ta
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full(d.q.shape[:2], float("nan"), device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    say(f"noalloc {what}: {ta.launch_info(d.shape)}")
    assert _noalloc(d, out, lse, status) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref_o, ref_l = run_verify(d)
    assert ta.get_error(d.workspace) == 0
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), what
    o_want, l_want, _ = oracle.verify(inp)
    tol_o, tol_l = tolerances(inp)
    assert_close(host(out), o_want, tol_o, f"noalloc {what} o")
    assert_close_lse(host(lse), l_want, tol_l, f"noalloc {what} lse")


def test_noalloc_matches_verify_two_calls():
    big = make_config(2)            # one sequence, 8192-token prefix, 26 chunks per group
    small = small_inputs(500, dtype="bf16", B=3, Hq=8, Hkv=2, D=128,
                         prefix_lens=(700, 64, 1500), trees=[TREE_12, [-1, 0, 1], [-1]])
    _check_against_verify(big, to_device(big), "8k verify")
    _check_against_verify(small, to_device(small), "smaller batch after it")


def test_noalloc_ticket_mode_and_fp32():
    lens = np.random.default_rng(501).integers(300, 3000, 40)
    many = small_inputs(501, dtype="bf16", B=40, Hq=8, Hkv=2, D=128,
                        prefix_lens=tuple(int(x) for x in lens), trees=[[-1, 0, 0]] * 40)
    _check_against_verify(many, to_device(many, split_tokens=128), "ticket mode")
    f32 = small_inputs(502, dtype="f32", B=2, Hq=4, Hkv=1, D=64, prefix_lens=(900, 30))
    _check_against_verify(f32, to_device(f32), "fp32")


def test_noalloc_device_error_reported_then_cleared():
    inp = small_inputs(503, dtype="bf16", B=2, Hq=4, Hkv=2, D=128, prefix_lens=(2000, 300))
    d = to_device(inp, max_prefix_len=2000)
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    d.prefix_lens[1] = 2001                      # beyond the declared bound
    say("noalloc: prefix length beyond the bound")
    assert _noalloc(d, out, lse, status) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 6               # TA_ERR_BAD_PREFIX
    d.prefix_lens[1] = int(inp.prefix_lens[1])
    say("noalloc: clean call after the error")
    _check_against_verify(inp, d, "after an error")
    # no status word: the call still runs and clears nothing it should keep
    say("noalloc: no status word")
    assert _noalloc(d, out, lse, None) == 0
    torch.cuda.synchronize()
    ref_o, _ = run_verify(d)
    assert torch.equal(out, ref_o)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import tree_attention_verify_attn_amd as ta
    from tree_attention_verify_attn_amd._lib import load
    # the batch-256 ragged shape needs far more partial slots than 32 MiB
    s = ta.make_shape(batch=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      max_blocks_per_seq=512, max_tree_nodes=12, max_prefix_len=32768,
                      total_tree_nodes=1536, num_blocks=14000, dtype=ta.DTYPE_BF16)
    assert ta.workspace_size(s) > 32 << 20
    fake = 0x100000
    rc = load().tree_attn_verify_noalloc(ctypes.byref(s), *([fake] * 11), None, None)
    assert rc == 9                               # TA_ERR_SCRATCH, nothing launched
