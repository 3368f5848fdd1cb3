"""Helpers for the GPU parity tests: move generated inputs to the device and call
the HIP library through its binding."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import tree_attention_verify_attn_amd as ta
from workloads import TreeVerifyInputs

BF16_TOL_O = 2e-2     # max |o - o*| for bf16 inputs
BF16_TOL_LSE = 1e-3   # max |lse - lse*| for bf16 inputs
F32_TOL_O = 1e-5      # max |o - o*| for fp32 inputs
F32_TOL_LSE = 1e-5


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says which it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@dataclass
class DeviceInputs:
    shape: object
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    prefix_lens: torch.Tensor
    k_tree: torch.Tensor
    v_tree: torch.Tensor
    parents: torch.Tensor
    tree_offsets: torch.Tensor
    workspace: torch.Tensor


def _dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_device(inp: TreeVerifyInputs, *, split_tokens: int = 0, max_prefix_len=None,
              max_tree_nodes=None, device="cuda") -> DeviceInputs:
    shape = ta.make_shape(
        batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
        head_dim=inp.head_dim, max_blocks_per_seq=inp.max_blocks_per_seq,
        max_tree_nodes=max_tree_nodes or max(1, inp.max_tree_nodes),
        max_prefix_len=inp.max_prefix_len if max_prefix_len is None else max_prefix_len,
        total_tree_nodes=inp.total_tree_nodes, num_blocks=inp.num_blocks,
        dtype=ta.DTYPE_BF16 if inp.dtype == "bf16" else ta.DTYPE_F32,
        softmax_scale=inp.softmax_scale, split_tokens=split_tokens)
    return DeviceInputs(
        shape=shape,
        q=_dev(inp.q, inp.dtype, device),
        k_cache=_dev(inp.k_cache, inp.dtype, device),
        v_cache=_dev(inp.v_cache, inp.dtype, device),
        block_table=_dev(inp.block_table, "i32", device),
        prefix_lens=_dev(inp.prefix_lens, "i32", device),
        k_tree=_dev(inp.k_tree, inp.dtype, device),
        v_tree=_dev(inp.v_tree, inp.dtype, device),
        parents=_dev(inp.parents, "i32", device),
        tree_offsets=_dev(inp.tree_offsets, "i32", device),
        workspace=ta.alloc_workspace(shape, device),
    )


def run_verify(d: DeviceInputs, **kw):
    out, lse = ta.verify(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                         d.k_tree, d.v_tree, d.parents, d.tree_offsets, d.workspace, **kw)
    torch.cuda.synchronize()
    return out, lse


def run_split(d: DeviceInputs):
    """prefix pass + mask + suffix pass + merge as four library calls."""
    mask = ta.build_mask(d.shape, d.parents, d.tree_offsets, d.workspace)
    po, pl = ta.prefix(d.shape, d.q, d.k_cache, d.v_cache, d.block_table, d.prefix_lens,
                       d.tree_offsets, d.workspace)
    so, sl = ta.suffix(d.shape, d.q, d.k_tree, d.v_tree, mask, d.tree_offsets)
    out, lse = ta.merge(po, pl, so, sl, out_dtype=int(d.shape.dtype))
    torch.cuda.synchronize()
    return out, lse, (po, pl, so, sl, mask)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def tolerances(inp: TreeVerifyInputs):
    return (BF16_TOL_O, BF16_TOL_LSE) if inp.dtype == "bf16" else (F32_TOL_O, F32_TOL_LSE)


def assert_close_lse(got: np.ndarray, want: np.ndarray, tol: float, what: str) -> None:
    # -inf must match exactly; finite values within tol
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{what}: -inf pattern differs"
    fin = np.isfinite(want)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values"
    err = np.max(np.abs(got[fin] - want[fin])) if fin.any() else 0.0
    assert err <= tol, f"{what}: max |lse err| {err:.3g} > {tol}"


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str) -> float:
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"{what}: max |err| {err:.3g} > {tol}"
    return err
