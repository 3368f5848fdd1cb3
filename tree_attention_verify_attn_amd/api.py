"""Python binding of libtreeattn.so: argument marshalling only.

Every function here checks tensor metadata, passes raw device pointers and the
current HIP stream to the C entry point of the same name, and raises on a
non-zero status.  No arithmetic of the method happens in Python; there is no
CPU or PyTorch fallback.  Entry points and their semantics are documented in
include/tree_attn.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import Shape, load

DTYPE_F32 = 0
DTYPE_BF16 = 1
_TORCH_DTYPE = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}


class TreeAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__(f"{where}: {status_string(code)} (status {code})")


def status_string(code: int) -> str:
    return load().tree_attn_status_string(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != 0:
        raise TreeAttnError(code, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _want(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_shape(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
               max_blocks_per_seq: int, max_tree_nodes: int, max_prefix_len: int,
               total_tree_nodes: int, num_blocks: int, dtype: int,
               softmax_scale: float = 0.0, split_tokens: int = 0,
               block_size: int = 64) -> Shape:
    return Shape(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, block_size=block_size,
                 max_blocks_per_seq=max_blocks_per_seq, max_tree_nodes=max_tree_nodes,
                 max_prefix_len=max_prefix_len, total_tree_nodes=total_tree_nodes,
                 num_blocks=num_blocks, split_tokens=split_tokens,
                 softmax_scale=softmax_scale, dtype=dtype)


def workspace_size(shape: Shape) -> int:
    return int(load().tree_attn_workspace_size(ctypes.byref(shape)))


def split_tokens(shape: Shape) -> int:
    return int(load().tree_attn_split_tokens(ctypes.byref(shape)))


def launch_info(shape: Shape) -> dict:
    """How tree_attn_verify would launch for `shape` (tree_attn_launch_info)."""
    info = (ctypes.c_int32 * 4)()
    _check(load().tree_attn_launch_info(ctypes.byref(shape), info), "tree_attn_launch_info")
    return {"split_tokens": info[0], "grid": info[1], "max_items": info[2],
            "mode": ("first_round", "ticket", "device", "two_launch")[info[3]]}


def alloc_workspace(shape: Shape, device="cuda", min_bytes: int = 256) -> torch.Tensor:
    """Zero-filled workspace (torch allocation; the library itself never allocates)."""
    n = max(workspace_size(shape), min_bytes)
    if n == 0:
        raise TreeAttnError(1, "alloc_workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(load().tree_attn_workspace_init(ws.data_ptr(), ws.numel(), _stream(stream)),
           "tree_attn_workspace_init")


def _elem(shape: Shape) -> torch.dtype:
    return _TORCH_DTYPE[int(shape.dtype)]


def _mask_shape(shape: Shape):
    """[N] with one 64-bit word per node up to 64-node trees, else [N, W]."""
    W = (int(shape.max_tree_nodes) + 63) // 64
    return (shape.total_tree_nodes,) if W == 1 else (shape.total_tree_nodes, W)


def build_mask(shape: Shape, parents: torch.Tensor, tree_offsets: torch.Tensor,
               workspace: torch.Tensor, mask: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    N = shape.total_tree_nodes
    _want(parents, "parents", torch.int32, (N,))
    _want(tree_offsets, "tree_offsets", torch.int32, (shape.batch + 1,))
    mshape = _mask_shape(shape)
    if mask is None:
        mask = torch.empty(mshape, dtype=torch.int64, device=parents.device)
    _want(mask, "mask", torch.int64, mshape)
    _check(load().tree_attn_build_mask(ctypes.byref(shape), _ptr(parents), _ptr(tree_offsets),
                                       _ptr(mask), _ptr(workspace), workspace.numel(),
                                       _stream(stream)), "tree_attn_build_mask")
    return mask


def _check_prefix_inputs(shape, q, k_cache, v_cache, block_table, prefix_lens, tree_offsets):
    N, Hq, Hkv, D = (shape.total_tree_nodes, shape.num_q_heads, shape.num_kv_heads,
                     shape.head_dim)
    el = _elem(shape)
    _want(q, "q", el, (N, Hq, D))
    _want(k_cache, "k_cache", el, (shape.num_blocks, Hkv, shape.block_size, D))
    _want(v_cache, "v_cache", el, (shape.num_blocks, Hkv, shape.block_size, D))
    _want(block_table, "block_table", torch.int32, (shape.batch, shape.max_blocks_per_seq))
    _want(prefix_lens, "prefix_lens", torch.int32, (shape.batch,))
    _want(tree_offsets, "tree_offsets", torch.int32, (shape.batch + 1,))


def prefix(shape: Shape, q, k_cache, v_cache, block_table, prefix_lens, tree_offsets,
           workspace, o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    _check_prefix_inputs(shape, q, k_cache, v_cache, block_table, prefix_lens, tree_offsets)
    N, Hq, D = shape.total_tree_nodes, shape.num_q_heads, shape.head_dim
    if o is None:
        o = torch.empty(N, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(N, Hq, dtype=torch.float32, device=q.device)
    _want(o, "o_prefix", torch.float32, (N, Hq, D))
    _want(lse, "lse_prefix", torch.float32, (N, Hq))
    _check(load().tree_attn_prefix(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(prefix_lens), _ptr(tree_offsets),
                                   _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream(stream)), "tree_attn_prefix")
    return o, lse


def suffix(shape: Shape, q, k_tree, v_tree, mask, tree_offsets,
           o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    N, Hq, Hkv, D = (shape.total_tree_nodes, shape.num_q_heads, shape.num_kv_heads,
                     shape.head_dim)
    el = _elem(shape)
    _want(q, "q", el, (N, Hq, D))
    _want(k_tree, "k_tree", el, (N, Hkv, D))
    _want(v_tree, "v_tree", el, (N, Hkv, D))
    _want(mask, "mask", torch.int64, _mask_shape(shape))
    _want(tree_offsets, "tree_offsets", torch.int32, (shape.batch + 1,))
    if o is None:
        o = torch.empty(N, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(N, Hq, dtype=torch.float32, device=q.device)
    _want(o, "o_suffix", torch.float32, (N, Hq, D))
    _want(lse, "lse_suffix", torch.float32, (N, Hq))
    _check(load().tree_attn_suffix(ctypes.byref(shape), _ptr(q), _ptr(k_tree), _ptr(v_tree),
                                   _ptr(mask), _ptr(tree_offsets), _ptr(o), _ptr(lse),
                                   _stream(stream)), "tree_attn_suffix")
    return o, lse


def merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
          out_dtype: int = DTYPE_F32, out: Optional[torch.Tensor] = None,
          lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    D = o_a.shape[-1]
    rows = o_a.numel() // D
    _want(o_a, "o_a", torch.float32)
    _want(o_b, "o_b", torch.float32, tuple(o_a.shape))
    _want(lse_a, "lse_a", torch.float32, tuple(o_a.shape[:-1]))
    _want(lse_b, "lse_b", torch.float32, tuple(o_a.shape[:-1]))
    if out is None:
        out = torch.empty(o_a.shape, dtype=_TORCH_DTYPE[out_dtype], device=o_a.device)
    if lse is None:
        lse = torch.empty(o_a.shape[:-1], dtype=torch.float32, device=o_a.device)
    _want(out, "out", _TORCH_DTYPE[out_dtype], tuple(o_a.shape))
    _want(lse, "lse_out", torch.float32, tuple(o_a.shape[:-1]))
    _check(load().tree_attn_merge(rows, D, out_dtype, _ptr(o_a), _ptr(lse_a), _ptr(o_b),
                                  _ptr(lse_b), _ptr(out), _ptr(lse), _stream(stream)),
           "tree_attn_merge")
    return out, lse


def verify(shape: Shape, q, k_cache, v_cache, block_table, prefix_lens, k_tree, v_tree,
           parents, tree_offsets, workspace, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, want_lse: bool = True,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    _check_prefix_inputs(shape, q, k_cache, v_cache, block_table, prefix_lens, tree_offsets)
    N, Hq, Hkv, D = (shape.total_tree_nodes, shape.num_q_heads, shape.num_kv_heads,
                     shape.head_dim)
    el = _elem(shape)
    _want(k_tree, "k_tree", el, (N, Hkv, D))
    _want(v_tree, "v_tree", el, (N, Hkv, D))
    _want(parents, "parents", torch.int32, (N,))
    if out is None:
        out = torch.empty(N, Hq, D, dtype=el, device=q.device)
    _want(out, "out", el, (N, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty(N, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _want(lse, "lse_out", torch.float32, (N, Hq))
    _check(load().tree_attn_verify(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(prefix_lens), _ptr(k_tree),
                                   _ptr(v_tree), _ptr(parents), _ptr(tree_offsets), _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream(stream)), "tree_attn_verify")
    return out, lse


def verify_incache(shape: Shape, q, k_cache, v_cache, block_table, prefix_lens, parents,
                   tree_offsets, workspace, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused verify with the tree K/V rows in the paged cache right after each
    prefix (tree_attn_verify_incache)."""
    _check_prefix_inputs(shape, q, k_cache, v_cache, block_table, prefix_lens, tree_offsets)
    N, Hq, D = shape.total_tree_nodes, shape.num_q_heads, shape.head_dim
    el = _elem(shape)
    _want(parents, "parents", torch.int32, (N,))
    if out is None:
        out = torch.empty(N, Hq, D, dtype=el, device=q.device)
    _want(out, "out", el, (N, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty(N, Hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _want(lse, "lse_out", torch.float32, (N, Hq))
    _check(load().tree_attn_verify_incache(ctypes.byref(shape), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(block_table), _ptr(prefix_lens),
                                           _ptr(parents), _ptr(tree_offsets), _ptr(out), _ptr(lse),
                                           _ptr(workspace), workspace.numel(), _stream(stream)),
           "tree_attn_verify_incache")
    return out, lse


def commit_incache(shape: Shape, parents, tree_offsets, accept_len, accept_path, k_cache,
                   v_cache, block_table, prefix_lens, workspace, stream=None) -> None:
    """Compact the accepted paths in place in the in-cache layout and advance
    prefix_lens (tree_attn_commit_incache)."""
    N, B, Hkv, D = (shape.total_tree_nodes, shape.batch, shape.num_kv_heads, shape.head_dim)
    el = _elem(shape)
    _want(parents, "parents", torch.int32, (N,))
    _want(tree_offsets, "tree_offsets", torch.int32, (B + 1,))
    _want(accept_len, "accept_len", torch.int32, (B,))
    _want(accept_path, "accept_path", torch.int32, (B, shape.max_tree_nodes))
    _want(k_cache, "k_cache", el, (shape.num_blocks, Hkv, 64, D))
    _want(v_cache, "v_cache", el, (shape.num_blocks, Hkv, 64, D))
    _want(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _want(prefix_lens, "prefix_lens", torch.int32, (B,))
    _check(load().tree_attn_commit_incache(ctypes.byref(shape), _ptr(parents), _ptr(tree_offsets),
                                           _ptr(accept_len), _ptr(accept_path), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(block_table), _ptr(prefix_lens),
                                           _ptr(workspace), workspace.numel(), _stream(stream)),
           "tree_attn_commit_incache")


def accept_greedy(shape: Shape, parents, tree_offsets, draft_tokens, target_argmax, workspace,
                  stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Greedy path acceptance (tree_attn_accept_greedy): returns accept_len [B],
    accept_path [B, max_tree_nodes] and bonus_token [B], all int32."""
    N, B, Tm = shape.total_tree_nodes, shape.batch, shape.max_tree_nodes
    _want(parents, "parents", torch.int32, (N,))
    _want(tree_offsets, "tree_offsets", torch.int32, (B + 1,))
    _want(draft_tokens, "draft_tokens", torch.int32, (N,))
    _want(target_argmax, "target_argmax", torch.int32, (N,))
    dev = parents.device
    n = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(B, Tm, dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    _check(load().tree_attn_accept_greedy(ctypes.byref(shape), _ptr(parents), _ptr(tree_offsets),
                                          _ptr(draft_tokens), _ptr(target_argmax), _ptr(n),
                                          _ptr(path), _ptr(bonus), _ptr(workspace),
                                          workspace.numel(), _stream(stream)),
           "tree_attn_accept_greedy")
    return n, path, bonus


def commit(shape: Shape, k_tree, v_tree, parents, tree_offsets, accept_len, accept_path,
           k_cache, v_cache, block_table, prefix_lens, free_blocks, free_count: int, workspace,
           blocks_taken: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """Commit accepted paths into the paged cache in place (tree_attn_commit).
    Updates k_cache, v_cache, block_table and prefix_lens; returns blocks_taken
    (int32 [1]) when given."""
    N, B, Hkv, D = (shape.total_tree_nodes, shape.batch, shape.num_kv_heads, shape.head_dim)
    el = _elem(shape)
    _want(k_tree, "k_tree", el, (N, Hkv, D))
    _want(v_tree, "v_tree", el, (N, Hkv, D))
    _want(parents, "parents", torch.int32, (N,))
    _want(tree_offsets, "tree_offsets", torch.int32, (B + 1,))
    _want(accept_len, "accept_len", torch.int32, (B,))
    _want(accept_path, "accept_path", torch.int32, (B, shape.max_tree_nodes))
    _want(k_cache, "k_cache", el, (shape.num_blocks, Hkv, 64, D))
    _want(v_cache, "v_cache", el, (shape.num_blocks, Hkv, 64, D))
    _want(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _want(prefix_lens, "prefix_lens", torch.int32, (B,))
    if free_count > 0:
        _want(free_blocks, "free_blocks", torch.int32)
        if free_blocks.numel() < free_count:
            raise ValueError("free_blocks holds fewer than free_count entries")
    if blocks_taken is not None:
        _want(blocks_taken, "blocks_taken", torch.int32, (1,))
    _check(load().tree_attn_commit(ctypes.byref(shape), _ptr(k_tree), _ptr(v_tree), _ptr(parents),
                                   _ptr(tree_offsets), _ptr(accept_len), _ptr(accept_path),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                   _ptr(prefix_lens), _ptr(free_blocks) if free_count > 0 else None,
                                   int(free_count), _ptr(blocks_taken), _ptr(workspace),
                                   workspace.numel(), _stream(stream)), "tree_attn_commit")
    return blocks_taken


def get_error(workspace: torch.Tensor, stream=None) -> int:
    """Synchronise the stream, read and clear the device-side error flag."""
    return int(load().tree_attn_get_error(_ptr(workspace), _stream(stream)))
