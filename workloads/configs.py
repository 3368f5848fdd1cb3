"""The five seeded synthetic tree-verify workloads and a general input builder.

Everything here is input preparation: random draws, rounding to the storage
dtype, and placement into a paged KV pool.  No attention arithmetic lives in
this module.

Recipe (the pages fix no seed, distribution or layout; these readings are the
plain ones the rest of the material supports):

* RNG: NumPy PCG64 ``default_rng(seed)``, seed = 1000 + config index.
* Draw order: prefix lengths -> trees -> block permutation -> q -> prefix K
  (logical order: sequence, block, head, slot, dim) -> prefix V -> tree K ->
  tree V.
* Values: i.i.d. N(0, 1) in fp32, multiplied by ``key_scale`` for keys, then
  rounded once to the storage dtype (bf16: round-to-nearest-even on the fp32
  bits).  Both the oracle and the GPU read those same stored bits.
* Paged pool: 64-token blocks, pool layout ``[num_blocks, H_kv, 64, D]``.  The
  logical blocks of all sequences are placed at the physical indices given by a
  seeded permutation of the pool.  Slots past a sequence's prefix length inside
  its last block hold NaN, spare pool blocks hold NaN, and unused block-table
  entries hold -1 (poison: a correct reader never touches them).
* Trees: a parent array per sequence with local indices, -1 for the root and
  parent[i] < i (topological order), packed back to back; ``tree_offsets``
  gives each sequence's start row.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BLOCK = 64

TREE_SINGLE = [-1]
TREE_CHAIN4 = [-1, 0, 1, 2]
TREE_12 = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 6]
TREE_CFG1 = [-1, 0, 0, 1]

CONFIG_NAMES = {
    1: "tiny-fp32: B=1 Hq=4 Hkv=1 D=64 prefix=128 contiguous, tree [-1,0,0,1]",
    2: "llama3.1-8b-verify: bf16 B=1 Hq=32 Hkv=8 D=128 prefix=8192 paged, 12-node tree",
    3: "70b-head-share: bf16 B=32 Hq=8 Hkv=1 D=128 prefix~U[1024,8192] paged, chain-4",
    4: "maverick-head-share: bf16 B=1 Hq=5 Hkv=1 D=128 prefix=8192 paged, 12-node tree, keys x2",
    5: "ragged-b256: bf16 B=256 Hq=32 Hkv=8 D=128 prefix lognormal(med 2048, sigma 1) "
       "clip[16,32768], trees {1,chain-4,12} p=.2/.5/.3",
    # beyond the five verify workloads: trees of more than 64 nodes (split path)
    6: "llama3.1-8b-verify-256-node-tree: bf16 B=1 Hq=32 Hkv=8 D=128 prefix=8192 paged, "
       "random 256-node tree",
    7: "draft-side-multi-round: bf16 B=8 Hq=32 Hkv=8 D=128 prefix U{16..100}, random 128-node trees",
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


@dataclass
class TreeVerifyInputs:
    """Host copy of one tree-verify batch, in the exact layout the C-ABI takes.

    Arrays with ``dtype == "bf16"`` hold raw bf16 bit patterns as uint16;
    ``"f32"`` arrays hold float32.
    """

    name: str
    seed: int
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    softmax_scale: float
    q: np.ndarray             # [N, Hq, D]
    k_cache: np.ndarray       # [num_blocks, Hkv, 64, D]
    v_cache: np.ndarray       # [num_blocks, Hkv, 64, D]
    block_table: np.ndarray   # int32 [B, max_blocks_per_seq], -1 = unused
    prefix_lens: np.ndarray   # int32 [B]
    k_tree: np.ndarray        # [N, Hkv, D]
    v_tree: np.ndarray        # [N, Hkv, D]
    parents: np.ndarray       # int32 [N], local indices
    tree_offsets: np.ndarray  # int32 [B + 1]
    block_size: int = BLOCK
    # optional logical (unpaged) prefix K/V per sequence, [P_b, Hkv, D] each
    k_prefix_logical: Optional[List[np.ndarray]] = field(default=None, repr=False)
    v_prefix_logical: Optional[List[np.ndarray]] = field(default=None, repr=False)

    @property
    def total_tree_nodes(self) -> int:
        return int(self.tree_offsets[-1])

    @property
    def tree_sizes(self) -> np.ndarray:
        return np.diff(self.tree_offsets).astype(np.int64)

    @property
    def max_tree_nodes(self) -> int:
        return int(self.tree_sizes.max()) if self.batch else 0

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max()) if self.batch else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def tree(self, b: int) -> np.ndarray:
        return self.parents[self.tree_offsets[b]:self.tree_offsets[b + 1]]


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(
    *,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    prefix_lens: Sequence[int],
    trees: Sequence[Sequence[int]],
    rng: np.random.Generator,
    seed: int = -1,
    name: str = "custom",
    softmax_scale: Optional[float] = None,
    key_scale: float = 1.0,
    permute_blocks: bool = True,
    spare_blocks: int = 0,
    extra_table_cols: int = 0,
    keep_logical: bool = False,
) -> TreeVerifyInputs:
    """Draw one batch.  ``prefix_lens`` and ``trees`` were already drawn by the caller."""
    B = len(prefix_lens)
    assert len(trees) == B
    Hq, Hkv, D = int(num_q_heads), int(num_kv_heads), int(head_dim)
    P = np.asarray(prefix_lens, dtype=np.int64)
    nblk = (P + BLOCK - 1) // BLOCK
    n_logical = int(nblk.sum())
    num_blocks = n_logical + int(spare_blocks)
    max_blocks = int(nblk.max()) if B else 0
    max_blocks += int(extra_table_cols)
    max_blocks = max(max_blocks, 1)

    # block permutation (drawn before any value)
    if permute_blocks:
        phys = rng.permutation(num_blocks)[:n_logical]
    else:
        phys = np.arange(n_logical)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)
    for b in range(B):
        table[b, :nblk[b]] = phys[starts[b]:starts[b + 1]]

    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(t) for t in trees])
    N = int(offsets[-1])
    parents = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees]) if N else \
        np.zeros(0, dtype=np.int32)

    q = _store(rng.standard_normal((N, Hq, D), dtype=np.float32), dtype)

    store_dt = np.uint16 if dtype == "bf16" else np.float32
    nan_val = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)

    def draw_pool(scale: float):
        pool = np.full((num_blocks, Hkv, BLOCK, D), nan_val, dtype=store_dt)
        logical = [] if keep_logical else None
        for b in range(B):
            nb = int(nblk[b])
            if nb == 0:
                if keep_logical:
                    logical.append(np.zeros((0, Hkv, D), dtype=store_dt))
                continue
            x = rng.standard_normal((nb, Hkv, BLOCK, D), dtype=np.float32)
            if scale != 1.0:
                x *= np.float32(scale)
            xs = _store(x, dtype)
            used = int(P[b]) - (nb - 1) * BLOCK
            if used < BLOCK:   # poison the unused tail of the last block
                xs[nb - 1, :, used:, :] = nan_val
            pool[table[b, :nb]] = xs
            if keep_logical:
                lg = xs.transpose(0, 2, 1, 3).reshape(nb * BLOCK, Hkv, D)[:int(P[b])]
                logical.append(np.ascontiguousarray(lg))
        return pool, logical

    k_cache, k_log = draw_pool(key_scale)
    v_cache, v_log = draw_pool(1.0)
    kt = rng.standard_normal((N, Hkv, D), dtype=np.float32)
    if key_scale != 1.0:
        kt *= np.float32(key_scale)
    k_tree = _store(kt, dtype)
    v_tree = _store(rng.standard_normal((N, Hkv, D), dtype=np.float32), dtype)

    scale = float(softmax_scale) if softmax_scale else 1.0 / float(np.sqrt(D))
    return TreeVerifyInputs(
        name=name, seed=int(seed), dtype=dtype, batch=B, num_q_heads=Hq,
        num_kv_heads=Hkv, head_dim=D, softmax_scale=scale, q=q, k_cache=k_cache,
        v_cache=v_cache, block_table=table, prefix_lens=P.astype(np.int32),
        k_tree=k_tree, v_tree=v_tree, parents=parents, tree_offsets=offsets,
        k_prefix_logical=k_log, v_prefix_logical=v_log,
    )


def make_config(index: int, seed: Optional[int] = None, keep_logical: bool = False,
                batch_override: Optional[int] = None) -> TreeVerifyInputs:
    """Build config ``index`` (1..5: the verify workloads; 6, 7: trees of more
    than 64 nodes).  ``batch_override`` shrinks configs 3, 5 and 7 for tests
    (same recipe, first draws only)."""
    if seed is None:
        seed = 1000 + index
    rng = np.random.default_rng(seed)
    name = f"cfg{index}"
    if index == 1:
        return make_inputs(dtype="f32", num_q_heads=4, num_kv_heads=1, head_dim=64,
                           prefix_lens=[128], trees=[TREE_CFG1], rng=rng, seed=seed,
                           name=name, softmax_scale=1.0 / 8.0, permute_blocks=False,
                           keep_logical=keep_logical)
    if index == 2:
        return make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           prefix_lens=[8192], trees=[TREE_12], rng=rng, seed=seed,
                           name=name, keep_logical=keep_logical)
    if index == 3:
        B = 32 if batch_override is None else int(batch_override)
        lens = rng.integers(1024, 8192 + 1, size=B)
        return make_inputs(dtype="bf16", num_q_heads=8, num_kv_heads=1, head_dim=128,
                           prefix_lens=lens, trees=[TREE_CHAIN4] * B, rng=rng, seed=seed,
                           name=name, keep_logical=keep_logical)
    if index == 4:
        return make_inputs(dtype="bf16", num_q_heads=5, num_kv_heads=1, head_dim=128,
                           prefix_lens=[8192], trees=[TREE_12], rng=rng, seed=seed,
                           name=name, key_scale=2.0, keep_logical=keep_logical)
    if index == 5:
        B = 256 if batch_override is None else int(batch_override)
        z = rng.standard_normal(B)
        lens = np.clip(np.rint(np.exp(np.log(2048.0) + z)), 16, 32768).astype(np.int64)
        kinds = rng.choice(3, size=B, p=[0.2, 0.5, 0.3])
        menu = (TREE_SINGLE, TREE_CHAIN4, TREE_12)
        trees = [menu[k] for k in kinds]
        return make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           prefix_lens=lens, trees=trees, rng=rng, seed=seed,
                           name=name, keep_logical=keep_logical)
    if index == 6:
        tree = _random_tree(rng, 256)
        return make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           prefix_lens=[8192], trees=[tree], rng=rng, seed=seed,
                           name=name, keep_logical=keep_logical)
    if index == 7:
        B = 8 if batch_override is None else int(batch_override)
        lens = rng.integers(16, 100 + 1, size=B)
        trees = [_random_tree(rng, 128) for _ in range(B)]
        return make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           prefix_lens=lens, trees=trees, rng=rng, seed=seed,
                           name=name, keep_logical=keep_logical)
    raise ValueError(f"config index must be 1..7, got {index}")


def _random_tree(rng: np.random.Generator, T: int) -> List[int]:
    """Seeded random topologically ordered parent array: node i's parent is
    uniform over the earlier nodes."""
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
