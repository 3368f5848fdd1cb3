"""Shared test helpers: input builders and independent reference pieces.

Nothing here imports the HIP binding; the oracle is imported only by the tests
that use it.
"""
from __future__ import annotations

import os
from fractions import Fraction
from typing import List, Sequence

import numpy as np

from workloads import TreeVerifyInputs, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_mask_table():
    """Parse tests/golden/masks.txt -> list of (name, parents, words)."""
    out = []
    with open(os.path.join(GOLDEN, "masks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, par, words = [s.strip() for s in line.split("|")]
            parents = [int(x) for x in par.split(",")]
            masks = [int(x, 16) for x in words.split(",")]
            out.append((name, parents, masks))
    return out


def read_hand_example():
    """Parse tests/golden/hand_example.txt -> {piece: {node: (o0, o1, lse)}}."""
    out = {}
    with open(os.path.join(GOLDEN, "hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            piece, node, o0, o1, lse = line.split()
            assert lse.startswith("ln")
            out.setdefault(piece, {})[int(node)] = (
                float(Fraction(o0)), float(Fraction(o1)), float(np.log(int(lse[2:]))))
    return out


def manual_inputs(*, q, k_prefix, v_prefix, k_tree, v_tree, trees, scale,
                  dtype="f32", name="manual") -> TreeVerifyInputs:
    """Build inputs from explicit logical arrays (identity paging, 64-token blocks).

    q: [N, Hq, D]; k_prefix/v_prefix: list over sequences of [P_b, Hkv, D];
    k_tree/v_tree: [N, Hkv, D]; trees: list of parent lists.
    """
    B = len(trees)
    q = np.asarray(q, dtype=np.float32)
    N, Hq, D = q.shape
    Hkv = np.asarray(k_tree).shape[1]
    P = [int(np.asarray(k).shape[0]) for k in k_prefix]
    nblk = [(p + 63) // 64 for p in P]
    nb_total = max(1, sum(nblk))
    kc = np.full((nb_total, Hkv, 64, D), np.nan, dtype=np.float32)
    vc = np.full((nb_total, Hkv, 64, D), np.nan, dtype=np.float32)
    table = np.full((B, max(1, max(nblk) if nblk else 1)), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        kb = np.asarray(k_prefix[b], dtype=np.float32)
        vb = np.asarray(v_prefix[b], dtype=np.float32)
        for j in range(nblk[b]):
            n = min(64, P[b] - 64 * j)
            kc[nxt, :, :n, :] = kb[64 * j:64 * j + n].transpose(1, 0, 2)
            vc[nxt, :, :n, :] = vb[64 * j:64 * j + n].transpose(1, 0, 2)
            table[b, j] = nxt
            nxt += 1
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(t) for t in trees])
    parents = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees])
    assert offsets[-1] == N
    return TreeVerifyInputs(
        name=name, seed=-1, dtype=dtype, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, softmax_scale=float(scale), q=q, k_cache=kc, v_cache=vc,
        block_table=table, prefix_lens=np.asarray(P, dtype=np.int32),
        k_tree=np.asarray(k_tree, dtype=np.float32),
        v_tree=np.asarray(v_tree, dtype=np.float32), parents=parents,
        tree_offsets=offsets,
        k_prefix_logical=[np.asarray(k, dtype=np.float32) for k in k_prefix],
        v_prefix_logical=[np.asarray(v, dtype=np.float32) for v in v_prefix],
    )


def random_tree(rng: np.random.Generator, T: int, forest_p: float = 0.0) -> List[int]:
    """Random topologically ordered parent array of T nodes."""
    par = [-1]
    for i in range(1, T):
        if forest_p and rng.random() < forest_p:
            par.append(-1)
        else:
            par.append(int(rng.integers(0, i)))
    return par[:T]


def small_inputs(seed: int, *, dtype="f32", B=2, Hq=4, Hkv=2, D=16,
                 prefix_lens: Sequence[int] = (70, 5), trees=None, key_scale=1.0,
                 permute=True, spare_blocks=3, keep_logical=True) -> TreeVerifyInputs:
    rng = np.random.default_rng(seed)
    if trees is None:
        trees = [random_tree(rng, int(rng.integers(1, 9))) for _ in range(B)]
    return make_inputs(dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       prefix_lens=list(prefix_lens), trees=trees, rng=rng, seed=seed,
                       name=f"small{seed}", key_scale=key_scale,
                       permute_blocks=permute, spare_blocks=spare_blocks,
                       keep_logical=keep_logical)


def dp_masks(parents: Sequence[int]) -> List[int]:
    """Ancestor-or-self masks by combining each parent's word with the node's own
    bit (parents precede children).  Written here independently of the oracle's
    parent walk so that each checks the other."""
    m: List[int] = []
    for i, p in enumerate(parents):
        m.append((m[p] if p >= 0 else 0) | (1 << i))
    return m


def f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Test-side widening of stored values (bf16 bits or fp32) to float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    hi = np.asarray(x, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
    return hi.view(np.float32).astype(np.float64)
