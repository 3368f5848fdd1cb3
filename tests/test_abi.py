"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad host arguments before touching the device."""
import ctypes
import os
import re

import pytest

import tree_attention_verify_attn_amd as ta
from tree_attention_verify_attn_amd._lib import EXPORTED, Shape, load

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")

FAKE = 0x100000  # aligned non-null address; never dereferenced on these paths


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(tree_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(EXPORTED) == header_functions()


def test_library_exports_every_header_symbol():
    lib = load()
    for name in header_functions():
        assert hasattr(lib, name), name


def test_shape_struct_layout_matches_header():
    # 11 int32, one float, one enum (int32) -> 13 * 4 bytes
    assert ctypes.sizeof(Shape) == 52


def shape(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_blocks_per_seq=128,
                max_tree_nodes=12, max_prefix_len=8192, total_tree_nodes=12, num_blocks=128,
                dtype=ta.DTYPE_BF16)
    base.update(kw)
    return ta.make_shape(**base)


def test_workspace_size_valid_and_monotone():
    a = ta.workspace_size(shape(split_tokens=256))
    b = ta.workspace_size(shape(split_tokens=256, max_prefix_len=4096))
    c = ta.workspace_size(shape(split_tokens=256, batch=2, max_prefix_len=8192))
    assert a > 0 and b > 0 and c > 0
    assert b < a < c


@pytest.mark.parametrize("kw", [
    dict(head_dim=96), dict(head_dim=256), dict(block_size=32), dict(max_tree_nodes=257),
    dict(batch=5000),
    # more than 2^18 groups (sequence, KV head, 64-row pass)
    dict(batch=2048, num_q_heads=64, num_kv_heads=64, max_tree_nodes=256, total_tree_nodes=256),
])
def test_unsupported_shapes(kw):
    s = shape(**kw)
    assert ta.workspace_size(s) == 0
    rc = load().tree_attn_verify(ctypes.byref(s), *([FAKE] * 11), FAKE, 1 << 40, None)
    assert rc == 2  # TA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(num_q_heads=30), dict(batch=0), dict(num_kv_heads=0), dict(max_tree_nodes=0),
    dict(max_prefix_len=-1), dict(max_prefix_len=128 * 64 + 1), dict(split_tokens=100),
    dict(dtype=7), dict(num_blocks=0), dict(max_blocks_per_seq=0),
])
def test_invalid_shapes(kw):
    s = shape(**kw)
    assert ta.workspace_size(s) == 0
    rc = load().tree_attn_verify(ctypes.byref(s), *([FAKE] * 11), FAKE, 1 << 40, None)
    assert rc == 1  # TA_ERR_INVALID_ARG


def test_null_and_misaligned_pointers():
    s = shape()
    lib = load()
    args = [FAKE] * 11
    for i in range(11):
        bad = list(args)
        bad[i] = None
        if i == 10:   # lse_out may be null; block_table is index 3
            continue
        assert lib.tree_attn_verify(ctypes.byref(s), *bad, FAKE, 1 << 40, None) == 1, i
    mis = list(args)
    mis[0] = FAKE + 2
    assert lib.tree_attn_verify(ctypes.byref(s), *mis, FAKE, 1 << 40, None) == 1


def test_workspace_checks():
    s = shape()
    lib = load()
    need = ta.workspace_size(s)
    assert lib.tree_attn_verify(ctypes.byref(s), *([FAKE] * 11), FAKE, need - 1, None) == 4
    assert lib.tree_attn_verify(ctypes.byref(s), *([FAKE] * 11), None, need, None) == 4
    assert lib.tree_attn_prefix(ctypes.byref(s), *([FAKE] * 8), FAKE + 8, need, None) == 4


def test_merge_argument_checks():
    lib = load()
    assert lib.tree_attn_merge(-1, 128, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.tree_attn_merge(4, 126, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.tree_attn_merge(4, 128, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.tree_attn_merge(0, 128, 0, None, None, None, None, None, None, None) == 0


def test_status_strings():
    for code in range(10):
        assert ta.status_string(code) and ta.status_string(code) != "unknown status"
    assert ta.status_string(99) == "unknown status"


def test_split_tokens_bounds():
    for kw in [dict(), dict(batch=256), dict(max_prefix_len=32768, max_blocks_per_seq=512),
               dict(split_tokens=64, max_prefix_len=32768, max_blocks_per_seq=512)]:
        s = shape(**kw)
        c = ta.split_tokens(s)
        assert c % 64 == 0 and 64 <= c <= 4096
        assert -(-s.max_prefix_len // c) <= 64    # at most 64 chunks per prefix


@pytest.mark.parametrize("T", [65, 200, 256])
def test_large_trees_accepted_by_every_entry_point(T):
    # trees of 65..256 nodes: every entry point takes the shape and gets as
    # far as its workspace check (a null workspace is refused, not the shape),
    # before touching any device pointer
    s = shape(max_tree_nodes=T, total_tree_nodes=T)
    assert ta.workspace_size(s) > 0
    assert ta.split_tokens(s) > 0
    lib = load()
    assert lib.tree_attn_verify(ctypes.byref(s), *([FAKE] * 11), None, 1 << 40, None) == 4
    assert lib.tree_attn_verify_incache(ctypes.byref(s), *([FAKE] * 9), None, 1 << 40, None) == 4
    assert lib.tree_attn_accept_greedy(ctypes.byref(s), *([FAKE] * 7), None, 1 << 40, None) == 4
    assert lib.tree_attn_commit_incache(ctypes.byref(s), *([FAKE] * 8), None, 1 << 40, None) == 4
    assert lib.tree_attn_commit(ctypes.byref(s), *([FAKE] * 11), 4, FAKE, None, 1 << 40, None) == 4


def test_trees_beyond_256_nodes_refused():
    s = shape(max_tree_nodes=257, total_tree_nodes=257)
    lib = load()
    assert lib.tree_attn_accept_greedy(ctypes.byref(s), *([FAKE] * 7), FAKE, 1 << 40, None) == 2
    assert lib.tree_attn_verify_incache(ctypes.byref(s), *([FAKE] * 9), FAKE, 1 << 40, None) == 2


def test_launch_info_mode_choice():
    """The host's launch plan (no GPU here: sized for a full MI355X, one
    workgroup per CU on 256 CUs)."""
    # one sequence, 8 KV heads, 8192 tokens: every item in the first round,
    # many chunks a group: the partials are combined by a second launch
    i = ta.launch_info(shape())
    assert i["mode"] == "two_launch"
    assert i["max_items"] == 8 * -(-8192 // i["split_tokens"]) and i["max_items"] <= i["grid"] <= 256
    # the same with 2048-token chunks (4 a group): two launches as well; with
    # one chunk a group the attention kernel writes the output rows itself
    i = ta.launch_info(shape(split_tokens=2048))
    assert i["mode"] == "two_launch" and i["max_items"] == 32
    i = ta.launch_info(shape(split_tokens=4096, max_prefix_len=4096))
    assert i["mode"] == "first_round" and i["max_items"] == 8
    # trees of more than 64 nodes take two launches too, except bf16 at head
    # dim 64, whose large-tree kernel has only the one-launch form
    big = dict(max_tree_nodes=100, total_tree_nodes=100, num_q_heads=8, num_kv_heads=8,
               max_prefix_len=4096, split_tokens=256)
    assert ta.launch_info(shape(**big))["mode"] == "two_launch"
    assert ta.launch_info(shape(**big, head_dim=64, dtype=ta.DTYPE_F32))["mode"] == "two_launch"
    assert ta.launch_info(shape(**big, head_dim=64))["mode"] == "first_round"
    # one sequence forced into small chunks: at most 64 chunks a group (64 tokens
    # become 128), 8 * 64 items handed out by ticket
    i = ta.launch_info(shape(split_tokens=64))
    assert i["split_tokens"] == 128
    assert i["mode"] == "ticket" and i["max_items"] == 512 and i["grid"] == 256
    # more groups than workgroups: ticket mode whatever the prefix lengths
    i = ta.launch_info(shape(batch=256, max_prefix_len=32768, max_blocks_per_seq=512,
                             total_tree_nodes=1536))
    assert i["mode"] == "ticket"
    # a batch whose groups fit the grid: the kernel picks the chunk from the actual lengths
    i = ta.launch_info(shape(batch=32, num_q_heads=8, num_kv_heads=1, total_tree_nodes=128))
    assert i["mode"] == "device"
    # short prefixes stream in one chunk per sequence: one sequence up to 3
    # blocks (one launch, no exchange), from 4 blocks two launches again
    for P, mode in ((1, "first_round"), (150, "first_round"), (192, "first_round"),
                    (193, "two_launch"), (256, "two_launch")):
        i = ta.launch_info(shape(max_prefix_len=P, max_blocks_per_seq=8))
        assert i["mode"] == mode, (P, i)
        if mode == "first_round":
            assert i["split_tokens"] == 64 * -(-P // 64) and i["max_items"] == 8, (P, i)
    # a batch up to 6 blocks (8 with 32 groups or more): one chunk per
    # sequence, chosen by the host (one workgroup per group); past that the
    # kernel picks the chunk (and still takes one chunk a sequence when the
    # actual lengths are that short)
    i = ta.launch_info(shape(batch=8, max_prefix_len=384, max_blocks_per_seq=6,
                             total_tree_nodes=96, num_q_heads=8, num_kv_heads=1))
    assert i["split_tokens"] == 384 and i["mode"] == "first_round" and i["max_items"] == 16  # 2 row passes
    i = ta.launch_info(shape(batch=8, max_prefix_len=385, max_blocks_per_seq=7,
                             total_tree_nodes=96, num_q_heads=8, num_kv_heads=1))
    assert i["split_tokens"] < 385 and i["mode"] == "device"
    i = ta.launch_info(shape(batch=8, max_prefix_len=512, max_blocks_per_seq=8,
                             total_tree_nodes=96))  # 64 groups
    assert i["split_tokens"] == 512 and i["mode"] == "first_round" and i["max_items"] == 64
    i = ta.launch_info(shape(batch=8, max_prefix_len=513, max_blocks_per_seq=9,
                             total_tree_nodes=96))
    assert i["split_tokens"] < 513 and i["mode"] == "device"
    with pytest.raises(ta.TreeAttnError):
        ta.launch_info(shape(head_dim=96))
    assert load().tree_attn_launch_info(ctypes.byref(shape()), None) == 1


# ---- the measurement library (streaming-read floor kernel)
FLOOR_HEADER = os.path.join(ROOT, "include", "ta_floor.h")


def floor_lib():
    from tree_attention_verify_attn_amd.build import FLOOR_LIB_PATH
    lib = ctypes.CDLL(FLOOR_LIB_PATH)
    lib.ta_floor_read.restype = ctypes.c_int
    lib.ta_floor_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_floor_library_exports_its_header_symbols():
    names = re.findall(r"\b(ta_floor_\w+)\s*\(", open(FLOOR_HEADER).read())
    assert sorted(set(names)) == ["ta_floor_gather", "ta_floor_read"]
    for n in names:
        assert hasattr(floor_lib(), n)


@pytest.mark.parametrize("args", [
    (None, FAKE, 4, 1024, 8, 256, 4),          # null base
    (FAKE, None, 4, 1024, 8, 256, 4),          # null tile list
    (FAKE, FAKE, 0, 1024, 8, 256, 4),          # no tiles
    (FAKE, FAKE, 4, 1000, 8, 256, 4),          # tile not a multiple of 16
    (FAKE, FAKE, 4, 48, 8, 256, 4),            # 3 words a tile: not a power of two
    (FAKE + 8, FAKE, 4, 1024, 8, 256, 4),      # misaligned base
    (FAKE, FAKE, 5000, 1024, 1, 256, 4),       # more than 4096 tiles a workgroup
    (FAKE, FAKE, 4, 1024, 8, 96, 4),           # threads not a multiple of 64
    (FAKE, FAKE, 4, 1024, 8, 256, 3),          # unsupported loads in flight
])
def test_floor_gather_rejects_bad_arguments(args):
    lib = floor_lib()
    lib.ta_floor_gather.restype = ctypes.c_int
    lib.ta_floor_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    base, offs, n, tb, grid, threads, loads = args
    assert lib.ta_floor_gather(base, offs, n, tb, grid, threads, loads, FAKE, None) == 1


@pytest.mark.parametrize("args", [
    (None, 1024, 8, 256, 4),        # null source
    (FAKE, 0, 8, 256, 4),           # no bytes
    (FAKE, 1000, 8, 256, 4),        # not a multiple of 16
    (FAKE + 8, 1024, 8, 256, 4),    # misaligned source
    (FAKE, 1024, 0, 256, 4),        # empty grid
    (FAKE, 1024, 65537, 256, 4),    # grid too large
    (FAKE, 1024, 8, 96, 4),         # threads not a multiple of 64
    (FAKE, 1024, 8, 1024, 4),       # threads above 512
    (FAKE, 1024, 8, 256, 3),        # unsupported loads in flight
])
def test_floor_read_rejects_bad_arguments(args):
    src, nbytes, grid, threads, loads = args
    assert floor_lib().ta_floor_read(src, nbytes, grid, threads, loads, FAKE, None) == 1
    assert floor_lib().ta_floor_read(FAKE, 1024, 8, 256, 4, None, None) == 1
