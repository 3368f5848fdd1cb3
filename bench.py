#!/usr/bin/env python3
"""Benchmark of the fused tree-verify attention call on one MI355X.

One step = one ``tree_attn_verify`` call (prefix pass + tree mask + suffix pass +
merge, one kernel launch) over one batch of seeded synthetic input that is
already resident in HBM.  Default workload: the Llama-3.1-8B-shaped verify step
(bf16, batch 1, 32 query / 8 KV heads, head dim 128, 8192-token paged prefix,
12-node tree).

Timing protocol
* The 256 MB last-level cache is larger than one batch (33.8 MB), so the step
  rotates over R replicas (>= 1 GiB together) of what differs from one model
  layer to the next -- the KV pool, q and the tree K/V -- and every step reads
  them from HBM.  The block table, prefix lengths, parent array and tree
  offsets are shared by every layer of a verify step, so one copy serves all
  replicas, as it would in a layer loop.
* W warm-up steps, then K timed steps queued back to back on one stream.  The
  GPU is first held by a short spin kernel so that the host queues all K steps
  before the first one starts; one pair of HIP events on the launch stream
  brackets the K steps (events between steps would themselves cost several
  microseconds at this scale).
* ms_per_step = (end event - start event) / K.  With one kernel per step this is
  the kernel's average duration plus the (sub-0.1 us) gap between queued
  launches; value = algorithmic bytes / ms_per_step.
* cpu_baseline: the fp64 NumPy oracle on the same workload, on this host.
* after_verify: greedy acceptance and the commit of the accepted paths into the
  paged cache, timed on a 256-sequence batch (see bench_after_verify).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify attention µs/call + achieved HBM GB/s (% of peak), 8k ctx"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3   # dense fp32 matrix peak
# counter-measured HBM traffic of the fused kernel, per workload (see profiles/)
TRAFFIC_FILES = {
    2: os.path.join(ROOT, "profiles", "attn_kernel_llama8b_verify_8k_traffic.json"),
    3: os.path.join(ROOT, "profiles", "attn_kernel_70b_head_share_b32_traffic.json"),
    4: os.path.join(ROOT, "profiles", "attn_kernel_maverick_head_share_8k_traffic.json"),
    5: os.path.join(ROOT, "profiles", "attn_kernel_ragged_b256_traffic.json"),
}
# counter-measured MFMA busy cycles and bf16 MFMA work of the fused kernel (see profiles/)
MFMA_FILE = os.path.join(ROOT, "profiles", "attn_kernel_mfma_counters.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ancestor_pairs(parents) -> int:
    """sum over nodes of |ancestor-or-self set| (for the flop count)."""
    total = 0
    par = [int(x) for x in parents]
    for i in range(len(par)):
        j = i
        while j != -1:
            total += 1
            j = par[j]
    return total


def algorithmic_bytes(inp) -> int:
    s = inp.elem_bytes
    Hq, Hkv, D = inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    tot = 0
    for b in range(inp.batch):
        P = int(inp.prefix_lens[b])
        T = int(inp.tree_offsets[b + 1] - inp.tree_offsets[b])
        tot += (2 * P * Hkv * D * s + T * Hq * D * s + 2 * T * Hkv * D * s + T * Hq * D * s
                + 4 * T * Hq + 4 * math.ceil(P / 64) + 4 * T + 8)
    return tot


def algorithmic_flops(inp) -> int:
    Hq, D = inp.num_q_heads, inp.head_dim
    tot = 0
    for b in range(inp.batch):
        lo, hi = int(inp.tree_offsets[b]), int(inp.tree_offsets[b + 1])
        P = int(inp.prefix_lens[b])
        tot += 4 * Hq * D * ((hi - lo) * P + ancestor_pairs(inp.parents[lo:hi]))
    return tot


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_attention_verify_attn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(config_index: int, split: int):
    """HBM bytes per call (both launches of a two-launch call) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources and
    the same workload; else None."""
    path = TRAFFIC_FILES.get(config_index)
    if path is None:
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_source_hash():
        return None
    if rec.get("config") != config_index or rec.get("split_tokens") != split:
        return None
    return rec.get("bytes_per_call")


def measured_mfma(config_index: int, split: int):
    """(counted MFMA utilisation, counted bf16 MFMA flops) of the fused kernel
    from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources and the same workload; else (None, None)."""
    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f).get(str(config_index))
    except (OSError, ValueError):
        return None, None
    if not rec or rec.get("kernel_sha") != kernel_source_hash() or rec.get("split_tokens") != split:
        return None, None
    return rec.get("mfma_util_counted"), rec.get("mfma_flops_counted")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s: float, nbytes: int):
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    calls = 0
    c0 = time.process_time()
    t0 = time.perf_counter()
    while True:
        oracle.verify(inp)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cpu_s = time.process_time() - c0
    per = el / calls
    return {
        "value": nbytes / per / 1e9,
        "unit": "GB/s",
        "us_per_call": per * 1e6,
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{calls} full fp64 oracle verify call(s) of the benchmark workload, "
                  f"{el:.1f} s wall clock ({cpu_s:.1f} s of process CPU time) on {cpu_model()}, "
                  f"{threads} BLAS threads",
        "clock": "wall",
    }


def summarize_trace(path: str, kernel: str) -> dict:
    """Per-dispatch duration statistics of the kernels whose name contains
    `kernel`, from a rocprofv3 --kernel-trace CSV (kernel_trace.csv)."""
    import csv
    durs = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel in row.get("Kernel_Name", ""):
                durs.append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    if not durs:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} in {path}")
    out = {"kernel": kernel, **_dist(durs)}
    # a call made in two launches: each attention dispatch followed by a
    # combine_kernel dispatch on the same queue; per call, the span from the
    # first's start to the second's end (the gap between them included)
    with open(path, newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    spans, comb = [], []
    for a, b in zip(rows, rows[1:]):
        if kernel in a.get("Kernel_Name", "") and "combine_kernel" in b.get("Kernel_Name", ""):
            spans.append((int(b["End_Timestamp"]) - int(a["Start_Timestamp"])) / 1e3)
            comb.append((int(b["End_Timestamp"]) - int(b["Start_Timestamp"])) / 1e3)
    if spans:
        out["combine_kernel"] = _dist(comb)
        out["call_span"] = _dist(spans)
    return out


def _dist(durs) -> dict:
    import statistics
    q = statistics.quantiles(durs, n=10, method="inclusive")
    return {"dispatches": len(durs), "mean_us": round(statistics.fmean(durs), 3),
            "p10_us": round(q[0], 3), "median_us": round(statistics.median(durs), 3),
            "p90_us": round(q[8], 3), "min_us": round(min(durs), 3), "max_us": round(max(durs), 3)}


def kv_tiles(inp):
    """Byte offsets of the paged K and V tiles a verify call reads, in the order
    the attention kernel streams them (sequence, KV head, block; K then V),
    within one buffer holding the K pool and then the V pool; and the tile and
    pool sizes."""
    import numpy as np
    Hkv, D = inp.num_kv_heads, inp.head_dim
    tile = 64 * D * inp.elem_bytes
    pool = inp.num_blocks * Hkv * tile
    parts = []
    for b in range(inp.batch):
        nb = -(-int(inp.prefix_lens[b]) // 64)
        ids = inp.block_table[b, :nb].astype(np.int64)
        for g in range(Hkv):
            k = (ids * Hkv + g) * tile
            parts.append(np.stack([k, k + pool], axis=1).reshape(-1))
    offs = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return offs, tile, pool


def floor_run(torch, nbytes: int, steps: int, replica_bytes: float, inp=None) -> dict:
    """Reference floors for a launch that streams `nbytes` from HBM, timed like
    the benchmark (rotating replicas of at least `replica_bytes` in total so
    every step reads HBM, the GPU held while the host queues the K steps, one
    event pair around them): a device-wide sum of the bytes (read only), a
    device copy of them (read + write), a one-workgroup empty launch, the
    measurement library's plain streaming read of the bytes, and (with the
    workload's inputs) its gather read of the paged K/V tiles the call reads."""
    n = nbytes // 2
    R = max(1, math.ceil(replica_bytes / nbytes))
    src = [torch.randn(n, device="cuda").to(torch.bfloat16) for _ in range(R)]
    dst = [torch.empty_like(x) for x in src]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    torch.cuda._sleep(1_000_000)
    s1.record()
    torch.cuda.synchronize()
    per_cycle_ms = max(s0.elapsed_time(s1), 1e-3) / 1_000_000

    def timed(fn):
        for i in range(10):
            fn(i % R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int((20.0 + 0.1 * steps) / per_cycle_ms))
        e0.record()
        for i in range(steps):
            fn(i % R)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    read_us = timed(lambda r: torch.sum(src[r], dtype=torch.float32))
    copy_us = timed(lambda r: dst[r].copy_(src[r]))
    empty_us = timed(lambda r: torch.cuda._sleep(0))
    # the measurement library's streaming read (libtafloor.so): the same bytes
    # (rounded down to 16), read once and folded, for a few launch shapes
    lib = floor_lib()
    nb16 = (2 * n) // 16 * 16
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def stream_read(grid, threads, loads):
        def fn(r):
            rc = lib.ta_floor_read(ctypes.c_void_p(src[r].data_ptr()), nb16, grid, threads, loads,
                                   ctypes.c_void_p(sink.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"ta_floor_read failed ({rc})")
        return timed(fn)

    shapes = {"256x512x4": (256, 512, 4), "1024x512x4": (1024, 512, 4),
              "4096x512x4": (4096, 512, 4), "2048x256x8": (2048, 256, 8)}
    sr = {k: round(stream_read(*v), 3) for k, v in shapes.items()}
    best = min(sr, key=sr.get)
    gather = {}
    if inp is not None:
        import numpy as np
        offs, tile, pool = kv_tiles(inp)
        del src, dst
        Rg = max(1, math.ceil(replica_bytes / (2 * pool)))
        pools = [torch.empty(2 * pool, dtype=torch.uint8, device="cuda") for _ in range(Rg)]
        d_offs = torch.from_numpy(np.ascontiguousarray(offs)).cuda()
        gbytes = len(offs) * tile

        def gather_read(grid, threads, loads):
            def fn(r):
                rc = lib.ta_floor_gather(ctypes.c_void_p(pools[r % Rg].data_ptr()),
                                         ctypes.c_void_p(d_offs.data_ptr()), len(offs), tile, grid,
                                         threads, loads, ctypes.c_void_p(sink.data_ptr()), stream)
                if rc != 0:
                    raise RuntimeError(f"ta_floor_gather failed ({rc})")
            return timed(fn)

        gshapes = {k: v for k, v in (("256x512x4", (256, 512, 4)), ("1024x512x4", (1024, 512, 4)),
                                     ("2048x256x8", (2048, 256, 8)))
                   if -(-len(offs) // v[0]) <= 4096}
        gr = {k: round(gather_read(*v), 3) for k, v in gshapes.items()}
        gbest = min(gr, key=gr.get)
        gather = {"gather_tiles": len(offs), "gather_tile_bytes": tile, "gather_bytes": gbytes,
                  "gather_replicas": Rg, "gather_read_us": gr, "gather_read_best_us": gr[gbest],
                  "gather_read_best_shape": gbest,
                  "gather_read_best_GBps": round(gbytes / gr[gbest] / 1e3, 1)}
    return {"floor_bytes": 2 * n, "replicas": R, "steps": steps, **gather,
            "stream_read_bytes": nb16,
            "stream_read_us": sr,
            "stream_read_best_us": sr[best], "stream_read_best_shape": best,
            "stream_read_best_GBps": round(nb16 / sr[best] / 1e3, 1),
            "stream_read_one_wg_per_cu_GBps": round(nb16 / sr["256x512x4"] / 1e3, 1),
            "sum_read_us": round(read_us, 3), "sum_read_GBps": round(2 * n / read_us / 1e3, 1),
            "copy_us": round(copy_us, 3), "copy_GBps_read_plus_write": round(4 * n / copy_us / 1e3, 1),
            "empty_launch_us": round(empty_us, 3)}


def floor_lib():
    """ctypes handle of the measurement library (streaming-read floor kernel)."""
    from tree_attention_verify_attn_amd.build import FLOOR_LIB_PATH
    if not os.path.exists(FLOOR_LIB_PATH):
        raise RuntimeError(f"{FLOOR_LIB_PATH} is missing: build it with "
                           "`python -m tree_attention_verify_attn_amd.build`")
    lib = ctypes.CDLL(FLOOR_LIB_PATH)
    lib.ta_floor_read.restype = ctypes.c_int
    lib.ta_floor_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ta_floor_gather.restype = ctypes.c_int
    lib.ta_floor_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    return lib


def incache_layout(inp):
    """The same batch with each tree's K/V rows also written into the paged
    cache right after its prefix (two spare blocks and table columns per
    sequence are added for the region); input preparation only."""
    import copy

    import numpy as np

    from workloads import place_tree_in_cache
    B = inp.batch
    nan = np.uint16(0x7FC0) if inp.dtype == "bf16" else np.float32(np.nan)
    pad = np.full((2 * B,) + inp.k_cache.shape[1:], nan, dtype=inp.k_cache.dtype)
    ext = copy.copy(inp)
    ext.k_cache = np.concatenate([inp.k_cache, pad])
    ext.v_cache = np.concatenate([inp.v_cache, pad])
    ext.block_table = np.concatenate(
        [inp.block_table, np.full((B, 2), -1, dtype=np.int32)], axis=1)
    ic, _ = place_tree_in_cache(ext, np.random.default_rng(inp.seed + 7))
    return ic


def bench_after_verify(ta, torch, np, steps: int) -> dict:
    """Greedy acceptance and commit timed on a 256-sequence batch with the
    ragged workload's tree mix (1-node / chain-4 / 12-node at 0.2/0.5/0.3),
    32 query / 8 KV heads, head dim 128, bf16.  Prefix lengths are the ragged
    workload's draws modulo 128 (the commit touches only the blocks at the
    prefix end, so the block-boundary mix is what matters).  Acceptance: K
    calls back to back between two events.  Commit: each call is bracketed by
    its own events after the block table and prefix lengths are restored, so
    every call appends the same rows; median reported.  A spin kernel holds
    the GPU while the host queues the timed calls, so host overhead is not
    timed."""
    from workloads import TREE_12, TREE_CHAIN4, TREE_SINGLE, free_list, make_inputs, make_tokens
    rng = np.random.default_rng(1005)
    B = 256
    z = rng.standard_normal(B)
    lens = (np.clip(np.rint(np.exp(np.log(2048.0) + z)), 16, 32768).astype(np.int64) % 128)
    kinds = rng.choice(3, size=B, p=[0.2, 0.5, 0.3])
    trees = [(TREE_SINGLE, TREE_CHAIN4, TREE_12)[k] for k in kinds]
    inp = make_inputs(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                      prefix_lens=lens, trees=trees, rng=rng, spare_blocks=2 * B,
                      extra_table_cols=1)
    draft, argmax = make_tokens(inp.parents, inp.tree_offsets, rng, p_match=0.7, vocab=32000)
    free = free_list(inp, rng)

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    shape = ta.make_shape(batch=B, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          max_blocks_per_seq=inp.max_blocks_per_seq, max_tree_nodes=12,
                          max_prefix_len=inp.max_prefix_len, total_tree_nodes=inp.total_tree_nodes,
                          num_blocks=inp.num_blocks, dtype=ta.DTYPE_BF16)
    ws = ta.alloc_workspace(shape)
    par, off = dev(inp.parents), dev(inp.tree_offsets)
    dr, am = dev(draft), dev(argmax)
    kt, vt = dev(inp.k_tree), dev(inp.v_tree)
    kc, vc = dev(inp.k_cache), dev(inp.v_cache)
    table0, plen0 = dev(inp.block_table), dev(inp.prefix_lens)
    table, plen = table0.clone(), plen0.clone()
    freed = dev(free)
    taken = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib = ta._lib.load()
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    path = torch.empty(B, 12, dtype=torch.int32, device="cuda")
    bonus = torch.empty(B, dtype=torch.int32, device="cuda")
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    acc_args = (ctypes.byref(shape), par.data_ptr(), off.data_ptr(), dr.data_ptr(), am.data_ptr(),
                n.data_ptr(), path.data_ptr(), bonus.data_ptr(), ws.data_ptr(), ws.numel(), sh)
    com_args = (ctypes.byref(shape), kt.data_ptr(), vt.data_ptr(), par.data_ptr(), off.data_ptr(),
                n.data_ptr(), path.data_ptr(), kc.data_ptr(), vc.data_ptr(), table.data_ptr(),
                plen.data_ptr(), freed.data_ptr(), len(free), taken.data_ptr(), ws.data_ptr(),
                ws.numel(), sh)

    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1_000_000)
    c1.record()
    torch.cuda.synchronize()
    per_cycle_ms = max(c0.elapsed_time(c1), 1e-3) / 1_000_000

    def hold():  # keep the GPU busy while the host queues the timed calls (~100 us each)
        torch.cuda._sleep(int(0.1 * steps / per_cycle_ms))

    for _ in range(5):
        lib.tree_attn_accept_greedy(*acc_args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold()
    e0.record()
    for _ in range(steps):
        lib.tree_attn_accept_greedy(*acc_args)
    e1.record()
    torch.cuda.synchronize()
    accept_us = e0.elapsed_time(e1) * 1e3 / steps
    rows = int(n.sum().item())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for _ in range(3):
        table.copy_(table0)
        plen.copy_(plen0)
        lib.tree_attn_commit(*com_args)
    torch.cuda.synchronize()
    hold()
    for a, b in evs:
        table.copy_(table0)
        plen.copy_(plen0)
        a.record()
        lib.tree_attn_commit(*com_args)
        b.record()
    torch.cuda.synchronize()
    commit_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
    err = ta.get_error(ws)
    if err != 0:
        raise RuntimeError(f"device error in acceptance/commit: {ta.status_string(err)}")
    moved = 2 * rows * 8 * 128 * 2  # K and V rows read and written once each
    return {
        "workload": "256 sequences, tree mix 1/chain-4/12 (0.2/0.5/0.3), Hkv 8, D 128, bf16",
        "accept_greedy_us": round(accept_us, 3),
        "commit_us": round(commit_us, 3),
        "commit_rows": rows,
        "commit_blocks_taken": int(taken.item()),
        "commit_row_bytes_moved": 2 * moved,
        "commit_GBps": round(2 * moved / (commit_us * 1e-6) / 1e9, 2),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2,
                    help="workload 1..5 (default 2); 6, 7: trees of more than 64 nodes")
    ap.add_argument("--split-tokens", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--entry", choices=("verify", "split", "incache"), default="verify",
                    help="fused single launch (default), the four-call split path, or the fused "
                         "launch with the tree rows kept in the paged cache after each prefix")
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-after-verify", action="store_true",
                    help="skip timing greedy acceptance and the cache commit")
    ap.add_argument("--floor", action="store_true",
                    help="instead of the benchmark, time plain device reads and copies of the "
                         "workload's algorithmic bytes (reference floors), one JSON line")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-dispatch p10 / median / p90 of the attention kernel from a "
                         "rocprofv3 --kernel-trace CSV and exit (no GPU needed)")
    ap.add_argument("--trace-kernel", default="attn_kernel",
                    help="kernel-name substring for --summarize-trace")
    ap.add_argument("--copy-bytes", type=float, default=0.0,
                    help="instead of the benchmark, run --steps plain device-to-device copies "
                         "of this many bytes (reference for the HBM traffic counters)")
    args = ap.parse_args()

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.trace_kernel)))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is single-process; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tree_attention_verify_attn_amd as ta
    from tree_attention_verify_attn_amd._lib import load
    from workloads import CONFIG_NAMES, make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_bytes > 0:
        n = int(args.copy_bytes) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "copies": max(1, args.steps)}))
        return 0
    lib = load()

    log(f"building workload cfg{args.config}")
    inp = make_config(args.config)
    if args.floor:
        res = floor_run(torch, algorithmic_bytes(inp), args.steps, args.replica_bytes, inp)
        res["workload"] = CONFIG_NAMES[args.config]
        print(json.dumps(res), flush=True)
        return 0
    if inp.max_tree_nodes > 64 and args.entry == "incache":
        log("in-cache tree rows are for trees of up to 64 nodes; using the fused verify")
        args.entry = "verify"
    if args.entry == "incache":
        inp = incache_layout(inp)
    nbytes = algorithmic_bytes(inp)
    flops = algorithmic_flops(inp)
    dt = ta.DTYPE_BF16 if inp.dtype == "bf16" else ta.DTYPE_F32
    shape = ta.make_shape(batch=inp.batch, num_q_heads=inp.num_q_heads,
                          num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                          max_blocks_per_seq=inp.max_blocks_per_seq,
                          max_tree_nodes=inp.max_tree_nodes, max_prefix_len=inp.max_prefix_len,
                          total_tree_nodes=inp.total_tree_nodes, num_blocks=inp.num_blocks,
                          dtype=dt, softmax_scale=inp.softmax_scale,
                          split_tokens=args.split_tokens)
    split = ta.split_tokens(shape)

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    host_arrays = [inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.prefix_lens,
                   inp.k_tree, inp.v_tree, inp.parents, inp.tree_offsets]
    per_layer = (0, 1, 2, 5, 6)  # q, k_cache, v_cache, k_tree, v_tree
    footprint = sum(host_arrays[i].nbytes for i in per_layer)
    R = max(1, math.ceil(args.replica_bytes / footprint))
    log(f"per-layer footprint {footprint / 1e6:.1f} MB -> {R} replicas; split_tokens {split}")
    first = [dev(a) for a in host_arrays]
    replicas = [first] + [[t.clone() if i in per_layer else t for i, t in enumerate(first)]
                          for _ in range(R - 1)]
    ws = ta.alloc_workspace(shape)
    N, Hq, D = inp.total_tree_nodes, inp.num_q_heads, inp.head_dim
    outs = [torch.empty(N, Hq, D, dtype=first[0].dtype, device="cuda") for _ in range(R)]
    lses = [torch.empty(N, Hq, dtype=torch.float32, device="cuda") for _ in range(R)]
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    call_args = []
    for r in range(R):
        q, kc, vc, bt, pl, kt, vt, par, off = replicas[r]
        call_args.append((ctypes.byref(shape), q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                          bt.data_ptr(), pl.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                          par.data_ptr(), off.data_ptr(), outs[r].data_ptr(),
                          lses[r].data_ptr(), wsp, wsn, sh))
    verify = lib.tree_attn_verify

    if args.entry == "incache":
        verify_ic = lib.tree_attn_verify_incache

        def step(r):
            a = call_args[r]
            rc = verify_ic(*a[:6], *a[8:])    # no separate tree K/V tensors
            if rc:
                raise RuntimeError(f"tree_attn_verify_incache: {ta.status_string(rc)}")
    elif args.entry == "verify":
        def step(r):
            rc = verify(*call_args[r])
            if rc:
                raise RuntimeError(f"tree_attn_verify: {ta.status_string(rc)}")
    else:
        # split path: mask build + prefix pass + suffix pass + merge, four launches
        masks = torch.empty(N, dtype=torch.int64, device="cuda")
        po = torch.empty(N, Hq, D, dtype=torch.float32, device="cuda")
        pl = torch.empty(N, Hq, dtype=torch.float32, device="cuda")
        so = torch.empty_like(po)
        sl = torch.empty_like(pl)
        sp = ctypes.byref(shape)

        def step(r):
            q, kc, vc, bt, pl_, kt, vt, par, off = replicas[r]
            rc = lib.tree_attn_build_mask(sp, par.data_ptr(), off.data_ptr(), masks.data_ptr(),
                                          wsp, wsn, sh)
            rc = rc or lib.tree_attn_prefix(sp, q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                            bt.data_ptr(), pl_.data_ptr(), off.data_ptr(),
                                            po.data_ptr(), pl.data_ptr(), wsp, wsn, sh)
            rc = rc or lib.tree_attn_suffix(sp, q.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                                            masks.data_ptr(), off.data_ptr(), so.data_ptr(),
                                            sl.data_ptr(), sh)
            rc = rc or lib.tree_attn_merge(N * Hq, D, int(shape.dtype), po.data_ptr(),
                                           pl.data_ptr(), so.data_ptr(), sl.data_ptr(),
                                           outs[r].data_ptr(), lses[r].data_ptr(), sh)
            if rc:
                raise RuntimeError(f"split path: {ta.status_string(rc)}")

    # correctness spot check of the benchmarked call itself
    step(0)
    torch.cuda.synchronize()
    err = ta.get_error(ws)
    if err != 0:
        raise RuntimeError(f"device error {ta.status_string(err)}")

    log(f"warm-up {args.warmup}")
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    # hold the GPU long enough for the host to queue every timed step
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    torch.cuda._sleep(1_000_000)
    s1.record()
    torch.cuda.synchronize()
    per_cycle_ms = max(s0.elapsed_time(s1), 1e-3) / 1_000_000
    hold_ms = 20.0 + 0.1 * args.steps
    cycles = int(hold_ms / per_cycle_ms)

    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {K} steps ({args.entry})")
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    torch.cuda._sleep(cycles)
    e0.record()
    for i in range(K):
        step(i % R)
    e1.record()
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / K
    kernel_ms = ms_per_step
    err = ta.get_error(ws)
    if err != 0:
        raise RuntimeError(f"device error during timing: {ta.status_string(err)}")

    # one call = one attention launch, or two (attention, then combine_kernel)
    # for a one-sequence shape in the two-launch mode; the roofline is taken
    # over the whole call either way
    launch_mode = ta.launch_info(shape)["mode"]
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.config, split) if args.entry == "verify" else None
    mfma_counted, mfma_flops = (measured_mfma(args.config, split) if args.entry == "verify"
                                else (None, None))
    # the roofline that bounds this workload: HBM unless its matrix work takes
    # longer at peak than its algorithmic bytes do (large trees, long prefixes)
    peak_tf = PEAK_BF16_TFLOPS if inp.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved_tf = flops / (kernel_ms * 1e-3) / 1e12
    mfma_bound = flops / (peak_tf * 1e12) > nbytes / (PEAK_HBM_GBS * 1e9)
    result = {
        "metric": METRIC,
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(ms_per_step * 1e3, 3),
        "entry": args.entry,
        "pct_of_peak_hbm": round(100.0 * nbytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(inp.total_tree_nodes / (ms_per_step * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "batch": inp.batch,
            "num_q_heads": inp.num_q_heads,
            "num_kv_heads": inp.num_kv_heads,
            "head_dim": inp.head_dim,
            "prefix_tokens": int(inp.prefix_lens.sum()),
            "tree_nodes": inp.total_tree_nodes,
            "split_tokens": split,
            "chunk_rule": ("host" if args.split_tokens > 0 or inp.batch == 1 else
                           "device: from the actual prefix lengths when the groups are fewer "
                           "than the workgroups, else split_tokens"),
            "replicas": R,
            "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops,
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(achieved_tf, 2) if mfma_bound else round(achieved, 2),
            "peak": peak_tf if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(achieved_tf / peak_tf if mfma_bound else achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "hbm_frac": round(achieved / PEAK_HBM_GBS, 4),
            "kernel": (f"attn_kernel<{'bf16' if inp.dtype == 'bf16' else 'f32'},{D},fused"
                       + (",tree segments in the ring" if inp.max_tree_nodes > 64 else "")
                       + (",two launches> + combine_kernel " if launch_mode == "two_launch"
                          else "> ")
                       + ("(tree_attn_verify)" if args.entry == "verify"
                          else "(tree_attn_verify_incache)")
                       if args.entry in ("verify", "incache")
                       else "split path: mask + prefix + suffix + merge kernels"),
            "launch_mode": launch_mode,
            "mfma_util": round(achieved_tf / peak_tf, 5),
            "mfma_util_counted": mfma_counted,
            "mfma_flops_counted": mfma_flops,
        },
        "host_wall_s": round(t_host, 3),
    }
    if not args.no_after_verify:
        log("acceptance and commit (after-verify step)")
        result["after_verify"] = bench_after_verify(ta, torch, np, 50)
    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, nbytes)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
