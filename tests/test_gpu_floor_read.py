"""The measurement library's streaming-read kernel reads every byte it is given:
each workgroup's word is the XOR of its share, compared with NumPy on the host.
(The benchmark's floor mode times this kernel; this checks that what it times
is a full read.)"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import say
from test_abi import floor_lib


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,grid,threads,loads", [
    (16, 1, 64, 2),
    (1 << 20, 256, 512, 4),
    ((1 << 20) + 48, 7, 192, 8),      # ragged last share
    (33802288, 256, 512, 4),          # the 8k verify's bytes, one workgroup per CU
    (33802288, 4096, 512, 4),
    (4096, 300, 256, 2),              # more workgroups than words: empty shares
])
def test_stream_read_covers_every_word(nbytes, grid, threads, loads):
    say(f"floor read bytes={nbytes} grid={grid} threads={threads} loads={loads}")
    rng = np.random.default_rng(nbytes ^ grid)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((grid,), -1, dtype=torch.int32, device="cuda")
    rc = floor_lib().ta_floor_read(ctypes.c_void_p(src.data_ptr()), nbytes, grid, threads, loads,
                                   ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    got = sink.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    per = -(-n16 // grid)
    quads = words.reshape(n16, 4)
    want = np.zeros(grid, dtype=np.uint32)
    for i in range(grid):
        share = quads[min(i * per, n16):min((i + 1) * per, n16)]
        if len(share):
            want[i] = np.bitwise_xor.reduce(share.reshape(-1))
    np.testing.assert_array_equal(got, want)


@pytest.mark.gpu
@pytest.mark.parametrize("ntiles,tile_bytes,grid,threads,loads", [
    (1, 16, 1, 64, 2),
    (300, 1024, 7, 192, 4),          # ragged last share
    (2048, 16384, 256, 512, 4),      # the 8k verify's K/V tiles, one workgroup per CU
    (100, 4096, 300, 256, 8),        # more workgroups than tiles: empty shares
])
def test_gather_read_covers_every_tile(ntiles, tile_bytes, grid, threads, loads):
    say(f"floor gather tiles={ntiles} tile_bytes={tile_bytes} grid={grid} threads={threads} loads={loads}")
    rng = np.random.default_rng(ntiles ^ tile_bytes)
    pool_tiles = ntiles + 17
    words = rng.integers(0, 2**32, size=pool_tiles * tile_bytes // 4, dtype=np.uint64).astype(np.uint32)
    order = rng.permutation(pool_tiles)[:ntiles].astype(np.int64)
    offs = order * tile_bytes
    src = torch.from_numpy(words.view(np.int32)).cuda()
    d_offs = torch.from_numpy(offs).cuda()
    sink = torch.full((grid,), -1, dtype=torch.int32, device="cuda")
    lib = floor_lib()
    lib.ta_floor_gather.restype = ctypes.c_int
    lib.ta_floor_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    rc = lib.ta_floor_gather(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(d_offs.data_ptr()),
                             ntiles, tile_bytes, grid, threads, loads, ctypes.c_void_p(sink.data_ptr()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    got = sink.cpu().numpy().view(np.uint32)
    tiles = words.reshape(pool_tiles, tile_bytes // 4)
    per = -(-ntiles // grid)
    want = np.zeros(grid, dtype=np.uint32)
    for i in range(grid):
        sel = order[i * per:(i + 1) * per]
        if len(sel):
            want[i] = np.bitwise_xor.reduce(tiles[sel].reshape(-1))
    np.testing.assert_array_equal(got, want)
