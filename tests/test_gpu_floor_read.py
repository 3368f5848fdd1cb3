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
