"""The streaming-read reference kernel (pgqa_stream_read): it reads every 16-byte
word exactly once (the XOR of all sink words equals the XOR of the buffer's
32-bit words, computed on the host), at grid sizes whose last round is ragged,
and rejects bad arguments on the host."""
import ctypes

import numpy as np
import pytest
import torch

import paged_gqa_decode_head_amd as pg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words16, grid", [(1, 1), (7, 1), (1000, 3), (65537, 0), (3 * 256 * 2 + 5, 3),
                                           (2_000_003, 768)])
def test_every_word_read_once(words16, grid):
    rng = np.random.default_rng(words16)
    host = rng.integers(0, 2**32, size=words16 * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    g = grid or 3 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((g * 256,), -1, dtype=torch.int32, device="cuda")
    pg.bind_stream_read(src, sink, grid)()
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_bad_arguments_rejected():
    lib = pg.lib()
    src = torch.zeros(1024, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.pgqa_stream_read(p(src), 4096, p(sink), 1024, 1, None) == pg.PGQA_OK
    torch.cuda.synchronize()
    assert lib.pgqa_stream_read(p(src), 4095, p(sink), 1024, 1, None) != pg.PGQA_OK  # not a multiple of 16
    assert lib.pgqa_stream_read(p(src), 0, p(sink), 1024, 1, None) != pg.PGQA_OK
    assert lib.pgqa_stream_read(p(src), 4096, p(sink), 1024, 2, None) != pg.PGQA_OK  # sink too small
    assert lib.pgqa_stream_read(p(src), 4096, p(sink), 1024, 70000, None) != pg.PGQA_OK
    host = torch.zeros(1024, dtype=torch.int32)
    assert lib.pgqa_stream_read(p(host), 4096, p(sink), 1024, 1, None) != pg.PGQA_OK  # host memory
