"""The benchmark's streaming-ceiling probe (q4_stream_read, through the C
ABI): it reads every byte once -- the XOR of its sink words equals the XOR
of the 32-bit words of the range -- and rejects bad arguments before
launching anything."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402

P = ctypes.c_void_p


@pytest.mark.parametrize("nbytes", [16, 48, 4096, 16 * 2048 * 256 * 4 + 16 * 37, 100_000_000 // 16 * 16])
def test_stream_read_reads_every_word(nbytes):
    rng = np.random.default_rng(9000 + nbytes % 1000)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    words = int(q4.lib.q4_stream_read_sink_words())
    sink = torch.full((words,), -1, dtype=torch.int32, device=DEV)
    st = q4.lib.q4_stream_read(P(src.data_ptr()), nbytes, P(sink.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == 0
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # the binding gives the same
    s2 = q4.q4_stream_read(src)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(s2.cpu().numpy().view(np.uint32)) == got


def test_stream_read_argument_errors():
    src = torch.zeros(64, dtype=torch.int32, device=DEV)
    sink = torch.zeros(int(q4.lib.q4_stream_read_sink_words()), dtype=torch.int32, device=DEV)
    L = q4.lib
    assert L.q4_stream_read(P(src.data_ptr()), 0, P(sink.data_ptr()), None) == 2      # size
    assert L.q4_stream_read(P(src.data_ptr()), 40, P(sink.data_ptr()), None) == 2     # not 16k
    assert L.q4_stream_read(None, 64, P(sink.data_ptr()), None) == 1                   # NULL
    assert L.q4_stream_read(P(src.data_ptr()), 64, None, None) == 1
    assert L.q4_stream_read(P(src.data_ptr() + 4), 64, P(sink.data_ptr()), None) == 3  # align
    torch.cuda.synchronize()
