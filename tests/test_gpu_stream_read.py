"""The measurement-only streaming-read kernel reads every word exactly once.

It is the practical read ceiling that the decode's HBM roofline is read
against, so the test checks that it really reads the whole buffer: the XOR of
its per-workgroup sink equals the XOR of all 32-bit words of the buffer.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import alibi_linear_position_amd as alibi
    return alibi.load_library()


@pytest.mark.parametrize("words,workgroups", [(4, 1), (4 * 1000 + 4, 7), (1 << 20, 64), ((1 << 22) + 12, 4096)])
def test_stream_read_sees_every_word(lib, words, workgroups):
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(workgroups, dtype=torch.int32, device="cuda")
    P = ctypes.c_void_p
    f = lib.alibi_debug_stream_read
    f.argtypes = [P, ctypes.c_longlong, P, ctypes.c_int, P]
    st = torch.cuda.current_stream().cuda_stream
    assert f(buf.data_ptr(), words * 4, sink.data_ptr(), workgroups, st) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    print(f"[parity] stream read {words} words over {workgroups} workgroups: {got:#010x} vs {want:#010x}", flush=True)
    assert got == want
