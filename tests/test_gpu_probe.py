"""The streaming-read probe (mk_stream_read) reads every byte it is given:
each thread's sink word is the XOR of the 32-bit words of the 16-byte words
it visited (grid-stride order), checked exactly against numpy."""
import ctypes

import numpy as np
import pytest
import torch

from persistent_interpreter_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 1000, 2048 * 256 * 8 + 12345])
def test_stream_read_folds_every_word(n16):
    L = B.lib()
    words = L.mk_stream_read_sink_words()
    rng = np.random.default_rng(n16)
    host = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((words,), -1, dtype=torch.int32, device="cuda")
    print(f"case: stream read of {n16} 16-byte words", flush=True)
    rc = L.mk_stream_read(ctypes.c_void_p(buf.data_ptr()), n16 * 16, ctypes.c_void_p(sink.data_ptr()),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == B.MK_OK
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    fold = np.bitwise_xor.reduce(host, axis=1)
    want = np.zeros(words, np.uint32)
    pad = (-n16) % words
    want[:] = np.bitwise_xor.reduce(np.concatenate([fold, np.zeros(pad, np.uint32)]).reshape(-1, words), axis=0)
    assert np.array_equal(got, want)
