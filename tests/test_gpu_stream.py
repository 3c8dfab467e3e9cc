"""The stream-read reference (kascade_stream_read), a measurement helper:
every 16-byte word of the buffer is read once, so the XOR it folds into the
sink equals NumPy's XOR of the same 32-bit words, at sizes that end inside a
load step, a workgroup's step and the grid's step."""
import sys

import numpy as np
import pytest
import torch

from long_context_anchor_amd import kascade as K

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, 10 * 2**20 + 16, 3 * 2**27 + 4096])
def test_stream_read_xor(nbytes):
    print("stream read", nbytes, flush=True)
    sys.stdout.flush()
    g = torch.Generator(device="cuda").manual_seed(nbytes % 1000)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64,
                        device="cuda").to(torch.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.check(K.kascade_stream_read(src, nbytes, sink), "stream_read")
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    # a second call folds the same value in again: the sink returns to zero
    K.check(K.kascade_stream_read(src, nbytes, sink), "stream_read")
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy()[0]) == 0
