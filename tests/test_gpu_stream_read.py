"""The streaming-read measurement kernel reads every byte once.

Its reduction (XOR of all 32-bit words, folded into sink[0]) is compared with
the host's: a pass that skipped or repeated a word gives another value.
"""
import numpy as np
import pytest

import non_causal_block_amd as nb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 32768, 32768 * 3 + 16 * 77, (1 << 20) + 16, 64 << 20])
def test_stream_read_touches_every_word(nbytes):
    import torch

    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    want = int(np.bitwise_xor.reduce(host))
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    assert nb.dflash_stream_read(dev, nbytes, sink, stream.cuda_stream) == nb.DFLASH_OK
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert int(got[0]) == want, (nbytes, hex(int(got[0])), hex(want))
