"""The streaming-read probe (a measurement helper in the same library): it
must read every word it is given, exactly once, or its rate means nothing.
Each workgroup's XOR of the words it read, combined, must equal the XOR of
the whole buffer."""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (16 * 1001, 3), (1 << 20, 64), ((1 << 24) + 48, 1024)])
def test_probe_reads_every_word_once(dev, nbytes, blocks):
    rng = np.random.Generator(np.random.PCG64(140))
    words = rng.integers(0, 2 ** 32, size=nbytes // 4 + 8, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
    sg.sgmv_stream_probe(src, sink, nbytes)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words[: nbytes // 4])


def test_probe_argument_errors(dev):
    src = torch.zeros(64, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for nbytes in (0, 24):
        with pytest.raises(sg.SGMVError):
            sg.sgmv_stream_probe(src, sink, nbytes)
