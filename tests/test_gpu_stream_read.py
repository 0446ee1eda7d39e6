"""swa_stream_read, the measuring aid for the streaming HBM read rate: every
32-bit word of the buffer is read exactly once, so the XOR of the sink (one
word per wave, every wave writes) equals the XOR of the buffer's words, bit
for bit.  Sizes: one 16-byte unit, ragged tails of the per-workgroup shares,
and a buffer of 96 MiB."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 16 * 2048 * 256 * 8 + 48, 96 << 20])
def test_stream_read_touches_every_word_once(nbytes):
    from decode_attention_fixed_amd import binding as B
    words = np.random.default_rng(nbytes % 1000).integers(0, 2**32, size=nbytes // 4,
                                                          dtype=np.uint32)
    x = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((B.STREAM_READ_SINK_BYTES // 4,), 0x5A5A5A5A, dtype=torch.int32,
                      device="cuda")
    B.stream_read(x, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
