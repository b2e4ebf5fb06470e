"""The streaming-read reference reads every byte of its range exactly once:
the XOR of the words it writes equals the XOR of every 32-bit word read."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, 64 << 20, (256 << 20) + 48])
def test_stream_read_covers_range(nbytes):
    import torch
    from speculative_decoding_argmax_amd import mtp
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4 + 8, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(mtp.MTP_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    mtp.mtp_stream_read(buf, sink, nbytes)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words[: nbytes // 4])
