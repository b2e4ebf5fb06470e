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


@pytest.mark.parametrize("wgs,iters,same", [(1, 8, False), (3, 5, False), (256, 16, False),
                                            (256, 4, True), (1024, 1, True)])
def test_probe_atomic_runs_every_chain(wgs, iters, same):
    """The atomic round-trip probe runs each workgroup's chain in full: every
    chain adds iters to its own word (all chains together to words[0] when
    they share it), leaves every other word alone, and reports a positive
    tick count."""
    import torch
    from speculative_decoding_argmax_amd import mtp
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    words = torch.zeros(64 * wgs + 64, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(wgs, dtype=torch.int64, device="cuda")
    mtp.mtp_probe_atomic(words, ticks, wgs, iters, same)
    torch.cuda.synchronize()
    w = words.cpu().numpy()
    want = np.zeros_like(w)
    if same:
        want[0] = wgs * iters
    else:
        want[0:64 * wgs:64] = iters
    assert np.array_equal(w, want)
    t = ticks.cpu().numpy() & ((1 << 63) - 1)
    assert (t > 0).all()
