"""The streaming-read diagnostic reads every byte exactly once: the XOR of its
per-workgroup words equals the XOR of the whole buffer, for slice counts that
divide the buffer, leave a ragged last slice, or exceed the number of words."""
import numpy as np
import pytest

from tests.gpu_helpers import note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


@pytest.mark.parametrize("nbytes,words", [(16, 1), (16, 7), (4096 * 16, 64), (1000 * 16 + 16, 37),
                                          (3 * (1 << 20), 8192)])
def test_stream_read_checksum(exq, nbytes, words):
    rng = np.random.default_rng(nbytes + words)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((words,), -1, dtype=torch.int32, device="cuda")
    note("stream read %d bytes over %d slices" % (nbytes, words))
    exq.exq_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), words)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_bad_arguments(exq):
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for args in ((buf.data_ptr(), 0, sink.data_ptr(), 4), (buf.data_ptr(), 24, sink.data_ptr(), 4),
                 (buf.data_ptr() + 4, 64, sink.data_ptr(), 4), (buf.data_ptr(), 64, sink.data_ptr(), 0)):
        with pytest.raises(exq.ExqError):
            exq.exq_stream_read(*args)
