"""Read-stream probe on the GPU: every 32-bit word of the buffer is read
exactly once (a word skipped or read twice changes the XOR of all words)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,sink_words", [(4, 1), (4 * 1023, 7), (4 * 1023, 4096),
                                              ((64 << 20) // 4 + 4 * 12345, 1 << 16)])
def test_stream_read_reads_every_word_once(words, sink_words):
    rng = np.random.default_rng(words + sink_words)
    host = rng.integers(-2**31, 2**31, size=words, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    sink = torch.zeros(sink_words, dtype=torch.int32, device="cuda")
    pa.pa_stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host.view(np.uint32))


@pytest.mark.parametrize("nbytes,wgs", [(16, 0), (16 * 1023, 1), (16 * 12345, 64), (16 * 12345, 0),
                                        ((64 << 20) + 16 * 777, 0), ((64 << 20) + 16 * 3, 128)])
def test_stream_copy_copies_every_byte_once(nbytes, wgs):
    """The copy probe reproduces the source bit for bit and writes nothing
    past the destination range (guard words on both sides)."""
    g = torch.Generator(device="cpu").manual_seed(nbytes + wgs)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    buf = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = buf[32:32 + nbytes]
    pa.pa_stream_copy(src, dst, wgs)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert (buf[:32] == 0xA5).all() and (buf[32 + nbytes:] == 0xA5).all()
