"""Read-stream probe on the GPU: every 32-bit word of the buffer is read
exactly once (a word skipped or read twice changes the XOR of all words)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_248_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 4 * 1023, (64 << 20) // 4 + 4 * 12345])
def test_stream_read_reads_every_word_once(words):
    rng = np.random.default_rng(words)
    host = rng.integers(-2**31, 2**31, size=words, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_stream_read(src, sink, magic=int(want) ^ 1)        # no match: nothing written
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    pa.pa_stream_read(src, sink, magic=int(want))
    torch.cuda.synchronize()
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want
