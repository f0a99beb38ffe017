"""GPU: the streaming-read yardstick reads every 32-bit word of its buffer
exactly once (an odd number of times): the XOR it leaves equals the XOR of
all words computed on the host, for sizes that end inside a 16 KiB chunk and
for several grid sizes."""
import numpy as np
import pytest
import torch

from paged_kv_cache_101_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16384, 16400, 3 * 16384 + 48, 5 << 20])
@pytest.mark.parametrize("wg", [0, 1, 7])
def test_stream_read_xor(gpu, nbytes, wg):
    rng = np.random.default_rng(nbytes + wg)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(gpu)
    sink = torch.zeros(1, dtype=torch.int32, device=gpu)
    B.pkv_stream_read(buf, sink, wg)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
