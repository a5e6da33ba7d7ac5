"""GPU test of the streaming-read diagnostic (pa_read_stream): every workgroup's XOR of the 32-bit
words of its slice equals numpy's, so every byte of the buffer was read once."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_cache_gqa_amd as pa  # noqa: E402


@pytest.mark.parametrize("grid,words_per_wg", [(1, 20), (3, 4000), (512, 8192), (4096, 1028)])
def test_read_stream_xor_per_slice(grid, words_per_wg):
    # words_per_wg: 32-bit words of each slice (a multiple of 4: whole 16-byte loads); 20 and 1028
    # leave a partial pass of the 4 x 256-load stride, 4000 several passes
    rng = np.random.default_rng(1009 + grid)
    host = rng.integers(-2**31, 2**31 - 1, size=grid * words_per_wg, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = pa.read_stream(buf, grid)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32).reshape(grid, words_per_wg), axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
