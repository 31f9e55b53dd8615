"""GPU check of the streaming-read measurement kernel (mi_hbm_stream_read):
every thread's folded word equals the XOR of exactly the 16-byte units it
owns (so the timed reads cover the buffer once and nothing else), and bad
arguments are refused (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()


@pytest.mark.parametrize("units,wgs", [(4096, 4), (4096 + 7, 4), (1 << 16, 64), (300, 3)])
def test_stream_read_folds_each_owned_unit_once(units, wgs):
    rng = np.random.default_rng(units + wgs)
    host = rng.integers(0, 2 ** 32, size=(units, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.full((wgs * 256,), -1, dtype=torch.int32, device=DEV)
    mk.mi_hbm_stream_read(src, units * 16, sink, wgs)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    per = units // wgs
    words = np.bitwise_xor.reduce(host, axis=1)          # fold of each 16-byte unit
    want = np.zeros(wgs * 256, np.uint32)
    for w in range(wgs):
        chunk = words[w * per:(w + 1) * per]
        for t in range(256):
            want[w * 256 + t] = np.bitwise_xor.reduce(chunk[t::256]) if t < per else 0
    assert np.array_equal(got, want)


def test_stream_read_argument_errors():
    src = torch.zeros(1024, dtype=torch.int32, device=DEV)
    sink = torch.zeros(256, dtype=torch.int32, device=DEV)
    for args in [(None, 4096, sink, 1), (src, 4096, None, 1), (src, 4095, sink, 1),
                 (src, 4096, sink, 0), (src, 4096, sink, 257), (src, 4096, sink, 70000)]:
        with pytest.raises(mk.MikvError):
            mk.mi_hbm_stream_read(*args)
    off = src.view(torch.uint8)[4:]                       # misaligned by 4 bytes
    with pytest.raises(mk.MikvError):
        mk.mi_hbm_stream_read(off, 16, sink, 1)
