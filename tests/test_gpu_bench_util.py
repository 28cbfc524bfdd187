"""The measurement-support kernels (streaming read, cache-flushing fill) read
and write exactly what they claim: checked bit for bit against the host."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 77, 96 << 20])
def test_stream_read_touches_every_word(gpu_lib, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.bench_stream_read(src, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == expect


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 33 << 20])
def test_fill_writes_the_pattern(gpu_lib, nbytes):
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    gpu_lib.bench_fill(dst, 0x5A5A1234)
    torch.cuda.synchronize()
    assert bool((dst == 0x5A5A1234).all())
