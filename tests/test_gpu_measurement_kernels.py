"""GPU checks of the measurement kernels that the bench line's ceilings come from: the
contiguous read (every byte of both buffers is read: the XOR of the per-wavefront checksums
equals the XOR of all 32-bit words, including sizes that end in a partial grid stride) and
the matrix-core loop (its clock readings are positive and its rate is below the part's
published dense bf16 peak)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


# 16 bytes (one load), 16,000 bytes (less than one grid stride), 8 MiB + 48 bytes (the
# paired loop and a remainder), 96 MiB (many strides)
@pytest.mark.parametrize("nbytes", [16, 16_000, 8 * 1024 * 1024 + 48, 96 * 1024 * 1024])
def test_stream_read_touches_every_word(nbytes):
    from content_adaptive_block_zone_amd import api
    g = torch.Generator().manual_seed(nbytes)
    n = nbytes // 4
    a = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int64, generator=g).to(torch.int32)
    b = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int64, generator=g).to(torch.int32)
    sink = torch.zeros(api.PRISM_BENCH_STREAM_SINK, dtype=torch.int32, device="cuda")
    print(f"[measure] stream read of 2 x {nbytes} bytes", flush=True)
    api.prism_bench_stream_read(a.cuda(), b.cuda(), sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(np.concatenate([a.numpy(), b.numpy()]).view(np.uint32))
    assert got == want


def test_mfma_peak_reports_a_clock_and_a_rate_below_the_peak():
    import bench
    print("[measure] matrix-core loop", flush=True)
    tf, mhz = bench.mfma_peak(torch.device("cuda:0"), reps=1)
    assert 500.0 < mhz < 3000.0
    assert 100.0 < tf <= bench.MI355X_BF16_DENSE_TFLOPS * 1.02
