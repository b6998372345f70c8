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


def test_tile_gather_copies_owner_rows_and_runs_every_list():
    """The forward's tile traffic without arithmetic: its one visible output is each owner
    block's valid Q rows copied to O (padding rows untouched), over lists of every length
    from none to all blocks, on the forward's own launch and schedule."""
    from content_adaptive_block_zone_amd import api
    nb, vol, d = 40, 64, 128
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(1, 2, nb * vol, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    rng = np.random.default_rng(5)
    bv = rng.integers(1, vol + 1, size=(1, 2, nb)).astype(np.int32)
    bv[0, 1, 3] = 0                                   # a dead owner block
    cnt = np.array([[[I % (nb + 1) for I in range(nb)] for _ in range(2)]], dtype=np.int32)
    idx = np.full((1, 2, nb, nb), -1, dtype=np.int32)
    for h in range(2):
        for I in range(nb):
            idx[0, h, I, :cnt[0, h, I]] = np.sort(rng.choice(nb, size=cnt[0, h, I], replace=False))
    sentinel = torch.full_like(q, 7.0)
    o = sentinel.clone()
    ws = torch.empty(api.prism_fwd_workspace_size(1, 2, nb, vol, d), dtype=torch.uint8, device="cuda")
    print("[measure] tile gather", flush=True)
    t = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    api.prism_bench_tile_gather(q, k, v, t(bv), t(idx), t(cnt), vol, o, ws)
    torch.cuda.synchronize()
    rows = torch.arange(vol, device="cuda")
    for h in range(2):
        for I in range(nb):
            sl = slice(I * vol, (I + 1) * vol)
            valid = rows < int(bv[0, h, I])
            assert torch.equal(o[0, h, sl][valid], q[0, h, sl][valid]), (h, I)
            assert torch.equal(o[0, h, sl][~valid], sentinel[0, h, sl][~valid]), (h, I)
