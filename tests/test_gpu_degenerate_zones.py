"""GPU parity of the zone statistics and the shape assignment on degenerate zones, which
the synthetic fields of the workloads never contain: a constant zone, zones that vary
along one axis only (t, h or w), a zone whose features and audio-to-video output are all
zero, and one random zone beside them.  The statistics must match the oracle (the float32
tolerances of the other stage tests); the shapes the GPU derives from its own statistics
must match the oracle's from its statistics, and, for the first four zones, the closed
forms the oracle is pinned to (no variation -> 4x4x4; variation along t only -> 1x8x8,
along h only -> 4x2x8, along w only -> 4x8x2: the block is thinnest along the varying
axis).  Both the bf16 path (d = 128) and the float32 path (d = 64) run."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import NEAR, STATS_ATOL, STATS_RTOL, f64, i32, log
from workloads.configs import CANDS_64

pytestmark = pytest.mark.gpu

GRID, ZONE = (4, 32, 48), (4, 16, 16)   # 1 x 2 x 3 zones
EXPECT = {0: (4, 4, 4), 1: (1, 8, 8), 2: (4, 2, 8), 3: (4, 8, 2)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def fields(d: int):
    """V and the A2V output [1, 1, N, d]; zone z = 3 * (h // 16) + w // 16."""
    T, H, W = GRID
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = (a.reshape(-1, 1).astype(np.float64) for a in (t, h, w))
    c = np.arange(d)[None, :] * 0.37
    z = (3 * (h // 16) + w // 16).ravel().astype(int)
    hl, wl = h % 16, w % 16
    V = np.zeros((T * H * W, d))
    V[z == 0] = 0.5
    V[z == 1] = np.sin(2.1 * t + c)[z == 1]
    V[z == 2] = np.sin(1.3 * hl + c)[z == 2]
    V[z == 3] = np.sin(1.3 * wl + c)[z == 3]
    V[z == 5] = np.random.default_rng(11).standard_normal(((z == 5).sum(), d))
    A = np.zeros((T * H * W, d))
    A[z != 4, 0] = 1.0
    return V[None, None], A[None, None]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16_d128", "f32_d64"])
def test_degenerate_zone_statistics_and_shapes(dtype, d):
    from content_adaptive_block_zone_amd import api
    V, A = fields(d)
    # the oracle sees the values the kernel reads (rounded to the storage type)
    Vt, At = (torch.from_numpy(x).to(dtype) for x in (V, A))
    Vr, Ar = (x.float().numpy().astype(np.float64) for x in (Vt, At))
    want_stats = O.zone_stats(Vr, Ar, GRID, ZONE)
    want_sid, want_margin = O.assign_shapes(want_stats, CANDS_64, ZONE, O.ShapeParams(), np.float32)
    assert [CANDS_64[i] for i in want_sid[0, 0, :4]] == [EXPECT[z] for z in range(4)]

    g = api.make_grid(GRID, ZONE)
    s = api.make_shapes(CANDS_64)
    nZ = api.prism_num_zones(g)
    stats = torch.empty(1, 1, nZ, 8, dtype=torch.float32, device="cuda")
    sid = torch.empty(1, 1, nZ, dtype=torch.int32, device="cuda")
    margin = torch.empty(1, 1, nZ, dtype=torch.float32, device="cuda")
    api.prism_zone_stats(Vt.cuda(), At.cuda(), g, stats)
    api.prism_assign_shapes(stats, g, s, api.make_shape_params(), sid, margin)
    torch.cuda.synchronize()
    got_stats, got_sid = f64(stats), i32(sid)
    log(f"[degenerate {dtype}] stats max abs diff {np.abs(got_stats - want_stats).max():.3e}; shapes "
        f"{[CANDS_64[i] for i in got_sid[0, 0]]} (oracle {[CANDS_64[i] for i in want_sid[0, 0]]})")
    assert np.isfinite(got_stats).all()
    assert (got_stats[..., 7] == want_stats[..., 7]).all()
    assert np.allclose(got_stats, want_stats, rtol=STATS_RTOL, atol=STATS_ATOL)
    for z in range(4):
        assert CANDS_64[got_sid[0, 0, z]] == EXPECT[z], (z, CANDS_64[got_sid[0, 0, z]])
    differ = got_sid != want_sid
    assert not (differ & ~(want_margin < NEAR)).any(), "a zone that is not a near-tie took another shape"
