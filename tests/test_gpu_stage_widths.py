"""GPU parity of the zone statistics, the shape assignment and the permutation with pooling
at the feature widths the other tests do not use: d = 32 and 256 (the statistics kernel
takes d in {32, 64, 128, 256}; the permutation moves any multiple of 16 bytes per row and
pools rows of up to 4 KB), in bf16 and float32, on a grid whose far zones are ragged along
all three axes, two heads, with random shape ids mixed in.  Statistics must match the
oracle within the float32 tolerances, shapes exactly (except counted near-ties), the
permuted tensor bit for bit and the block means within 1e-5."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import NEAR, STATS_ATOL, STATS_RTOL, f64, i32, log
from workloads.configs import CANDS_64

pytestmark = pytest.mark.gpu

GRID, ZONE = (6, 21, 37), (4, 16, 16)   # 2 x 2 x 3 zones, the far ones ragged in t, h and w


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 32), (torch.bfloat16, 256), (torch.float32, 32),
                                     (torch.float32, 256)], ids=["bf16_d32", "bf16_d256", "f32_d32", "f32_d256"])
def test_stats_shapes_permute_pool_at_width(dtype, d):
    from content_adaptive_block_zone_amd import api
    T, H, W = GRID
    N = T * H * W
    g = torch.Generator().manual_seed(d)
    # smooth-ish fields (a random walk along w) so that the zones differ in their statistics
    v = torch.randn(1, 2, T, H, W, d, generator=g).cumsum(dim=4).reshape(1, 2, N, d).to(dtype)
    a2v = torch.randn(1, 2, N, d, generator=g).to(dtype)
    q = torch.randn(1, 2, N, d, generator=g).to(dtype)
    vr, ar, qr = f64(v), f64(a2v), f64(q)

    want_stats = O.zone_stats(vr, ar, GRID, ZONE)
    want_sid, want_margin = O.assign_shapes(want_stats, CANDS_64, ZONE, O.ShapeParams(), np.float32)
    grid = api.make_grid(GRID, ZONE)
    shapes = api.make_shapes(CANDS_64)
    nZ, nb = api.prism_num_zones(grid), api.prism_num_blocks(grid, shapes)
    stats = torch.empty(1, 2, nZ, 8, dtype=torch.float32, device="cuda")
    sid = torch.empty(1, 2, nZ, dtype=torch.int32, device="cuda")
    api.prism_zone_stats(v.cuda(), a2v.cuda(), grid, stats)
    api.prism_assign_shapes(stats, grid, shapes, api.make_shape_params(), sid)
    torch.cuda.synchronize()
    got_stats, got_sid = f64(stats), i32(sid)
    log(f"[widths {dtype} d={d}] stats max abs diff {np.abs(got_stats - want_stats).max():.3e}")
    assert (got_stats[..., 7] == want_stats[..., 7]).all()
    assert np.allclose(got_stats, want_stats, rtol=STATS_RTOL, atol=STATS_ATOL)
    assert not ((got_sid != want_sid) & ~(want_margin < NEAR)).any()

    # permutation with pooling on the oracle's shapes, half of the zones given random shapes
    rng = np.random.default_rng(d)
    ids = want_sid.copy()
    mask = rng.random(ids.shape) < 0.5
    ids[mask] = rng.integers(0, len(CANDS_64), size=int(mask.sum()))
    tok = O.slot_map(GRID, ZONE, CANDS_64, ids)
    bv_o = O.block_valid(tok, 64)
    yp_o = O.permute(qr, tok)
    pool_o = O.pool_blocks(yp_o, bv_o, 64)
    y = torch.empty(1, 2, nb * 64, d, dtype=dtype, device="cuda")
    pooled = torch.empty(1, 2, nb, d, dtype=torch.float32, device="cuda")
    bv = torch.empty(1, 2, nb, dtype=torch.int32, device="cuda")
    api.prism_permute_pool(q.cuda(), y, grid, shapes, torch.from_numpy(ids.astype(np.int32)).cuda(), pooled, bv)
    torch.cuda.synchronize()
    assert (i32(bv) == bv_o).all()
    assert (f64(y) == yp_o).all()
    err = float(np.abs(f64(pooled) - pool_o).max())
    log(f"  permuted rows bit-exact; pooled means max-abs {err:.3e}")
    assert err <= 1e-5
    back = torch.empty_like(q).cuda()
    api.prism_permute(y, back, grid, shapes, torch.from_numpy(ids.astype(np.int32)).cuda(), inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), q)
