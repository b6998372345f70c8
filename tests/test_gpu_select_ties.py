"""GPU parity of the block selection when block probabilities tie exactly.  Sorting with
ties toward the lower key-block index makes the kept set unique even when the cut falls
inside a run of equal probabilities; the kernel then ranks the equal keys in block order
(wave ballots and prefix counts) instead of taking every block at the cut's key, a path
that rows of distinct random scores almost never reach.

Pooled features are chosen so that every score is exact in float32 whatever the order of
summation (key entries multiples of 1/8 in [-1/4, 1/4], query entries multiples of 1/8 up
to 4, d = 64, scale 1/8: every partial sum is a multiple of 1/64 below 64): equal key
features then give bitwise-equal probabilities on both sides.  Head 0 has zero query
features (every row uniform over the live blocks: the kept set is the lowest live indices,
a closed form); head 1 has key features shared by runs of five consecutive blocks.  Two
key blocks are dead.  Each (top_p, k_min, k_max) setting exercises Top-p cuts, the Top-k
clamp from above and below, and top_p = 1, and every row whose Top-p decision is not
within the near-tie margin of p must match the oracle exactly."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import i32, log

pytestmark = pytest.mark.gpu

NB, D, SCALE = 100, 64, 0.125
DEAD = (7, 50)
RUN = 5  # key blocks sharing one feature vector in head 1
SETTINGS = [(0.555, 2, 90), (0.555, 2, 40), (0.555, 70, 90), (0.3, 1, 90), (1.0, 2, 90)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def features():
    rng = np.random.default_rng(2024)
    q = np.zeros((1, 2, NB, D), dtype=np.float32)
    k = np.zeros((1, 2, NB, D), dtype=np.float32)
    q[0, 0] = 0.0
    k[0, 0] = rng.integers(-2, 3, size=(NB, D)) / 8.0
    q[0, 1] = rng.integers(-2, 3, size=(NB, D)) / 8.0 * rng.integers(1, 17, size=(NB, 1))  # flat to peaked rows
    groups = rng.integers(-2, 3, size=(NB // RUN + 1, D)) / 8.0
    k[0, 1] = groups[np.arange(NB) // RUN]
    bv = np.full((1, 2, NB), 64, dtype=np.int32)
    bv[0, :, list(DEAD)] = 0
    return q, k, bv


def robust_rows(q, k, bv, top_p):
    """Rows whose Top-p count is not decided within the near-tie margin of p (float64
    cumulative sums of the oracle's sorted probabilities)."""
    ok = {}
    for h in range(2):
        live = np.nonzero(bv[0, h] > 0)[0]
        for I in live:
            logits = (k[0, h, live] @ q[0, h, I]) * SCALE
            e = np.exp(logits.astype(np.float64) - logits.max())
            P = np.sort(e / e.sum())[::-1]
            C = np.cumsum(P)
            ok[(0, h, int(I))] = top_p >= 1 or bool(np.min(np.abs(C - top_p)) >= O.NEAR_TIE)
    return ok


@pytest.mark.parametrize("top_p,k_min,k_max", SETTINGS)
def test_selection_with_exact_ties(top_p, k_min, k_max):
    from content_adaptive_block_zone_amd import api
    q, k, bv = features()
    want, _ = O.select_blocks_all(q, k, bv, SCALE, top_p, k_min, k_max)
    live0 = np.nonzero(bv[0, 0] > 0)[0]
    # head 0, closed form: uniform rows keep the n lowest live indices
    n_p = len(live0) if top_p >= 1 else int(np.floor(top_p * len(live0))) + 1
    n0 = min(max(n_p, k_min), k_max, len(live0))
    for I in live0:
        assert np.array_equal(want[(0, 0, int(I))], live0[:n0]), ("oracle, uniform row", int(I))

    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()  # noqa: E731
    qb, kb, bvt = dev(q, torch.float32), dev(k, torch.float32), dev(bv, torch.int32)
    idx = torch.empty(1, 2, NB, k_max, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, 2, NB, dtype=torch.int32, device="cuda")
    rp = torch.empty(1, 2, NB + 1, dtype=torch.int32, device="cuda")
    ri = torch.empty(1, 2, NB * k_max, dtype=torch.int32, device="cuda")
    ws = torch.empty(api.prism_select_pooled_workspace_size(1, 2, NB), dtype=torch.uint8, device="cuda")
    api.prism_select_blocks_pooled(qb, kb, bvt, SCALE, api.make_select_params(top_p, k_min, k_max), idx, cnt, rp, ri,
                                   ws)
    torch.cuda.synchronize()
    gi, gc = i32(idx), i32(cnt)

    robust = robust_rows(q, k, bv, top_p)
    compared = split = 0
    for (b, h, I), s in want.items():
        got = gi[b, h, I, :gc[b, h, I]]
        if bv[b, h, I] == 0:
            assert gc[b, h, I] == 0, ("dead query block selects", h, I)
            continue
        if not robust[(b, h, I)]:
            continue
        assert np.array_equal(got, s), (top_p, k_min, k_max, h, I, got.tolist(), s.tolist())
        compared += 1
        # does the cut fall inside a run of equal probabilities?
        live = np.nonzero(bv[0, h] > 0)[0]
        logits = (k[0, h, live] @ q[0, h, I]) * SCALE
        kept = np.isin(live, s)
        if kept.any() and (~kept).any() and logits[kept].min() == logits[~kept].max():
            split += 1
    log(f"[ties] top_p {top_p} k {k_min}..{k_max}: {compared} rows compared exactly, {split} with the cut inside "
        f"a run of equal probabilities")
    assert compared >= 150
    assert split >= len(live0) - 1  # every uniform row of head 0 at least
    # the reverse index lists, for every key block, the query blocks that kept it, ascending
    for h in range(2):
        m = np.arange(k_max)[None, :] < gc[0, h][:, None]
        I = np.broadcast_to(np.arange(NB)[:, None], (NB, k_max))[m]
        J = gi[0, h][m]
        o = np.lexsort((I, J))
        r = i32(rp)[0, h]
        assert r[0] == 0 and r[-1] == m.sum() and (np.diff(r) == np.bincount(J, minlength=NB)).all()
        assert (i32(ri)[0, h, :r[-1]] == I[o]).all()
