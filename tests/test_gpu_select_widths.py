"""GPU parity of the block selection at every row width the library dispatches on: its
five workgroup shapes (up to 2,048 / 4,096 / 8,192 / 16,384 / 32,768 key blocks, the
largest width accepted).  Synthetic rows: each query
block's pooled feature has its own magnitude, so that some rows are flat (the Top-k clamp
decides) and some are peaked (Top-p decides); about 5 % of the blocks are dead and the
valid counts are ragged.  Sampled rows are compared with the oracle's selection (exact,
except for rows the oracle marks as near-ties); the reverse index is checked to be the
transpose of the whole selection."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import f64, i32, log

pytestmark = pytest.mark.gpu

VOL, D = 64, 32
TOP_P, K_MIN, K_MAX = 0.85, 8, 384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def make_case(nb: int, seed: int):
    """Q'/K' [1, 1, nb*64, D] bf16 with padding rows zero, and the valid counts."""
    rng = np.random.default_rng(seed)
    bv = rng.integers(10, VOL + 1, size=nb).astype(np.int32)
    bv[rng.random(nb) < 0.05] = 0
    amp_q = rng.uniform(0.0, 40.0, size=nb)
    dirs_q = rng.standard_normal((nb, D))
    dirs_k = rng.standard_normal((nb, D))
    rows = np.arange(VOL)[None, :, None]
    noise = lambda: rng.standard_normal((nb, VOL, D)).astype(np.float32) * 0.5  # noqa: E731
    q = (amp_q[:, None, None] * dirs_q[:, None, :] / math.sqrt(D) + noise()) * (rows < bv[:, None, None])
    k = (dirs_k[:, None, :] + noise()) * (rows < bv[:, None, None])
    to_t = lambda a: torch.from_numpy(a.reshape(1, 1, nb * VOL, D).astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    return to_t(q), to_t(k), bv.reshape(1, 1, nb)


def reverse_is_transpose(idx, cnt, rp, ri):
    """Vectorised form of the transpose property (one head)."""
    nb, km = idx.shape
    m = np.arange(km)[None, :] < cnt[:, None]
    I = np.broadcast_to(np.arange(nb)[:, None], (nb, km))[m]
    J = idx[m]
    o = np.lexsort((I, J))
    assert rp[0] == 0 and (np.diff(rp) >= 0).all() and rp[-1] == m.sum()
    assert (np.diff(rp) == np.bincount(J, minlength=nb)).all()
    assert (ri[:rp[-1]] == I[o]).all()


@pytest.mark.parametrize("nb", [1500, 3000, 6000, 9000, 16384, 20000, 32768])
def test_select_width(nb):
    from content_adaptive_block_zone_amd import api
    q, k, bv = make_case(nb, seed=nb)
    qd, kd = q.cuda(), k.cuda()
    bvd = torch.from_numpy(bv).cuda()
    idx = torch.empty((1, 1, nb, K_MAX), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1, 1, nb), dtype=torch.int32, device="cuda")
    rp = torch.empty((1, 1, nb + 1), dtype=torch.int32, device="cuda")
    ri = torch.empty((1, 1, nb * K_MAX), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.prism_select_workspace_size(1, 1, nb, D), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    api.prism_select_blocks(qd, kd, bvd, VOL, scale, api.make_select_params(TOP_P, K_MIN, K_MAX), idx, cnt, rp, ri, ws)
    torch.cuda.synchronize()
    gidx, gcnt = i32(idx)[0, 0], i32(cnt)[0, 0]
    qb = O.pool_blocks(f64(q), bv, VOL).astype(np.float32)
    kb = O.pool_blocks(f64(k), bv, VOL).astype(np.float32)
    rows = sorted(set(np.random.default_rng(nb + 1).choice(nb, size=40, replace=False).tolist()) | {0, nb - 1})
    sel, near = O.select_blocks(qb, kb, bv, scale, TOP_P, K_MIN, K_MAX, rows=rows)
    hard = [I for I in rows if gidx[I, :gcnt[I]].tolist() != sel[(0, 0, I)].tolist() and not near[(0, 0, I)]]
    n_topk = sum(int(gcnt[I]) == K_MAX for I in rows)
    log(f"[select nb={nb}] {len(hard)} hard mismatches of {len(rows)} rows; {n_topk} rows at k_max; "
        f"{sum(near.values())} near-tie rows")
    assert not hard
    assert (gidx[np.arange(K_MAX)[None, :] >= gcnt[:, None]] == -1).all()
    assert (gcnt[bv[0, 0] == 0] == 0).all()
    reverse_is_transpose(gidx, gcnt, i32(rp)[0, 0], i32(ri)[0, 0])
