"""GPU parity for query rows with nothing to attend: a live block whose list is empty, and
one whose list holds only a block without valid rows.  Such rows output 0 with LSE 0 (as
padding rows do) and get no gradient; the other blocks are unaffected.  Both attention
paths: the matrix-core one (bf16, 64-row blocks, d = 128) and the generic one (float32,
16-row blocks, d = 64)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import assert_close_grad, assert_close_out, f64, log

pytestmark = pytest.mark.gpu

NB = 12


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


@pytest.mark.parametrize("kind,vol,d", [("bf16", 64, 128), ("f32", 16, 64)])
def test_nothing_to_attend(kind, vol, d):
    from content_adaptive_block_zone_amd import api
    rng = np.random.default_rng(vol)
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    bv = rng.integers(1, vol + 1, size=(1, 1, NB)).astype(np.int32)
    bv[0, 0, 2] = 0
    live = np.flatnonzero(bv[0, 0] > 0)
    sel = {(0, 0, I): np.sort(rng.choice(live, size=4, replace=False)).astype(np.int32) for I in range(NB)}
    sel[(0, 0, 0)] = np.zeros(0, np.int32)              # empty list
    sel[(0, 0, 1)] = np.array([2], np.int32)            # only a block without valid rows
    sel[(0, 0, 2)] = np.zeros(0, np.int32)              # dead block
    idx, cnt = O.selection_arrays(sel, 1, 1, NB, 6)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    rows = (np.arange(vol)[None, :] < bv[0, 0][:, None]).reshape(NB * vol, 1)
    x = {n: torch.from_numpy(rng.standard_normal((1, 1, NB * vol, d)) * rows).to(dt) for n in ("q", "k", "v", "do")}
    n = {k: v.double().numpy() for k, v in x.items()}
    scale = 1.0 / math.sqrt(d)
    op_o, lse_o = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, sel, scale, vol)
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op_o, n["do"], lse_o, bv, sel, scale, vol)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    q, k, v, do = (x[m].cuda() for m in ("q", "k", "v", "do"))
    op = torch.full_like(q, 7.0)          # every output row must be written
    lse = torch.full((1, 1, NB * vol), 7.0, dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(q, k, v, i32(bv), i32(idx), i32(cnt), vol, scale, op, lse)
    torch.cuda.synchronize()
    got_o, got_l = f64(op), f64(lse)
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    assert (got_o[0, 0, :3 * vol] == 0).all() and (got_l[0, 0, :3 * vol] == 0).all()
    assert_close_out(got_o, op_o, kind, f"{kind}: O' with empty key sets")
    lerr = float(np.abs(got_l - lse_o).max())
    log(f"  lse max-abs {lerr:.3e}")
    assert lerr <= (2e-3 if kind == "bf16" else 1e-5)
    dq, dk, dv = (torch.full_like(q, 7.0) for _ in range(3))
    ws = torch.empty(api.prism_bwd_workspace_size(1, 1, NB, vol, d, dt), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(q, k, v, torch.from_numpy(op_o).to(dt).cuda(), do,
                              torch.from_numpy(lse_o.astype(np.float32)).cuda(), i32(bv), i32(idx), i32(cnt), i32(rp),
                              i32(ri), vol, scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    assert (f64(dq)[0, 0, :3 * vol] == 0).all()
    for name, got, want in (("dQ'", dq, dq_o), ("dK'", dk, dk_o), ("dV'", dv, dv_o)):
        assert_close_grad(f64(got), want, kind, f"{kind}: {name} with empty key sets")


def test_head_with_no_live_block():
    """Two heads through the C ABI: head 1 has no live block at all.  Its selection is
    empty (counts 0, lists -1, reverse pointers 0) and its attention outputs and gradients
    are zero; head 0's selection matches the oracle's (exact except counted near-ties),
    and the attention, run on the oracle's lists, matches the oracle on both heads
    (bf16 matrix-core path)."""
    from content_adaptive_block_zone_amd import api
    vol, d, nb, k_max, top_p, k_min = 64, 128, 24, 8, 0.9, 2
    rng = np.random.default_rng(5)
    bv = np.zeros((1, 2, nb), dtype=np.int32)
    bv[0, 0] = rng.integers(1, vol + 1, size=nb)
    rows = (np.arange(vol)[None, None, :] < bv[0][:, :, None]).reshape(1, 2, nb * vol, 1)
    x = {n: torch.from_numpy(rng.standard_normal((1, 2, nb * vol, d)) * rows).to(torch.bfloat16)
         for n in ("q", "k", "v", "do")}
    n = {m: t.double().numpy() for m, t in x.items()}
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (x[m].cuda() for m in ("q", "k", "v", "do"))
    bvd = torch.from_numpy(bv).cuda()
    # selection on the GPU against the oracle's
    idx = torch.empty((1, 2, nb, k_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1, 2, nb), dtype=torch.int32, device="cuda")
    rp = torch.empty((1, 2, nb + 1), dtype=torch.int32, device="cuda")
    ri = torch.empty((1, 2, nb * k_max), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.prism_select_workspace_size(1, 2, nb, d), dtype=torch.uint8, device="cuda")
    api.prism_select_blocks(q, k, bvd, vol, scale, api.make_select_params(top_p, k_min, k_max), idx, cnt, rp, ri, ws)
    torch.cuda.synchronize()
    gc, gi, grp = (t.cpu().numpy() for t in (cnt, idx, rp))
    assert (gc[0, 1] == 0).all() and (gi[0, 1] == -1).all() and (grp[0, 1] == 0).all()
    qb = O.pool_blocks(n["q"], bv, vol).astype(np.float32)
    kb = O.pool_blocks(n["k"], bv, vol).astype(np.float32)
    sel, near = O.select_blocks(qb, kb, bv, scale, top_p, k_min, k_max)
    hard = [I for I in range(nb) if gi[0, 0, I, :gc[0, 0, I]].tolist() != sel[(0, 0, I)].tolist()
            and not near[(0, 0, I)]]
    log(f"  head 0: {len(hard)} hard selection mismatches, {sum(near.values())} near-tie rows")
    assert not hard
    # attention on the oracle's lists; the backward from the oracle's forward outputs
    idx_o, cnt_o = O.selection_arrays(sel, 1, 2, nb, k_max)
    rp_o, ri_o = O.reverse_index_sorted(idx_o, cnt_o)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    op_o, lse_o = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, sel, scale, vol)
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op_o, n["do"], lse_o, bv, sel, scale, vol)
    op = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, nb * vol), 7.0, dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(q, k, v, bvd, i32(idx_o), i32(cnt_o), vol, scale, op, lse)
    dq, dk, dv = (torch.full_like(q, 7.0) for _ in range(3))
    wsb = torch.empty(api.prism_bwd_workspace_size(1, 2, nb, vol, d), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(q, k, v, torch.from_numpy(op_o).to(torch.bfloat16).cuda(), do,
                              torch.from_numpy(lse_o.astype(np.float32)).cuda(), bvd, i32(idx_o), i32(cnt_o),
                              i32(rp_o), i32(ri_o), vol, scale, dq, dk, dv, wsb)
    torch.cuda.synchronize()
    for t in (op, lse, dq, dk, dv):
        assert (f64(t)[0, 1] == 0).all()
    assert_close_out(f64(op), op_o, "bf16", "head without live blocks: O'")
    assert float(np.abs(f64(lse) - lse_o).max()) <= 2e-3
    for name, got, want in (("dQ'", dq, dq_o), ("dK'", dk, dk_o), ("dV'", dv, dv_o)):
        assert_close_grad(f64(got), want, "bf16", f"head without live blocks: {name}")
