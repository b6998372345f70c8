"""GPU tests of the matrix-core attention's workgroup schedule: the order in which the
workgroups of a sparse launch take their blocks (within each head, longest list first, in
bins of bound // 2048 + 1 lengths, bound = k_max for the query-major order and nb for the
key-major one).  The schedule sits in the entry points' workspace: the forward's first
B*Hh*nb int32 (then its fp16 copy of V), the backward's two orders (query-major, then
key-major, each rounded up to 256 bytes) after its D buffer of B*Hh*nb*64 floats (rounded
likewise).  Checked: each order
is a permutation of the head's blocks, heads in order, lengths non-increasing by bin; and
outputs of ordered launches over ragged lists (empty lists, dead blocks, lists of every
length up to k_max) against the oracle on every block."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import assert_close_grad, assert_close_out, f64, log

pytestmark = pytest.mark.gpu

VOL, D = 64, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def a256(x: int) -> int:
    return (x + 255) // 256 * 256


def make_lists(Hh: int, nb: int, k_max: int, seed: int):
    """Ragged selections: list lengths uniform over 0..k_max, about 5 % dead blocks (which
    select nothing and are selected by nobody), ragged valid counts."""
    rng = np.random.default_rng(seed)
    bv = rng.integers(1, VOL + 1, size=(1, Hh, nb)).astype(np.int32)
    bv[rng.random((1, Hh, nb)) < 0.05] = 0
    sel = {}
    for h in range(Hh):
        live = np.flatnonzero(bv[0, h] > 0)
        for I in range(nb):
            n = 0 if bv[0, h, I] == 0 else int(rng.integers(0, min(k_max, live.size) + 1))
            sel[(0, h, I)] = np.sort(rng.choice(live, size=n, replace=False)).astype(np.int32)
    idx, cnt = O.selection_arrays(sel, 1, Hh, nb, k_max)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    return bv, sel, idx, cnt, rp, ri


def check_order(order: np.ndarray, lens: np.ndarray, bound: int, what: str):
    """order int [Hh*nb] (ids h*nb + I), lens [Hh, nb]."""
    Hh, nb = lens.shape
    width = bound // 2048 + 1
    for h in range(Hh):
        o = order[h * nb:(h + 1) * nb].astype(np.int64)
        assert np.array_equal(np.sort(o), h * nb + np.arange(nb)), f"{what}: head {h} is not a permutation"
        b = np.minimum(lens[h][o - h * nb], bound) // width
        assert (np.diff(b) <= 0).all(), f"{what}: head {h} not longest first"
    log(f"  {what}: {Hh} heads x {nb} blocks, bin width {width}: permutation, longest first")


def run(Hh, nb, k_max, seed, with_oracle: bool):
    """Forward and backward through the C-ABI; with_oracle: the oracle's forward outputs are
    computed and fed to the backward (else the kernel's own)."""
    from content_adaptive_block_zone_amd import api
    bv, sel, idx, cnt, rp, ri = make_lists(Hh, nb, k_max, seed)
    g = torch.Generator().manual_seed(seed)
    shape = (1, Hh, nb * VOL, D)
    rows = torch.from_numpy((np.arange(VOL)[None, :] < bv[0][..., None]).reshape(1, Hh, nb * VOL, 1))
    q, k, v, do = ((torch.randn(shape, generator=g) * rows).to(torch.bfloat16) for _ in range(4))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(D)
    op = torch.zeros_like(qd)
    lse = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    wsf = torch.zeros(api.prism_fwd_workspace_size(1, Hh, nb, VOL, D), dtype=torch.uint8, device="cuda")
    # the schedule first, then the fp16 copy of V (two per-head words, then the copy)
    assert wsf.numel() == a256(Hh * nb * 4) + 2 * a256(Hh * 4) + a256(Hh * nb * VOL * D * 2)
    api.prism_sparse_attn_fwd(qd, kd, vd, i32(bv), i32(idx), i32(cnt), VOL, scale, op, lse, wsf)
    out = dict(q=q, k=k, v=v, do=do, bv=bv, sel=sel, scale=scale, op=op, lse=lse)
    op_in, lse_in = op, lse
    if with_oracle:
        n = {name: x.float().numpy().astype(np.float64) for name, x in (("q", q), ("k", k), ("v", v), ("do", do))}
        out["n"] = n
        out["op_o"], out["lse_o"] = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, sel, scale, VOL)
        op_in = torch.from_numpy(out["op_o"]).to(torch.bfloat16).cuda()
        lse_in = torch.from_numpy(out["lse_o"].astype(np.float32)).cuda()
    dq, dk, dv = (torch.zeros_like(qd) for _ in range(3))
    wsb = torch.zeros(api.prism_bwd_workspace_size(1, Hh, nb, VOL, D), dtype=torch.uint8, device="cuda")
    dbuf = a256(Hh * nb * VOL * 4)
    assert wsb.numel() == dbuf + 2 * a256(Hh * nb * 4)
    api.prism_sparse_attn_bwd(qd, kd, vd, op_in, dod, lse_in, i32(bv), i32(idx), i32(cnt), i32(rp), i32(ri), VOL, scale,
                              dq, dk, dv, wsb)
    torch.cuda.synchronize()
    lens_q = np.where(bv[0] > 0, cnt[0], 0)
    lens_k = np.diff(rp[0], axis=1)
    as_i32 = lambda t, off, n: t[off:off + 4 * n].cpu().numpy().view(np.int32)  # noqa: E731
    check_order(as_i32(wsf, 0, Hh * nb), lens_q, k_max, "forward order")
    check_order(as_i32(wsb, dbuf, Hh * nb), lens_q, k_max, "backward query-major order")
    check_order(as_i32(wsb, dbuf + a256(Hh * nb * 4), Hh * nb), lens_k, nb, "backward key-major order")
    out.update(dq=dq, dk=dk, dv=dv)
    return out


def test_schedule_parity_ragged():
    Hh, nb, k_max = 2, 96, 40
    r = run(Hh, nb, k_max, seed=11, with_oracle=True)
    n, op_o, lse_o = r["n"], r["op_o"], r["lse_o"]
    assert_close_out(f64(r["op"]), op_o, "bf16", "ordered launch: O'")
    lerr = float(np.abs(f64(r["lse"]) - lse_o).max())
    log(f"  lse max-abs {lerr:.3e}")
    assert lerr <= 2e-3
    # both backward passes ran from the oracle's forward outputs
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op_o, n["do"], lse_o, r["bv"], r["sel"],
                                         r["scale"], VOL)
    for name, got, want in (("dQ'", r["dq"], dq_o), ("dK'", r["dk"], dk_o), ("dV'", r["dv"], dv_o)):
        assert_close_grad(f64(got), want, "bf16", f"ordered launch: {name}")


def test_schedule_wide_bins():
    """Lengths past 2,048, so both orders bin several lengths together (widths 2 and 3)."""
    run(1, 4500, 2100, seed=12, with_oracle=False)
