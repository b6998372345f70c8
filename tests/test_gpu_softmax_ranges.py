"""GPU parity of the attention where the online softmax's reference maximum is tested hardest:
scores that grow from one streamed key block to the next by more than 2^8 in probability
(every step moves the maximum), scores that fall (the first block holds the maximum),
and rows whose probabilities span far beyond the bf16 and fp32 ranges.  All query blocks
select every key block, in ascending order, so the streaming order is the key order; the
oracle is the same masked attention in fp64."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import assert_close_grad, assert_close_out, dev, f64, log

pytestmark = pytest.mark.gpu

NB, VOL, D = 12, 64, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


SEEDS = {"rising": 1, "falling": 2, "wide": 3}


def u_of(kind: str) -> np.ndarray:
    """The common direction of make(kind)'s inputs."""
    rng = np.random.default_rng(SEEDS[kind])
    u = rng.standard_normal(D)
    return u / np.linalg.norm(u)


def make(kind: str, seed: int):
    """Q'/K'/V'/dO' [1, 1, NB*64, D]: K rows of block J carry a common direction u with
    weight w_J, and every query row carries u, so the scores of block J are about
    w_J * |u|^2 * scale apart from noise."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    if kind == "rising":          # each block's maximum about 7 (natural log) above the last
        w = 20.0 * np.arange(NB)
    elif kind == "falling":
        w = 20.0 * np.arange(NB)[::-1]
    else:                         # "wide": one block about 106 above the rest (e^-106 < fp32's range)
        w = np.zeros(NB)
        w[NB // 2] = 300.0
    q = rng.standard_normal((NB * VOL, D)) * 0.3 + 4.0 * u
    k = rng.standard_normal((NB * VOL, D)) * 0.3 + np.repeat(w, VOL)[:, None] * u
    v = rng.standard_normal((NB * VOL, D))
    do = rng.standard_normal((NB * VOL, D))
    to = lambda a: torch.from_numpy(a.reshape(1, 1, NB * VOL, D).astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    return to(q), to(k), to(v), to(do)


@pytest.mark.parametrize("kind", ["rising", "falling", "wide"])
def test_softmax_ranges(kind):
    from content_adaptive_block_zone_amd import api
    q, k, v, do = make(kind, seed=SEEDS[kind])
    bv = np.full((1, 1, NB), VOL, dtype=np.int32)
    sel = {(0, 0, I): np.arange(NB, dtype=np.int32) for I in range(NB)}
    idx, cnt = O.selection_arrays(sel, 1, 1, NB, NB)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    scale = 1.0 / math.sqrt(D)
    n = {name: x.float().numpy().astype(np.float64) for name, x in (("q", q), ("k", k), ("v", v), ("do", do))}
    s = (n["q"][0, 0] @ n["k"][0, 0].T) * scale
    log(f"[softmax {kind}] score range per row: {float((s.max(1) - s.min(1)).mean()):.1f} "
        f"(natural log units); block maxima {[round(float(s[:, J * VOL:(J + 1) * VOL].max()), 1) for J in range(0, NB, 4)]}")
    op_o, lse_o = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, sel, scale, VOL)
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op_o, n["do"], lse_o, bv, sel, scale, VOL)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    op = torch.zeros_like(qd)
    lse = torch.zeros(qd.shape[:3], dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(qd, kd, vd, i32(bv), i32(idx), i32(cnt), VOL, scale, op, lse)
    torch.cuda.synchronize()
    assert_close_out(f64(op), op_o, "bf16", f"{kind}: O'")
    lerr = float(np.abs(f64(lse) - lse_o).max())
    log(f"  lse max-abs {lerr:.3e}")
    assert lerr <= 2e-3
    # backward from the oracle's forward outputs
    dq, dk, dv = (torch.zeros_like(qd) for _ in range(3))
    ws = torch.empty(api.prism_bwd_workspace_size(1, 1, NB, VOL, D), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(qd, kd, vd, dev(op_o, torch.bfloat16), dod, torch.from_numpy(lse_o.astype(np.float32)).cuda(),
                              i32(bv), i32(idx), i32(cnt), i32(rp), i32(ri), VOL, scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    # dQ_i = scale * sum_j dS_ij k_j: where the k_j share a large component along u and the
    # row's probability sits in one block, that component is a sum of large terms that
    # cancel, and rounding dS to bf16 (as the products take it) leaves an error of up to
    # about scale * sum_j |dS_ij| |k_j.u| * 2^-8 in it.  That component is checked against
    # that bound; the rest of dQ, and dK and dV, against the usual bar.
    uu = u_of(kind)
    s_ = (n["q"][0, 0] @ n["k"][0, 0].T) * scale
    P = np.exp(s_ - lse_o[0, 0][:, None])
    dP = n["do"][0, 0] @ n["v"][0, 0].T
    Dv = (n["do"][0, 0] * op_o[0, 0]).sum(1, keepdims=True)
    dS = P * (dP - Dv)
    bound = scale * (np.abs(dS) @ np.abs(n["k"][0, 0] @ uu)) * 2.0 ** -8
    g = f64(dq)[0, 0]
    err_u = np.abs(g @ uu - dq_o[0, 0] @ uu)
    log(f"  {kind}: dQ' along u: max error / bound {float((err_u / np.maximum(bound, 1e-30)).max()):.3f}")
    assert (err_u <= bound + 1e-6).all()
    perp = lambda x: x - np.outer(x @ uu, uu)  # noqa: E731
    assert_close_grad(perp(g), perp(dq_o[0, 0]), "bf16", f"{kind}: dQ' across u")
    for name, got, want in (("dK'", dk, dk_o), ("dV'", dv, dv_o)):
        assert_close_grad(f64(got), want, "bf16", f"{kind}: {name}")
