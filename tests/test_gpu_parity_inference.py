"""GPU parity on the forward-only 2K-10s inference workload (61x90x160 = 878,400 tokens,
4 heads, 15,360 blocks per head), in the launch configuration `bench.py --workload 5
--forward-only` times.

Zone statistics, shapes and permutation are compared on every zone and slot.  The
selection is compared on a sample of query-block rows per head, which the oracle
computes row by row.  The forward is compared on sampled query blocks: stage-wise (the
oracle's permuted tensors and its selection of those blocks as input), and end to end
(the layer's own statistics, shapes and selection) where no near-tie went the other way."""

from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import NEAR, STATS_ATOL, STATS_RTOL, TOL, assert_close_out, dev, f64, i32, log
from workloads import workload
from workloads.synth import make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

WL = 5
N_ROWS = 256        # selection rows checked per head
N_QSAMPLE = 6       # forward query blocks per head


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


@functools.lru_cache(maxsize=1)
def case():
    w = workload(WL)
    log(f"[inference] generating {w.name}")
    x = make_inputs(w, seed=WL, with_grad=False)
    log("[inference] oracle stats, shapes, permutation, pooling")
    n = {k: v.float().numpy() for k, v in x.items()}          # bf16 values, exact in float32
    stats = O.zone_stats(n["v"], n["a2v"], w.grid, w.zone)
    sid, margin = O.assign_shapes(stats.astype(np.float32), list(w.cands), w.zone)
    tok = O.slot_map(w.grid, w.zone, list(w.cands), sid)
    bv = O.block_valid(tok, w.vol)
    qp, kp, vp = O.permute(n["q"], tok), O.permute(n["k"], tok), O.permute(n["v"], tok)
    del n
    qb, kb = O.pool_blocks(qp, bv, w.vol), O.pool_blocks(kp, bv, w.vol)
    scale = 1.0 / math.sqrt(w.d)
    rng = np.random.default_rng(500)
    rows = {h: np.sort(rng.choice(np.nonzero(bv[0, h] > 0)[0], size=N_ROWS, replace=False))
            for h in range(w.heads)}
    log("[inference] oracle selection of sampled rows")
    sel, near = {}, {}
    for h in range(w.heads):
        s, nr = O.select_blocks(qb[:, h:h + 1].astype(np.float32), kb[:, h:h + 1].astype(np.float32),
                                bv[:, h:h + 1], scale, w.top_p, w.k_min, w.k_max, rows=rows[h])
        sel.update({(0, h, I): v for (_, _, I), v in s.items()})
        near.update({(0, h, I): v for (_, _, I), v in nr.items()})
    qs = [(0, h, int(I)) for h in range(w.heads) for I in rows[h][:: N_ROWS // N_QSAMPLE][:N_QSAMPLE]]
    log(f"[inference] oracle forward on {len(qs)} query blocks")
    op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, scale, w.vol, blocks=qs)
    return dict(w=w, x=x, stats=stats, sid=sid, margin=margin, tok=tok, bv=bv, qp=qp, kp=kp, vp=vp,
                rows=rows, sel=sel, near=near, qs=qs, op=op, lse=lse, scale=scale)


def layer():
    from content_adaptive_block_zone_amd.pipeline import PrismLayer
    return PrismLayer.for_workload(workload(WL))


def test_inference_stats_shapes_permute():
    c = case()
    w, L = c["w"], layer()
    L.zone_stats(c["x"]["v"].cuda(), c["x"]["a2v"].cuda())
    got = f64(L.stats)
    assert (got[..., 7] == c["stats"][..., 7]).all()
    assert np.allclose(got, c["stats"], rtol=STATS_RTOL, atol=STATS_ATOL)
    L.stats.copy_(torch.from_numpy(c["stats"].astype(np.float32)))
    L.assign_shapes()
    mism = i32(L.shape_id) != c["sid"]
    log(f"[inference] shapes: {mism.sum()} mismatches, {(c['margin'] < NEAR).sum()} near-ties")
    assert not (mism & ~(c["margin"] < NEAR)).any()
    L.shape_id.copy_(torch.from_numpy(c["sid"]))
    L.permute(c["x"]["q"].cuda(), L.qp, block_valid=L.bvalid)
    assert (i32(L.bvalid) == c["bv"]).all()
    assert torch.equal(L.qp.cpu().float(), torch.from_numpy(c["qp"]).float())


def test_inference_select_sampled_rows():
    c = case()
    w, L = c["w"], layer()
    L.qp.copy_(dev(c["qp"], torch.bfloat16))
    L.kp.copy_(dev(c["kp"], torch.bfloat16))
    L.bvalid.copy_(torch.from_numpy(c["bv"]))
    L.select(from_slots=True)
    idx, cnt = i32(L.sel_idx), i32(L.sel_cnt)
    bad = near_bad = 0
    for (b, h, I), want in c["sel"].items():
        got = idx[b, h, I, :cnt[b, h, I]]
        if got.size != want.size or (got != want).any():
            if c["near"][(b, h, I)]:
                near_bad += 1
            else:
                bad += 1
    dens = np.mean([cnt[0, h].sum() / (c["bv"][0, h] > 0).sum() ** 2 for h in range(w.heads)])
    log(f"[inference] select: {bad} hard mismatches, {near_bad} near-tie mismatches of {len(c['sel'])} rows; "
        f"density {dens:.4f}")
    assert bad == 0


def test_inference_forward_sampled():
    c = case()
    w, L = c["w"], layer()
    for key, buf in (("qp", L.qp), ("kp", L.kp), ("vp", L.vp)):
        buf.copy_(dev(c[key], torch.bfloat16))
    L.bvalid.copy_(torch.from_numpy(c["bv"]))
    # the sampled blocks take the oracle's selection; other rows list nothing
    idx = np.full(tuple(L.sel_idx.shape), -1, dtype=np.int32)
    cnt = np.zeros(tuple(L.sel_cnt.shape), dtype=np.int32)
    for (b, h, I) in c["qs"]:
        s = c["sel"][(b, h, I)]
        idx[b, h, I, :s.size] = s
        cnt[b, h, I] = s.size
    L.sel_idx.copy_(torch.from_numpy(idx))
    L.sel_cnt.copy_(torch.from_numpy(cnt))
    L.attn_fwd()
    op, lse = f64(L.op), f64(L.lse)
    rs = [(b, h, slice(I * w.vol, I * w.vol + int(c["bv"][b, h, I]))) for (b, h, I) in c["qs"]]
    got = np.concatenate([op[b, h, s] for (b, h, s) in rs])
    want = np.concatenate([c["op"][b, h, s] for (b, h, s) in rs])
    assert_close_out(got, want, "bf16", f"inference fwd O' on {len(c['qs'])} query blocks")
    gl = np.concatenate([lse[b, h, s] for (b, h, s) in rs])
    wl = np.concatenate([c["lse"][b, h, s] for (b, h, s) in rs])
    assert np.abs(gl - wl).max() <= TOL["bf16"]["lse_abs"]


def test_inference_end_to_end_sampled():
    c = case()
    w, L = c["w"], layer()
    x = {k: v.cuda() for k, v in c["x"].items()}
    o = L.forward(x["q"], x["k"], x["v"], x["a2v"])
    torch.cuda.synchronize()
    if (i32(L.shape_id) != c["sid"]).any():
        pytest.skip("a near-tie zone took the other shape")
    idx, cnt = i32(L.sel_idx), i32(L.sel_cnt)
    qs = [(b, h, I) for (b, h, I) in c["qs"] if idx[b, h, I, :cnt[b, h, I]].tolist() == c["sel"][(b, h, I)].tolist()]
    assert len(qs) >= len(c["qs"]) - 2, "more than two sampled selections differ"
    tok = c["tok"]
    o_np = f64(o)
    rs = [(b, h, slice(I * w.vol, I * w.vol + int(c["bv"][b, h, I]))) for (b, h, I) in qs]
    got = np.concatenate([o_np[b, h][tok[b, h, s]] for (b, h, s) in rs])
    want = np.concatenate([c["op"][b, h, s] for (b, h, s) in rs])
    assert_close_out(got, want, "bf16", f"inference e2e O at sampled tokens ({len(qs)} blocks)")
