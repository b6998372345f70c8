"""GPU parity with block volumes mixed per zone (C_64 + C_128 + C_256 chosen by the
activity thresholds tau_128 / tau_256; Tables 9-11): statistics with the zone activity,
the multi-volume assignment, the permutation with per-zone volumes, the block heads, the
tile lists, and the whole layer forward and backward against the oracle's mixed chain, on
one head of the 720p-like workload (zones of varying anisotropy)."""

from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import (NEAR, STATS_ATOL, STATS_RTOL, assert_close_grad, assert_close_out,
                               check_reverse_is_transpose, dev, f64, i32, log, selection_from_arrays)
from workloads import CANDS_128, CANDS_256, workload
from workloads.synth import make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

WL, HEADS = 2, 1
TAUS = (O.TAU_128, O.TAU_256)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def cands():
    return list(workload(WL).cands) + CANDS_128 + CANDS_256


@functools.lru_cache(maxsize=1)
def inputs():
    w = workload(WL)
    x = make_inputs(w, seed=WL, heads=range(HEADS))
    return w, x, {k: v.float().numpy().astype(np.float64) for k, v in x.items()}


@functools.lru_cache(maxsize=1)
def oracle():
    w, _, n = inputs()
    log("[mixed] oracle chain")
    f = O.prism_forward(n["q"], n["k"], n["v"], n["a2v"], w.grid, w.zone, cands(), w.top_p, w.k_min, w.k_max,
                        mixed=TAUS)
    f["vact"] = O.zone_activity(n["v"], w.grid, w.zone)
    log("[mixed] oracle backward")
    f.update(O.prism_backward(f, n["do"]))
    return f


def layer():
    from content_adaptive_block_zone_amd.pipeline import PrismLayer
    return PrismLayer.for_workload(workload(WL), heads=HEADS, cands=cands(), mixed=TAUS)


def test_mixed_stages():
    w, x, n = inputs()
    f = oracle()
    L = layer()
    L.zone_stats(x["v"].cuda(), x["a2v"].cuda())
    assert np.allclose(f64(L.stats), f["stats"], rtol=STATS_RTOL, atol=STATS_ATOL)
    assert np.allclose(f64(L.vact), f["vact"], rtol=STATS_RTOL, atol=STATS_ATOL)
    # assignment from the oracle's statistics
    L.stats.copy_(torch.from_numpy(f["stats"].astype(np.float32)))
    L.vact.copy_(torch.from_numpy(f["vact"].astype(np.float32)))
    L.assign_shapes()
    sid, margin = O.assign_shapes_multi(f["stats"].astype(np.float32), f["vact"], cands(), w.zone)
    mism = i32(L.shape_id) != sid
    vols = np.array([np.prod(cands()[i]) for i in sid.ravel()])
    log(f"[mixed] zones by volume 64/128/256: {[(vols == v).sum() for v in (64, 128, 256)]}; "
        f"{mism.sum()} mismatches, {(margin < NEAR).sum()} near-ties")
    assert not (mism & ~(margin < NEAR)).any()
    assert len(set(vols.tolist())) >= 2, "the workload should exercise more than one block volume"
    # permutation and block heads with the oracle's shapes
    L.shape_id.copy_(torch.from_numpy(f["shape_id"]))
    L.permute_qkv(x["q"].cuda(), x["k"].cuda(), x["v"].cuda())
    assert torch.equal(L.qp.cpu().float(), torch.from_numpy(f["qp"]).float())
    assert torch.equal(L.vp.cpu().float(), torch.from_numpy(f["vp"]).float())
    assert (i32(L.unit_valid) == O.block_valid(f["tok"], 64)).all()
    assert (i32(L.bvalid) == f["bvalid"]).all()


def test_mixed_tile_lists():
    f = oracle()
    L = layer()
    L.qp.copy_(dev(f["qp"], torch.bfloat16))
    L.kp.copy_(dev(f["kp"], torch.bfloat16))
    L.bvalid.copy_(torch.from_numpy(f["bvalid"]))
    L.unit_valid.copy_(torch.from_numpy(O.block_valid(f["tok"], 64)))
    L.select(from_slots=True)
    bv, idx, cnt = i32(L.bvalid), i32(L.sel_idx), i32(L.sel_cnt)
    live = lambda nn: (int(nn) + 63) // 64  # noqa: E731
    tidx, tcnt = i32(L.tile_idx), i32(L.tile_cnt)
    want_cnt = np.zeros_like(tcnt)
    for h in range(HEADS):
        for I in np.nonzero(bv[0, h] > 0)[0]:
            lst = [int(J) + v for J in idx[0, h, I, :cnt[0, h, I]] for v in range(live(bv[0, h, J]))]
            for u in range(live(bv[0, h, I])):
                want_cnt[0, h, I + u] = len(lst)
                assert tidx[0, h, I + u, :len(lst)].tolist() == lst
    assert (tcnt == want_cnt).all()
    assert (tidx[np.arange(tidx.shape[-1]) >= tcnt[..., None]] == -1).all()
    check_reverse_is_transpose(tidx, tcnt, i32(L.tile_rev_ptr), i32(L.tile_rev_idx))


def test_mixed_attention_stagewise():
    """The oracle's permuted tensors, block heads and selection (with its reverse index)
    through the mixed tile expansion and the attention, forward and backward."""
    from content_adaptive_block_zone_amd import api
    w, _, _ = inputs()
    f = oracle()
    L = layer()
    bf = torch.bfloat16
    for key, buf in (("qp", L.qp), ("kp", L.kp), ("vp", L.vp)):
        buf.copy_(dev(f[key], bf))
    L.bvalid.copy_(torch.from_numpy(f["bvalid"]))
    L.unit_valid.copy_(torch.from_numpy(O.block_valid(f["tok"], 64)))
    idx, cnt = O.selection_arrays(f["sel"], w.B, HEADS, f["bvalid"].shape[-1], w.k_max)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    for key, buf in ((idx, L.sel_idx), (cnt, L.sel_cnt), (rp, L.rev_ptr), (ri, L.rev_idx)):
        buf.copy_(torch.from_numpy(np.ascontiguousarray(key).astype(np.int32)))
    api.prism_blocks_to_tiles_mixed(L.bvalid, L.sel_idx, L.sel_cnt, L.rev_ptr, L.rev_idx, L.max_units, L.tile_idx,
                                    L.tile_cnt, L.tile_rev_ptr, L.tile_rev_idx, L.ws_tiles)
    L.attn_fwd()
    valid = f["tok"] >= 0
    assert_close_out(f64(L.op)[valid], f["op"][valid], "bf16", "mixed O'")
    assert np.abs(f64(L.lse)[valid] - f["lse"][valid]).max() <= 2e-3
    # backward from the oracle's O', LSE and dO'
    L.op.copy_(dev(f["op"], bf))
    L.lse.copy_(torch.from_numpy(f["lse"].astype(np.float32)))
    g = L._grads()
    g["dop"].copy_(dev(f["dop"], bf))
    L.attn_bwd()
    want = O.sparse_attn_bwd(f["qp"], f["kp"], f["vp"], f64(L.op), f["dop"], f64(L.lse), f["bvalid"], f["sel"],
                             f["scale"], 64)
    for nm, buf, wi in (("dQ'", g["dqp"], want[0]), ("dK'", g["dkp"], want[1]), ("dV'", g["dvp"], want[2])):
        assert_close_grad(f64(buf)[valid], wi[valid], "bf16", f"mixed {nm}")


def test_mixed_layer_end_to_end():
    """The whole layer on the GPU against the oracle chain: shapes and selections equal
    except counted near-ties; O compared on every query block whose selection is the
    oracle's (a block's output depends on its own list only); gradients when no selection
    differs."""
    w, x, _ = inputs()
    f = oracle()
    L = layer()
    o = L.forward(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["a2v"].cuda())
    dq, dk, dv = L.backward(x["do"].cuda())
    torch.cuda.synchronize()
    sid = i32(L.shape_id)
    assert not ((sid != f["shape_id"]) & ~(f["shape_margin"] < NEAR)).any()
    if (sid != f["shape_id"]).any():
        pytest.skip("a near-tie zone took the other shape or volume")
    gsel = selection_from_arrays(i32(L.sel_idx), i32(L.sel_cnt))
    diff = [k for k in gsel if gsel[k].tolist() != f["sel"][k].tolist()]
    assert all(f["sel_near"][k] for k in diff)
    log(f"[mixed] {len(diff)} near-tie selection differences")
    bv, tok = f["bvalid"], f["tok"]
    same = [(b, h, I) for (b, h, I) in gsel if bv[b, h, I] > 0 and (b, h, I) not in set(diff)]
    rows = [(b, h, slice(I * 64, I * 64 + int(bv[b, h, I]))) for (b, h, I) in same]
    o_np = f64(o)
    got = np.concatenate([o_np[b, h][tok[b, h, s]] for (b, h, s) in rows])
    want = np.concatenate([f["op"][b, h, s] for (b, h, s) in rows])
    assert_close_out(got, want, "bf16", f"mixed e2e O on {len(same)} blocks")
    if diff:
        return
    for nm, got_, want_ in (("dQ", dq, f["dq"]), ("dK", dk, f["dk"]), ("dV", dv, f["dv"])):
        assert_close_grad(f64(got_), want_, "bf16", f"mixed e2e {nm}")
