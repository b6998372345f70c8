"""GPU parity when block lists outgrow the attention kernels' LDS copy of the list: one query
block selects every one of 2,200 key blocks (its list is longer than the 2,048 entries the
forward and dQ kernels keep in LDS) and every query block selects key blocks 0 and 1 (their
reverse lists, 2,200 long, are longer than the 1,280 entries the dK/dV kernel keeps).  Those
blocks take the path that reads the list from global memory per step; the others the LDS
path.  The forward and backward are compared with the oracle on sampled blocks, with the
oracle's own forward outputs fed to both backward passes."""

from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import assert_close_grad, assert_close_out, dev, f64, log

pytestmark = pytest.mark.gpu

NB, VOL, D = 2200, 64, 128
LONG_Q = 5                        # the query block that selects every key block
SAMPLE_Q = (0, 1, LONG_Q, 1000, NB - 1)
SAMPLE_K = (0, 1, LONG_Q, 1000, NB - 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


@functools.lru_cache(maxsize=1)
def case():
    g = torch.Generator().manual_seed(77)
    shape = (1, 1, NB * VOL, D)
    q, k, v, do = (torch.randn(shape, generator=g).to(torch.bfloat16) for _ in range(4))
    bvalid = np.full((1, 1, NB), VOL, dtype=np.int32)
    bvalid[0, 0, -1] = 20                      # a ragged last block
    sel = {(0, 0, I): np.unique(np.array([0, 1, I], dtype=np.int32)) for I in range(NB)}
    sel[(0, 0, LONG_Q)] = np.arange(NB, dtype=np.int32)
    idx, cnt = O.selection_arrays(sel, 1, 1, NB, NB)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    n = {name: x.float().numpy().astype(np.float64) for name, x in (("q", q), ("k", k), ("v", v), ("do", do))}
    scale = 1.0 / math.sqrt(D)
    log("[long lists] oracle forward")
    op, lse = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bvalid, sel, scale, VOL)
    log("[long lists] oracle backward on sampled blocks")
    blocks = [(0, 0, I) for I in SAMPLE_K]
    dq, dk, dv = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op, n["do"], lse, bvalid, sel, scale, VOL,
                                   q_blocks=[(0, 0, I) for I in SAMPLE_Q], k_blocks=blocks)
    return dict(q=q, k=k, v=v, do=do, bvalid=bvalid, idx=idx, cnt=cnt, rp=rp, ri=ri, op=op, lse=lse, dq=dq, dk=dk,
                dv=dv, scale=scale)


def rows_of(x, blocks, bvalid):
    return np.concatenate([x[0, 0, I * VOL: I * VOL + int(bvalid[0, 0, I])] for I in blocks])


def test_long_lists_forward():
    from content_adaptive_block_zone_amd import api
    c = case()
    assert int(c["cnt"][0, 0, LONG_Q]) == NB and int(c["rp"][0, 0, 1] - c["rp"][0, 0, 0]) == NB
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    q, k, v = (c[n].cuda() for n in ("q", "k", "v"))
    op = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(q, k, v, i32(c["bvalid"]), i32(c["idx"]), i32(c["cnt"]), VOL, c["scale"], op, lse)
    torch.cuda.synchronize()
    got, want = rows_of(f64(op), SAMPLE_Q, c["bvalid"]), rows_of(c["op"], SAMPLE_Q, c["bvalid"])
    assert_close_out(got, want, "bf16", "long lists: O' on sampled blocks")
    lerr = np.abs(rows_of(f64(lse), SAMPLE_Q, c["bvalid"]) - rows_of(c["lse"], SAMPLE_Q, c["bvalid"])).max()
    log(f"  lse max-abs {lerr:.3e}")
    assert lerr <= 2e-3


def test_long_lists_backward():
    from content_adaptive_block_zone_amd import api
    c = case()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    q, k, v, do = (c[n].cuda() for n in ("q", "k", "v", "do"))
    op = dev(c["op"], torch.bfloat16)
    lse = torch.from_numpy(c["lse"].astype(np.float32)).cuda()
    dq, dk, dv = (torch.zeros_like(q) for _ in range(3))
    ws = torch.empty(api.prism_bwd_workspace_size(1, 1, NB, VOL, D), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(q, k, v, op, do, lse, i32(c["bvalid"]), i32(c["idx"]), i32(c["cnt"]), i32(c["rp"]),
                              i32(c["ri"]), VOL, c["scale"], dq, dk, dv, ws)
    torch.cuda.synchronize()
    bv = c["bvalid"]
    assert_close_grad(rows_of(f64(dq), SAMPLE_Q, bv), rows_of(c["dq"], SAMPLE_Q, bv), "bf16", "long lists: dQ'")
    assert_close_grad(rows_of(f64(dk), SAMPLE_K, bv), rows_of(c["dk"], SAMPLE_K, bv), "bf16", "long lists: dK'")
    assert_close_grad(rows_of(f64(dv), SAMPLE_K, bv), rows_of(c["dv"], SAMPLE_K, bv), "bf16", "long lists: dV'")
