"""GPU parity of the sparse attention across softmax scales.  The kernels fold the scale
into base-2 exponents (scale * log2 e) and give query rows past a block's end an LSE of
+inf in the backward, so the sign and size of the scale reach every step of the softmax.
Each scale below is compared with the oracle on every block of a small problem with a
ragged last block: the forward (O and LSE), then the backward with the oracle's own forward
outputs fed to it.  Scales: the usual 1/sqrt(d), its negative, 2^-59 and 2^-70 (scores all
but equal: nearly uniform weights) and 0 (uniform attention, zero dQ and dK)."""

from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import TOL, assert_close_grad, assert_close_out, dev, f64, log

pytestmark = pytest.mark.gpu

NB, VOL, D = 48, 64, 128
RAGGED = 13  # valid rows of the last block
SCALES = (1.0 / math.sqrt(D), -1.0 / math.sqrt(D), 2.0 ** -59, 2.0 ** -70, 0.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


@functools.lru_cache(maxsize=1)
def problem():
    g = torch.Generator().manual_seed(404)
    shape = (1, 1, NB * VOL, D)
    q, k, v, do = (torch.randn(shape, generator=g).to(torch.bfloat16) for _ in range(4))
    bvalid = np.full((1, 1, NB), VOL, dtype=np.int32)
    bvalid[0, 0, -1] = RAGGED
    rng = np.random.default_rng(404)
    sel = {}
    for I in range(NB):
        pick = rng.choice(NB, size=10, replace=False)
        sel[(0, 0, I)] = np.unique(np.concatenate([pick, [I, NB - 1]]).astype(np.int32))
    idx, cnt = O.selection_arrays(sel, 1, 1, NB, int(max(len(s) for s in sel.values())))
    rp, ri = O.reverse_index_sorted(idx, cnt)
    n = {name: x.float().numpy().astype(np.float64) for name, x in (("q", q), ("k", k), ("v", v), ("do", do))}
    return dict(q=q, k=k, v=v, do=do, n=n, bvalid=bvalid, sel=sel, idx=idx, cnt=cnt, rp=rp, ri=ri)


IDS = ["inv_sqrt_d", "neg_inv_sqrt_d", "2^-59", "2^-70", "zero"]


def valid_rows(bv):
    return np.concatenate([np.arange(I * VOL, I * VOL + int(bv[0, 0, I])) for I in range(NB)])


@pytest.mark.parametrize("scale", SCALES, ids=IDS)
def test_forward_across_scales(scale):
    from content_adaptive_block_zone_amd import api
    c = problem()
    n, bv = c["n"], c["bvalid"]
    log(f"[scale paths] scale {scale:.3e}: oracle forward")
    op_o, lse_o = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, c["sel"], scale, VOL)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    q, k, v = (c[name].cuda() for name in ("q", "k", "v"))
    op = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(q, k, v, i32(bv), i32(c["idx"]), i32(c["cnt"]), VOL, scale, op, lse)
    torch.cuda.synchronize()
    rows = valid_rows(bv)
    assert_close_out(f64(op)[0, 0][rows], op_o[0, 0][rows], "bf16", f"scale {scale:.3e}: O'")
    lerr = float(np.abs(f64(lse)[0, 0][rows] - lse_o[0, 0][rows]).max())
    log(f"  LSE max-abs {lerr:.3e}")
    assert lerr <= TOL["bf16"]["lse_abs"]


@pytest.mark.parametrize("scale", SCALES, ids=IDS)
def test_backward_across_scales(scale):
    from content_adaptive_block_zone_amd import api
    c = problem()
    n, bv = c["n"], c["bvalid"]
    log(f"[scale paths] scale {scale:.3e}: oracle forward and backward")
    op, lse = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, c["sel"], scale, VOL)
    blocks = [(0, 0, I) for I in range(NB)]
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op, n["do"], lse, bv, c["sel"], scale, VOL,
                                         q_blocks=blocks, k_blocks=blocks)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    q, k, v, do = (c[name].cuda() for name in ("q", "k", "v", "do"))
    dq, dk, dv = (torch.zeros_like(q) for _ in range(3))
    ws = torch.empty(api.prism_bwd_workspace_size(1, 1, NB, VOL, D), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(q, k, v, dev(op, torch.bfloat16), do, torch.from_numpy(lse.astype(np.float32)).cuda(),
                              i32(bv), i32(c["idx"]), i32(c["cnt"]), i32(c["rp"]), i32(c["ri"]), VOL, scale,
                              dq, dk, dv, ws)
    torch.cuda.synchronize()
    valid = valid_rows(bv)
    pad = np.setdiff1d(np.arange(NB * VOL), valid)
    for name, got, want in (("dQ'", dq, dq_o), ("dK'", dk, dk_o), ("dV'", dv, dv_o)):
        g64 = f64(got)[0, 0]
        assert np.isfinite(g64).all(), f"{name}: non-finite values at scale {scale}"
        assert np.all(g64[pad] == 0.0), f"{name}: padding rows not zero at scale {scale}"
        if scale == 0.0 and name != "dV'":
            # dS is multiplied by the scale: exactly zero on both sides
            assert np.all(g64[valid] == 0.0) and np.all(want[0, 0][valid] == 0.0), name
            continue
        assert_close_grad(g64[valid], want[0, 0][valid], "bf16", f"scale {scale:.3e}: {name}")
