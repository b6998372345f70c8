"""GPU parity of the scalar attention kernels, which serve every combination the
matrix-core kernels do not (those take bf16 with d = 128 and 64-row blocks): float32 and
bf16, d = 64 and 128, blocks of 16, 32 and 64 rows.  Each combination runs a small sparse
problem with ragged blocks, a dead block and a live query block with an empty list; the
forward (O and LSE) and the backward (fed the oracle's own O and LSE) are compared with the
oracle on every block, at the float32 bar of 1e-5 or the bf16 bars."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from tests.parity_util import TOL, assert_close_grad, assert_close_out, dev, f64, log

pytestmark = pytest.mark.gpu

NB = 12
COMBOS = [("f32", 128, 64), ("f32", 64, 64), ("f32", 128, 32), ("bf16", 64, 64), ("bf16", 128, 16),
          ("bf16", 128, 32), ("bf16", 64, 16)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def problem(kind, d, vol):
    dt = torch.float32 if kind == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(d * 1000 + vol)
    rng = np.random.default_rng(d * 1000 + vol)
    bv = rng.integers(1, vol + 1, size=(1, 1, NB)).astype(np.int32)
    bv[0, 0, 4] = 0                                     # a dead block
    rows = np.arange(vol)[None, :, None]
    def field():                                        # noqa: E306  zero padding rows
        x = torch.randn(NB, vol, d, generator=g).numpy() * (rows < bv[0, 0][:, None, None])
        return torch.from_numpy(x.reshape(1, 1, NB * vol, d).astype(np.float32)).to(dt)
    q, k, v, do = field(), field(), field(), field()
    live = np.nonzero(bv[0, 0] > 0)[0]
    sel = {}
    for I in range(NB):
        if bv[0, 0, I] == 0:
            sel[(0, 0, I)] = np.zeros(0, dtype=np.int32)
        elif I == 7:                                    # a live query block that attends to nothing
            sel[(0, 0, I)] = np.zeros(0, dtype=np.int32)
        else:
            sel[(0, 0, I)] = np.sort(rng.choice(live, size=int(rng.integers(1, 7)), replace=False)).astype(np.int32)
    return dt, q, k, v, do, bv, sel


@pytest.mark.parametrize("kind,d,vol", COMBOS, ids=[f"{k}_d{d}_vol{v}" for k, d, v in COMBOS])
def test_generic_attention_forward_and_backward(kind, d, vol):
    from content_adaptive_block_zone_amd import api
    dt, q, k, v, do, bv, sel = problem(kind, d, vol)
    scale = 1.0 / math.sqrt(d)
    n = {name: f64(x) for name, x in (("q", q), ("k", k), ("v", v), ("do", do))}
    log(f"[generic {kind} d={d} vol={vol}] oracle")
    op_o, lse_o = O.sparse_attn_fwd(n["q"], n["k"], n["v"], bv, sel, scale, vol)
    blocks = [(0, 0, I) for I in range(NB)]
    dq_o, dk_o, dv_o = O.sparse_attn_bwd(n["q"], n["k"], n["v"], op_o, n["do"], lse_o, bv, sel, scale, vol,
                                         q_blocks=blocks, k_blocks=blocks)
    km = max(1, max(len(s) for s in sel.values()))
    idx, cnt = O.selection_arrays(sel, 1, 1, NB, km)
    rp, ri = O.reverse_index_sorted(idx, cnt)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()  # noqa: E731
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    op = torch.zeros_like(qg)
    lse = torch.zeros(qg.shape[:3], dtype=torch.float32, device="cuda")
    api.prism_sparse_attn_fwd(qg, kg, vg, i32(bv), i32(idx), i32(cnt), vol, scale, op, lse)
    dq, dk, dv = (torch.zeros_like(qg) for _ in range(3))
    ws = torch.empty(api.prism_bwd_workspace_size(1, 1, NB, vol, d, dt), dtype=torch.uint8, device="cuda")
    api.prism_sparse_attn_bwd(qg, kg, vg, dev(op_o, dt), dog, torch.from_numpy(lse_o.astype(np.float32)).cuda(),
                              i32(bv), i32(idx), i32(cnt), i32(rp), i32(ri), vol, scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    valid = np.concatenate([np.arange(I * vol, I * vol + int(bv[0, 0, I])) for I in range(NB)])
    assert_close_out(f64(op)[0, 0][valid], op_o[0, 0][valid], kind, f"{kind} d={d} vol={vol}: O'")
    lerr = float(np.abs(f64(lse)[0, 0][valid] - lse_o[0, 0][valid]).max())
    log(f"  LSE max-abs {lerr:.3e}")
    assert lerr <= TOL[kind]["lse_abs"]
    q7 = np.arange(7 * vol, 7 * vol + int(bv[0, 0, 7]))
    assert np.all(f64(op)[0, 0][q7] == 0.0), "a query block with an empty list must give zeros"
    for name, got, want in (("dQ'", dq, dq_o), ("dK'", dk, dk_o), ("dV'", dv, dv_o)):
        assert_close_grad(f64(got)[0, 0][valid], want[0, 0][valid], kind, f"{kind} d={d} vol={vol}: {name}")
