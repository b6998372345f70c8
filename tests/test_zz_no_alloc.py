"""The allocation-free backward (prism_sparse_attn_bwd_noalloc) against the allocating
one (prism_sparse_attn_bwd) through the C ABI: the same kernels on the library's static
scratch instead of a caller workspace.  Both are deterministic (no atomics; the
workgroup schedule only reorders independent blocks), so their outputs must be equal
bit for bit.  Three calls in a row share the one scratch array: the 480p-like layer with
three heads, then the same with one head (smaller, stale scratch from the first call),
then the tiny float32 workload (the scalar kernels)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.parity_util import log
from workloads import workload
from workloads.synth import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_adaptive_block_zone_amd import _lib
    _lib.load()


def layer_inputs(i, heads):
    """A layer run forward on the GPU: its permuted tensors, selection and LSE are the
    backward's inputs; dO' is a seeded draw."""
    from content_adaptive_block_zone_amd.pipeline import PrismLayer
    w = workload(i)
    x = make_inputs(w, seed=i, heads=range(heads))
    L = PrismLayer.for_workload(w, heads=heads, device="cuda")
    L.forward(*(x[n].cuda() for n in ("q", "k", "v", "a2v")))
    g = L._grads()
    g["dop"].copy_(torch.from_numpy(np.random.default_rng(7).standard_normal(tuple(g["dop"].shape)))
                   .to(g["dop"].dtype))
    torch.cuda.synchronize()
    return L


def both(L):
    from content_adaptive_block_zone_amd import api
    g = L._grads()
    bv, idx, cnt, rp, ri, vol = L._attn_lists()
    ref = [torch.full_like(g["dqp"], float("nan")) for _ in range(3)]
    api.prism_sparse_attn_bwd(L.qp, L.kp, L.vp, L.op, g["dop"], L.lse, bv, idx, cnt, rp, ri, vol, L.scale, *ref,
                              L.ws_bwd)
    got = [torch.full_like(g["dqp"], float("nan")) for _ in range(3)]
    api.prism_sparse_attn_bwd_noalloc(L.qp, L.kp, L.vp, L.op, g["dop"], L.lse, bv, idx, cnt, rp, ri, vol, L.scale,
                                      *got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("i,heads", [(1, 3), (1, 1), (0, 2)])
def test_noalloc_backward_equals_allocating_backward(i, heads):
    L = layer_inputs(i, heads)
    ref, got = both(L)
    for name, a, b in zip(("dQ'", "dK'", "dV'"), ref, got):
        assert not torch.isnan(a).any(), name
        assert torch.equal(a, b), f"workload {i}, {heads} heads: {name} differs"
    log(f"[noalloc] workload {i} with {heads} heads: dQ', dK', dV' bitwise equal "
        f"({L.B * L.Hh * L.Npad} rows, {L.ws_bwd.numel()} scratch bytes)")


def test_noalloc_rejects_sizes_past_its_scratch():
    import ctypes

    from content_adaptive_block_zone_amd import _lib
    lib = _lib.load()
    P = ctypes.c_void_p(256)          # never dereferenced: the size check fails first
    nb = (1 << 17) + 1                # 2^23 + 64 padded rows: D alone needs more than 32 MiB
    st = lib.prism_sparse_attn_bwd_noalloc(P, P, P, P, P, P, _lib.PRISM_BF16, P, P, P, 8, P, P, 1, 1, nb, 64, 128,
                                           0.1, P, P, P, None, None)
    assert st == _lib.PRISM_ERR_SHAPE, lib.prism_last_error()
    assert b"static scratch" in lib.prism_last_error()
