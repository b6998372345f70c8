"""Helpers shared by the GPU parity tests: tolerances, comparisons, oracle runs."""

from __future__ import annotations

import functools
import math
import os
import sys

import numpy as np
import torch

from oracle import prism_oracle as O
from workloads import workload
from workloads.synth import make_inputs

# Tolerances.  bf16: outputs max-abs 2e-2 and rel-L2 1e-2, gradients rel-L2 2e-2;
# float32: 1e-5.  Zone statistics are float32 sums of at most a zone's worth of pair
# terms (<= 4096): their rounding stays far below rel 1e-4 / abs 1e-5.
TOL = {
    "f32": dict(out_abs=1e-5, out_rel=1e-5, grad_rel=1e-5, lse_abs=1e-5),
    "bf16": dict(out_abs=2e-2, out_rel=1e-2, grad_rel=2e-2, lse_abs=2e-3),
}
STATS_RTOL, STATS_ATOL = 1e-4, 1e-5
NEAR = O.NEAR_TIE


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def i32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def dev(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / max(nb, 1e-30)


def torch_dtype(w) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


@functools.lru_cache(maxsize=2)
def inputs(i: int, seed: int = None):
    w = workload(i)
    return w, make_inputs(w, seed=i if seed is None else seed)


def np_inputs(x):
    return {k: f64(v) for k, v in x.items()}


def selection_from_arrays(idx: np.ndarray, cnt: np.ndarray):
    B, Hh, nb, _ = idx.shape
    return {(b, h, I): idx[b, h, I, :cnt[b, h, I]].astype(np.int32)
            for b in range(B) for h in range(Hh) for I in range(nb)}


def assert_close_out(got: np.ndarray, want: np.ndarray, kind: str, what: str):
    t = TOL[kind]
    mx = float(np.abs(got - want).max()) if got.size else 0.0
    rl = rel_l2(got, want)
    log(f"  {what}: max-abs {mx:.3e} rel-L2 {rl:.3e}")
    assert mx <= t["out_abs"], f"{what}: max-abs {mx} > {t['out_abs']}"
    assert rl <= t["out_rel"], f"{what}: rel-L2 {rl} > {t['out_rel']}"


def assert_close_grad(got: np.ndarray, want: np.ndarray, kind: str, what: str):
    rl = rel_l2(got, want)
    log(f"  {what}: rel-L2 {rl:.3e}")
    assert rl <= TOL[kind]["grad_rel"], f"{what}: rel-L2 {rl} > {TOL[kind]['grad_rel']}"


def check_reverse_is_transpose(idx, cnt, rev_ptr, rev_idx):
    """rev_* must list, for each key block, exactly the query blocks whose ELL row holds
    it, ascending (a property check written out here, independent of the oracle)."""
    B, Hh, nb, km = idx.shape
    for b in range(B):
        for h in range(Hh):
            rp = rev_ptr[b, h]
            assert rp[0] == 0 and (np.diff(rp) >= 0).all()
            assert rp[-1] == cnt[b, h].sum()
            pairs = [(int(J), I) for I in range(nb) for J in idx[b, h, I, :cnt[b, h, I]]]
            pairs.sort()
            lst = rev_idx[b, h, :rp[-1]]
            assert [I for (_, I) in pairs] == lst.tolist()
            counts = np.bincount(np.array([J for (J, _) in pairs], dtype=np.int64), minlength=nb)
            assert (np.diff(rp) == counts).all()


def oracle_fwd_blocks(qp, kp, vp, bv, sel, scale, vol, blocks, threads=None):
    """The oracle's sparse forward on the listed query blocks, the blocks split over a
    thread pool (one BLAS thread per call; the oracle's arithmetic is unchanged, each block
    is computed by one O.sparse_attn_fwd call exactly as in a serial run).  Returns O' and
    LSE of full shape with the listed blocks' rows filled, zeros elsewhere."""
    from concurrent.futures import ThreadPoolExecutor

    import threadpoolctl
    blocks = sorted(blocks)
    # widen once here (bf16 and float32 values are exact in float64), so that the calls
    # below do not each convert the whole tensors
    qp, kp, vp = (np.asarray(a, dtype=np.float64) for a in (qp, kp, vp))
    nt = max(1, min(threads or os.cpu_count() or 1, 16, len(blocks) or 1))
    chunks = [blocks[i::nt] for i in range(nt)]
    B, Hh, Np, _ = qp.shape
    O_ = np.zeros((B, Hh, Np, vp.shape[-1]))
    L_ = np.zeros((B, Hh, Np))

    def run(chunk):
        o, l = O.sparse_attn_fwd(qp, kp, vp, bv, sel, scale, vol, blocks=chunk)
        return chunk, o, l

    with threadpoolctl.threadpool_limits(1):
        with ThreadPoolExecutor(nt) as ex:
            for chunk, o, l in ex.map(run, chunks):
                for (b, h, I) in chunk:
                    rs = slice(I * vol, (I + 1) * vol)
                    O_[b, h, rs] = o[b, h, rs]
                    L_[b, h, rs] = l[b, h, rs]
    return O_, L_
