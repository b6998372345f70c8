"""Find the scalar Q gain that puts a workload's mean selected density in its target band.

Test infrastructure (uses only the oracle and the input generator).  The selection
density of a head is sum(cnt) / (live query blocks * live key blocks).  Pooled block
means are linear in Q, so the gain scales every pooled score; the script bisects the
gain on the oracle's selection of a row sample and prints it.  The printed value is
copied into the workload table (workloads/configs.py, q_gain) by hand.

    python -m oracle.calibrate_gain 4
"""

from __future__ import annotations

import math
import sys

import numpy as np

from oracle import prism_oracle as O


def density_for_gain(gain, heads, scale, w):
    """Mean over heads of the sampled rows' selected fraction of live key blocks."""
    tot = 0.0
    for (qbar, kbar, bv, rows) in heads:
        sel, _ = O.select_blocks(qbar * gain, kbar, bv, scale, w.top_p, w.k_min, w.k_max, rows=rows)
        tot += np.mean([s.size for s in sel.values()]) / (bv[0, 0] > 0).sum()
    return tot / len(heads)


def calibrate(i: int, n_rows: int = 96, seed: int = 0):
    from workloads import workload
    from workloads.synth import make_inputs
    w = workload(i)
    rng = np.random.default_rng(seed)
    heads = []
    for h in range(w.heads):                 # one head at a time keeps host memory bounded
        x = make_inputs(w, seed=i, heads=[h], q_gain=1.0, with_grad=False)
        n = {k: v.float().numpy().astype(np.float64) for k, v in x.items()}
        del x
        stats = O.zone_stats(n["v"], n["a2v"], w.grid, w.zone)
        sid, _ = O.assign_shapes(stats.astype(np.float32), list(w.cands), w.zone)
        tok = O.slot_map(w.grid, w.zone, list(w.cands), sid)
        bv = O.block_valid(tok, w.vol)
        qbar = O.pool_blocks(O.permute(n["q"], tok), bv, w.vol).astype(np.float32)
        kbar = O.pool_blocks(O.permute(n["k"], tok), bv, w.vol).astype(np.float32)
        del n
        rows = np.sort(rng.choice(np.nonzero(bv[0, 0] > 0)[0], size=n_rows, replace=False))
        heads.append((qbar, kbar, bv, rows))
        print(f"head {h} pooled", flush=True)
    scale = 1.0 / math.sqrt(w.d)
    lo_t, hi_t = w.density_target
    target = 0.5 * (lo_t + hi_t)
    lo, hi = 0.25, 64.0                      # density falls as the gain grows
    for _ in range(30):
        mid = math.sqrt(lo * hi)
        dens = density_for_gain(mid, heads, scale, w)
        print(f"gain {mid:.5f}: density {dens:.4f}", flush=True)
        if abs(dens - target) < 0.002:
            break
        if dens > target:
            lo = mid
        else:
            hi = mid
    return mid, dens


if __name__ == "__main__":
    g, d = calibrate(int(sys.argv[1]))
    print(f"q_gain = {g:.4f} (density {d:.4f})")
