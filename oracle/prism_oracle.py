"""Plain, slow CPU oracle of Prism's block-sparse video self-attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import or run this module.  The
product path (the HIP library and its Python binding) never calls it, and this module
shares no code, table or helper with that path.

Sources.  The method is described by the Prism paper ("Prism: Dynamic Sparse Attention
for Native 2K Joint Video-Audio Generation Model Training"), through its abstract,
the caption of Figure 2 (architecture), Table 7 and its caption (Top-k / Top-p),
Tables 9 and 10 with their captions (the per-channel variance of Eq. 1, the audio
coupling gate, the audio directional variance, the power law b*_d ~ g_d^-alpha and the
quantization of Eq. 7), and Table 11 with its caption (shape notation b_T b_H b_W, equal
volumes within a candidate set).  The pages print neither Eq. 1 nor Eq. 7 nor the
method section; where they are silent this file takes one plain reading, stated at
the step that needs it, and the readings are listed together in the design notes.

Precision.  Continuous quantities are computed in float64 on the input values as
given (bf16 inputs are exact in float64).  The two steps where floating point decides
an integer -- the argmin over candidate shapes and the Top-k/Top-p cut -- run in the
kernel's precision (float32) by default, so that both sides take the decision in the
same precision; pins may run them in float64.

Parity: every function here is pinned by the CPU tests (closed forms, brute force,
textbook special cases, finite differences); none is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Shape = Tuple[int, int, int]

# ---------------------------------------------------------------------------------
# Pinned constants of the shape rule and of the selection (the pages leave all open).
# ---------------------------------------------------------------------------------
ALPHA = 0.5        # exponent of b*_d ~ g_d^-alpha (Table 10 ablates 1/3, 1, 2; default is none of them)
TAU_LO = 1.0       # audio gate is 0 at or below the head-mean A2V norm ...
TAU_HI = 2.0       # ... and 1 at twice the head-mean or more
G_MIN = 1e-3       # floor on the guidance so that log2 is defined for flat zones
EPS = 1e-12        # guard of every ratio
NEAR_TIE = 1e-4    # relative margin under which a discrete decision counts as a near-tie


@dataclass(frozen=True)
class ShapeParams:
    alpha: float = ALPHA
    tau_lo: float = TAU_LO
    tau_hi: float = TAU_HI
    g_min: float = G_MIN
    eps: float = EPS


# =================================================================================
# Shapes and candidate sets (Table 11 caption: shapes are written b_T b_H b_W and
# every shape of one candidate set C_64 / C_128 / C_256 holds the same token count).
# =================================================================================

def parse_shape_code(code: str) -> Shape:
    """'824' -> (8, 2, 4); '1x4x16' -> (1, 4, 16)."""
    parts = code.split("x") if "x" in code else list(code)
    if len(parts) != 3:
        raise ValueError(f"bad shape code {code!r}")
    return tuple(int(p) for p in parts)  # type: ignore[return-value]


def candidate_volume(cands: Sequence[Shape]) -> int:
    """Common token count of a candidate set; raises if the volumes differ."""
    vols = {bt * bh * bw for (bt, bh, bw) in cands}
    if len(vols) != 1:
        raise ValueError(f"candidate shapes have unequal volumes {sorted(vols)}")
    return vols.pop()


# =================================================================================
# Geometry: macro-zones (abstract; Figure 2 caption).
# Reading: zones of fixed extents (zt, zh, zw) tile the (T, H, W) grid from the
# origin; the grid is padded at its far edges up to a multiple of the zone; zones are
# numbered in t-major raster order.  Tokens are numbered n = (t*H + h)*W + w.
# =================================================================================

def zone_counts(grid, zone) -> Tuple[int, int, int]:
    return tuple(-(-g // z) for g, z in zip(grid, zone))  # type: ignore[return-value]


def num_zones(grid, zone) -> int:
    a, b, c = zone_counts(grid, zone)
    return a * b * c


def zone_view(X: np.ndarray, grid, zone) -> Tuple[np.ndarray, np.ndarray]:
    """Regroup the token axis of X [..., N, C] into zones.

    Returns Xz [..., nZ, zt, zh, zw, C] (zeros at padding) and the validity mask
    [nZ, zt, zh, zw] (True where the position lies inside the real grid)."""
    T, H, W = grid
    zt, zh, zw = zone
    nzt, nzh, nzw = zone_counts(grid, zone)
    lead = X.shape[:-2]
    C = X.shape[-1]
    Xg = X.reshape(lead + (T, H, W, C))
    pad = [(0, 0)] * len(lead) + [(0, nzt * zt - T), (0, nzh * zh - H), (0, nzw * zw - W), (0, 0)]
    Xp = np.pad(Xg, pad)
    Xp = Xp.reshape(lead + (nzt, zt, nzh, zh, nzw, zw, C))
    k = len(lead)
    perm = list(range(k)) + [k, k + 2, k + 4, k + 1, k + 3, k + 5, k + 6]
    Xz = Xp.transpose(perm).reshape(lead + (nzt * nzh * nzw, zt, zh, zw, C))
    m = np.zeros((nzt * zt, nzh * zh, nzw * zw), dtype=bool)
    m[:T, :H, :W] = True
    m = m.reshape(nzt, zt, nzh, zh, nzw, zw).transpose(0, 2, 4, 1, 3, 5).reshape(-1, zt, zh, zw)
    return Xz, m


def directional_semivariance(Xz: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Lag-one semivariance of each channel along t, h and w inside each zone.

    Reading of Eq. 1 (not printed; Table 9 caption names it the video channel-wise
    variance guidance, computed per channel): the variance of a feature along axis d
    is taken as half the mean squared increment between neighbours along d,
        gamma_{d,c} = 1/2 * mean over pairs (x, x+e_d) of (X[x,c] - X[x+e_d,c])^2,
    over pairs whose two tokens both lie inside the zone and inside the real grid.
    A zone with no pair along d gets gamma_d = 0.

    Xz [..., nZ, zt, zh, zw, C] -> gamma [..., nZ, 3, C] (float64)."""
    Xz = Xz.astype(np.float64, copy=False)
    out = np.zeros(Xz.shape[:-4] + (3,) + Xz.shape[-1:], dtype=np.float64)
    for d in range(3):
        ax = Xz.ndim - 4 + d           # axis of Xz holding spatial dim d
        n = Xz.shape[ax]
        a = np.take(Xz, range(1, n), axis=ax)
        b = np.take(Xz, range(0, n - 1), axis=ax)
        pm = np.take(mask, range(1, n), axis=1 + d) & np.take(mask, range(0, n - 1), axis=1 + d)
        pmf = pm.astype(np.float64)[..., None]                    # [nZ, .., .., .., 1]
        ssd = ((a - b) ** 2 * pmf).sum(axis=(-4, -3, -2))         # [..., nZ, C]
        cnt = pmf.sum(axis=(-4, -3, -2))                          # [nZ, 1]
        gam = np.where(cnt > 0, 0.5 * ssd / np.maximum(cnt, 1.0), 0.0)
        out[..., d, :] = gam
    return out


def zone_stats(v: np.ndarray, a2v: np.ndarray, grid, zone, eps: float = EPS,
               global_variance: bool = False) -> np.ndarray:
    """Per-zone statistics, float64 [B, Hh, nZ, 8]:
        [0:3]  r_{v,d}: video channel-wise directional share along t, h, w
        [3:6]  gamma^a_d: directional semivariance of the A2V norm map
        [6]    m_z: mean A2V norm over the zone's valid tokens
        [7]    n_z: number of valid tokens

    Video (abstract: variance of the video features taken per channel; Table 9
    caption: per channel, on value features by default): per channel c the share of each axis is
    s_{d,c} = gamma_{d,c} / (sum_d' gamma_{d',c} + eps) and r_{v,d} = mean_c s_{d,c}.
    Audio (abstract: norms of the audio-to-video cross-attention output): the
    per-token norm a_x = ||O_a2v[x]||_2, its zone mean m_z, and the same lag-one
    semivariance on the scalar map a (Table 9 caption: audio directional variance).

    global_variance (Table 9 caption, the variant without per-channel variance: the
    feature variance is computed across all channels jointly): the channel-mean
    semivariance gbar_d = mean_c gamma_{d,c} replaces the per-channel shares, and
    r_{v,d} = gbar_d / (sum_d' gbar_d' + eps)."""
    v = np.asarray(v, dtype=np.float64)
    a2v = np.asarray(a2v, dtype=np.float64)
    B, Hh, N, C = v.shape
    nZ = num_zones(grid, zone)
    out = np.zeros((B, Hh, nZ, 8), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            Vz, mask = zone_view(v[b, h], grid, zone)
            gv = directional_semivariance(Vz, mask)                        # [nZ, 3, C]
            if global_variance:
                gbar = gv.mean(axis=2)                                     # [nZ, 3]
                out[b, h, :, 0:3] = gbar / (gbar.sum(axis=1, keepdims=True) + eps)
            else:
                share = gv / (gv.sum(axis=1, keepdims=True) + eps)
                out[b, h, :, 0:3] = share.mean(axis=2)
            a = np.sqrt((a2v[b, h] ** 2).sum(axis=1))                     # [N]
            Az, _ = zone_view(a[:, None], grid, zone)                     # [nZ, zt, zh, zw, 1]
            out[b, h, :, 3:6] = directional_semivariance(Az, mask)[:, :, 0]
            nval = mask.reshape(nZ, -1).sum(axis=1).astype(np.float64)
            out[b, h, :, 6] = Az[..., 0].reshape(nZ, -1).sum(axis=1) / nval
            out[b, h, :, 7] = nval
    return out


def zone_stats_bruteforce(v: np.ndarray, a2v: np.ndarray, grid, zone, eps: float = EPS,
                          global_variance: bool = False) -> np.ndarray:
    """Same quantities as zone_stats, by explicit loops over zones, tokens and axes
    (tiny inputs only); used to pin the vectorised version."""
    T, H, W = grid
    zt, zh, zw = zone
    nzt, nzh, nzw = zone_counts(grid, zone)
    B, Hh, N, C = v.shape
    out = np.zeros((B, Hh, nzt * nzh * nzw, 8))
    for b in range(B):
        for hh in range(Hh):
            a = [math.sqrt(sum(float(x) ** 2 for x in a2v[b, hh, n])) for n in range(N)]
            for it in range(nzt):
                for ih in range(nzh):
                    for iw in range(nzw):
                        z = (it * nzh + ih) * nzw + iw
                        toks = [(t, h, w) for t in range(it * zt, min(T, it * zt + zt))
                                for h in range(ih * zh, min(H, ih * zh + zh))
                                for w in range(iw * zw, min(W, iw * zw + zw))]
                        inzone = set(toks)
                        ssd_v = np.zeros((3, C))
                        ssd_a = np.zeros(3)
                        cnt = np.zeros(3)
                        for (t, h, w) in toks:
                            n0 = (t * H + h) * W + w
                            for d, (dt, dh, dw) in enumerate(((1, 0, 0), (0, 1, 0), (0, 0, 1))):
                                nb = (t + dt, h + dh, w + dw)
                                if nb in inzone:
                                    n1 = (nb[0] * H + nb[1]) * W + nb[2]
                                    cnt[d] += 1
                                    ssd_v[d] += (v[b, hh, n0].astype(np.float64) - v[b, hh, n1]) ** 2
                                    ssd_a[d] += (a[n0] - a[n1]) ** 2
                        gv = np.array([0.5 * ssd_v[d] / cnt[d] if cnt[d] else np.zeros(C) for d in range(3)])
                        ga = np.array([0.5 * ssd_a[d] / cnt[d] if cnt[d] else 0.0 for d in range(3)])
                        if global_variance:
                            gbar = [sum(gv[d]) / C for d in range(3)]
                            out[b, hh, z, 0:3] = [g / (sum(gbar) + eps) for g in gbar]
                        else:
                            share = gv / (gv.sum(axis=0, keepdims=True) + eps)
                            out[b, hh, z, 0:3] = share.mean(axis=1)
                        out[b, hh, z, 3:6] = ga
                        out[b, hh, z, 6] = sum(a[(t * H + h) * W + w] for (t, h, w) in toks) / len(toks)
                        out[b, hh, z, 7] = len(toks)
    return out


def zone_activity(v: np.ndarray, grid, zone) -> np.ndarray:
    """Video activity of every zone, float64 [B, Hh, nZ]: the channel-mean lag-one
    semivariance summed over the three axes, sum_d mean_c gamma_{d,c} (the magnitude that
    the per-axis shares of zone_stats normalise away).  Used by the multi-volume reading
    (assign_shapes_multi)."""
    v = np.asarray(v, dtype=np.float64)
    B, Hh, N, C = v.shape
    out = np.zeros((B, Hh, num_zones(grid, zone)))
    for b in range(B):
        for h in range(Hh):
            Vz, mask = zone_view(v[b, h], grid, zone)
            out[b, h] = directional_semivariance(Vz, mask).mean(axis=2).sum(axis=1)
    return out


def a2v_norm(q: np.ndarray, ka: np.ndarray, va: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Per-token norm of the audio-to-video cross-attention output (abstract: the shapes
    follow the feature norms of the A2V cross-attention output): video queries q
    [B,Hh,N,C] attend densely to audio keys ka and values va [B,Hh,Na,C];
    a_x = || softmax_j(q_x . ka_j * scale) va ||_2, float64 [B, Hh, N].
    zone_stats(v, a[..., None]) then gives the statistics of the norm map (the norm of a
    one-element row is its value)."""
    q, ka, va = (np.asarray(x, dtype=np.float64) for x in (q, ka, va))
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    s = (q @ np.swapaxes(ka, -1, -2)) * scale
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    o = (e / e.sum(axis=-1, keepdims=True)) @ va
    return np.sqrt((o * o).sum(axis=-1))


# =================================================================================
# Shape assignment (abstract: finer partitioning along axes of rapid visual variation
# and strong audio-visual coupling; Table 9 caption: r_{v,d}, gate a-bar, v-hat_{a,d};
# Table 10 caption: b*_d ~ g_d^-alpha and the quantization of Eq. 7).
# =================================================================================

def shape_guidance(stats: np.ndarray, p: ShapeParams = ShapeParams(), dtype=np.float32):
    """Gate a-bar [B,Hh,nZ], audio share v-hat [B,Hh,nZ,3] and guidance g [B,Hh,nZ,3].

    Readings: the head-mean norm m-bar is the mean of a over all valid tokens of the
    head (= sum_z m_z n_z / sum_z n_z); the gate a-bar_z = clamp((m_z/m-bar - tau_lo) /
    (tau_hi - tau_lo), 0, 1); v-hat_{a,d} = gamma^a_d / (sum_d gamma^a_d + eps); the two
    signals mix convexly by the gate, g_d = max((1 - a-bar) r_{v,d} + a-bar v-hat_{a,d}, g_min)."""
    s = np.asarray(stats).astype(dtype)
    f = lambda x: dtype(x)  # noqa: E731
    rv, ga, m, n = s[..., 0:3], s[..., 3:6], s[..., 6], s[..., 7]
    mbar = (m * n).sum(axis=-1, dtype=dtype) / n.sum(axis=-1, dtype=dtype)        # [B, Hh]
    ratio = m / np.maximum(mbar, f(p.eps))[..., None]
    abar = np.clip((ratio - f(p.tau_lo)) / (f(p.tau_hi) - f(p.tau_lo)), f(0.0), f(1.0))
    vhat = ga / ((ga[..., 0] + ga[..., 1] + ga[..., 2])[..., None] + f(p.eps))
    g = (f(1.0) - abar)[..., None] * rv + abar[..., None] * vhat
    g = np.maximum(g, f(p.g_min))
    return abar.astype(dtype), vhat.astype(dtype), g.astype(dtype)


def ideal_log_extents(g: np.ndarray, vol: int, alpha: float = ALPHA, dtype=np.float32) -> np.ndarray:
    """lambda_d = log2(vol)/3 - alpha (log2 g_d - mean_d' log2 g_d').

    Power law b*_d ~ g_d^-alpha (Table 10 caption), normalised so that the ideal
    extents multiply to the block volume (sum_d lambda_d = log2 vol)."""
    g = np.asarray(g).astype(dtype)
    L = np.log2(g).astype(dtype)
    mean = (L[..., 0] + L[..., 1] + L[..., 2]) / dtype(3.0)
    return (dtype(math.log2(vol) / 3.0) - dtype(alpha) * (L - mean[..., None])).astype(dtype)


def feasible(cand: Shape, zone) -> bool:
    """A candidate can tile a zone iff each of its extents divides the zone's extent."""
    return all(z % c == 0 for c, z in zip(cand, zone))


def quantize_shape(lam: np.ndarray, cands: Sequence[Shape], zone, dtype=np.float32):
    """Reading of Eq. 7: the nearest feasible candidate in log2 extents,
        argmin_c sum_d (log2 c_d - lambda_d)^2   (exact ties -> lowest list index),
    and its relative margin (D_2 - D_1) / max(D_2, 1e-12) to the runner-up."""
    lam = np.asarray(lam).astype(dtype)
    C = len(cands)
    D = np.full(lam.shape[:-1] + (C,), np.inf, dtype=dtype)
    for c, shp in enumerate(cands):
        if not feasible(shp, zone):
            continue
        lc = np.array([math.log2(x) for x in shp], dtype=dtype)
        e = lc - lam
        D[..., c] = e[..., 0] * e[..., 0] + e[..., 1] * e[..., 1] + e[..., 2] * e[..., 2]
    sid = np.argmin(D, axis=-1)                                   # first minimum
    Ds = np.sort(D, axis=-1)
    d1 = Ds[..., 0].astype(np.float64)
    d2 = Ds[..., 1].astype(np.float64) if C > 1 else np.full_like(d1, np.inf)
    with np.errstate(invalid="ignore"):
        margin = np.where(np.isinf(d2), 1.0, (d2 - d1) / np.maximum(d2, 1e-12))
    return sid.astype(np.int32), margin


def assign_shapes(stats: np.ndarray, cands: Sequence[Shape], zone, p: ShapeParams = ShapeParams(),
                  dtype=np.float32):
    """Shape id [B,Hh,nZ] (index into cands) and margin [B,Hh,nZ] for every zone."""
    vol = candidate_volume(cands)
    _, _, g = shape_guidance(stats, p, dtype)
    lam = ideal_log_extents(g, vol, p.alpha, dtype)
    return quantize_shape(lam, cands, zone, dtype)


TAU_128 = 1.0      # zones with activity below this take 128-token blocks ...
TAU_256 = 0.5      # ... and below this 256-token blocks


def assign_shapes_multi(stats: np.ndarray, vact: np.ndarray, cands: Sequence[Shape], zone,
                        p: ShapeParams = ShapeParams(), tau_128: float = TAU_128, tau_256: float = TAU_256,
                        dtype=np.float32):
    """Shapes from a candidate list that mixes 64-, 128- and 256-token shapes (Tables 9 and
    11: sets C_64, C_128, C_256; Table 10 caption: thresholds tau_128 / tau_256 of the block
    shape assignment).  The pages give no rule for the volume; reading:
        rho_z = vact_z / (mean of vact over the head's zones)   (0 if that mean is 0)
        act_z = rho_z + a-bar_z                                  (a-bar: the audio gate)
        volume 256 if act_z < tau_256, 128 if act_z < tau_128, else 64,
    falling back to the next smaller volume when no shape of the chosen volume tiles the
    zone; the shape is then the Eq. 7 choice (quantize_shape) among the candidates of that
    volume, with lambda built for that volume.  Smooth zones without audio coupling take
    the largest blocks.  Returns (shape id into cands, margin), the margin being the
    smaller of the shape margin and the relative distance |act - tau| / tau to each
    threshold, so that a near-threshold zone counts as a near-tie."""
    abar, _, g = shape_guidance(stats, p, dtype)
    vact = np.asarray(vact).astype(dtype)
    n = np.asarray(stats)[..., 7]
    live = n > 0
    cntz = np.maximum(live.sum(axis=-1), 1).astype(dtype)
    mean = (np.where(live, vact, dtype(0)).sum(axis=-1, dtype=dtype) / cntz).astype(dtype)   # [B, Hh]
    with np.errstate(invalid="ignore", divide="ignore"):
        rho = np.where(mean[..., None] > 0, vact / mean[..., None], dtype(0)).astype(dtype)
    act = (rho + abar).astype(dtype)
    vols = sorted({bt * bh * bw for (bt, bh, bw) in cands})
    if 64 not in vols:
        raise ValueError("the candidate list needs 64-token shapes")

    def has_feasible(vol):
        return any(feasible(c, zone) and c[0] * c[1] * c[2] == vol for c in cands)

    B, Hh, nZ = act.shape
    sid = np.zeros((B, Hh, nZ), dtype=np.int32)
    margin = np.zeros((B, Hh, nZ))
    for b in range(B):
        for h in range(Hh):
            for z in range(nZ):
                a = act[b, h, z]
                want = 256 if a < dtype(tau_256) else (128 if a < dtype(tau_128) else 64)
                while want > 64 and not (want in vols and has_feasible(want)):
                    want //= 2
                idx = [i for i, c in enumerate(cands) if c[0] * c[1] * c[2] == want]
                lam = ideal_log_extents(g[b, h, z][None], want, p.alpha, dtype)
                j, m = quantize_shape(lam, [cands[i] for i in idx], zone, dtype)
                sid[b, h, z] = idx[int(j[0])]
                thr = [abs(float(a) - t) / t for t in (tau_128, tau_256)]
                margin[b, h, z] = min([float(m[0])] + thr)
    return sid, margin


# =================================================================================
# Permutation into blocks (abstract: tokens within each block stay coherent, so each
# block must be a contiguous run; Figure 2 caption).
# Reading of the slot order: zones in raster order; the zone's blocks in raster order
# over its block grid (zt/bt, zh/bh, zw/bw); inside a block, its tokens that lie in the
# real grid first, in raster order over the block, then its padding slots.  A block cut
# by the grid's far edge keeps a valid sub-box (et, eh, ew) at its origin, so the j-th
# valid token is that sub-box's j-th token in raster order.
# =================================================================================

def slot_map(grid, zone, cands: Sequence[Shape], shape_id: np.ndarray) -> np.ndarray:
    """Token index of every slot, int64 [B, Hh, Npad] (-1 at padding slots)."""
    T, H, W = grid
    zt, zh, zw = zone
    nzt, nzh, nzw = zone_counts(grid, zone)
    Vz = zt * zh * zw
    sid = np.asarray(shape_id)
    B, Hh, nZ = sid.shape
    out = np.full((B, Hh, nZ * Vz), -1, dtype=np.int64)
    for z in range(nZ):
        it, ih, iw = z // (nzh * nzw), (z // nzw) % nzh, z % nzw
        for b in range(B):
            for h in range(Hh):
                bt, bh, bw = cands[int(sid[b, h, z])]
                S = bt * bh * bw                      # this zone's block volume
                nbz = Vz // S
                nbh, nbw = zh // bh, zw // bw
                for blk in range(nbz):
                    t0 = it * zt + (blk // (nbh * nbw)) * bt
                    h0 = ih * zh + ((blk // nbw) % nbh) * bh
                    w0 = iw * zw + (blk % nbw) * bw
                    et, eh, ew = (max(0, min(bt, T - t0)), max(0, min(bh, H - h0)), max(0, min(bw, W - w0)))
                    if et * eh * ew == 0:
                        continue
                    j = np.arange(et * eh * ew)
                    tt = t0 + j // (eh * ew)
                    hh = h0 + (j // ew) % eh
                    ww = w0 + j % ew
                    base = z * Vz + blk * S
                    out[b, h, base:base + j.size] = (tt * H + hh) * W + ww
    return out


def block_valid(tok: np.ndarray, vol: int) -> np.ndarray:
    """Valid-slot count of every block, int32 [B, Hh, nb] (0 marks a dead block)."""
    B, Hh, Np = tok.shape
    return (tok >= 0).reshape(B, Hh, Np // vol, vol).sum(axis=-1).astype(np.int32)


def block_heads(tok: np.ndarray, shape_id: np.ndarray, cands: Sequence[Shape], zone, unit: int = 64) -> np.ndarray:
    """Block-level valid counts for zones of different block volumes, int32
    [B, Hh, Npad/unit]: a block is identified by its first unit (a run of `unit` slots),
    which holds the whole block's valid count; its other units hold 0.  Because a block's
    valid slots come first, its valid rows are the n rows from its first unit on, so
    pool_blocks, the selection and sparse attention take these counts with vol = unit."""
    B, Hh, Np = tok.shape
    Vz = zone[0] * zone[1] * zone[2]
    per_unit = block_valid(tok, unit)
    out = np.zeros_like(per_unit)
    upz = Vz // unit
    for b in range(B):
        for h in range(Hh):
            for z in range(Np // Vz):
                bt, bh, bw = cands[int(shape_id[b, h, z])]
                g = bt * bh * bw // unit
                for u0 in range(z * upz, (z + 1) * upz, g):
                    out[b, h, u0] = per_unit[b, h, u0:u0 + g].sum()
    return out


def permute(x: np.ndarray, tok: np.ndarray) -> np.ndarray:
    """[B, Hh, N, C] -> [B, Hh, Npad, C] in slot order, zeros at padding slots."""
    B, Hh, N, C = x.shape
    y = np.zeros((B, Hh, tok.shape[-1], C), dtype=x.dtype)
    for b in range(B):
        for h in range(Hh):
            valid = tok[b, h] >= 0
            y[b, h, valid] = x[b, h, tok[b, h, valid]]
    return y


def unpermute(y: np.ndarray, tok: np.ndarray, N: int) -> np.ndarray:
    """[B, Hh, Npad, C] -> [B, Hh, N, C]; padding slots are dropped."""
    B, Hh, Np, C = y.shape
    x = np.zeros((B, Hh, N, C), dtype=y.dtype)
    for b in range(B):
        for h in range(Hh):
            valid = tok[b, h] >= 0
            x[b, h, tok[b, h, valid]] = y[b, h, valid]
    return x


# =================================================================================
# Block pooling and hybrid Top-k/Top-p selection (abstract: block-level features and
# a hybrid block selection that sets per-query sparsity; Figure 2 caption: hybrid
# Top-k/Top-p block-sparse attention; Table 7 caption: Top-p keeps the smallest set of
# key blocks whose cumulative attention weight exceeds the threshold).
# =================================================================================

def pool_blocks(xp: np.ndarray, bvalid: np.ndarray, vol: int) -> np.ndarray:
    """Mean of each block's valid rows, float64 [B, Hh, nb, C] (zeros for dead blocks).
    Valid rows of a block are its first bvalid slots (see slot_map)."""
    B, Hh, Np, C = xp.shape
    nb = Np // vol
    # rows I*vol .. I*vol + n - 1; with mixed volumes a block identified by its first unit
    # runs past that unit, so the sum is a difference of prefix sums, not a per-unit sum
    cs = np.concatenate([np.zeros((B, Hh, 1, C)), np.cumsum(xp.astype(np.float64), axis=2)], axis=2)
    start = (np.arange(nb) * vol)[None, None, :]
    end = start + np.asarray(bvalid)
    s = np.take_along_axis(cs, end[..., None], axis=2) - np.take_along_axis(cs, np.broadcast_to(start, end.shape)[..., None], axis=2)
    return s / np.maximum(bvalid, 1)[..., None]


def hybrid_count(P_sorted: np.ndarray, top_p: float, k_min: int, k_max: int, dtype=np.float32) -> Tuple[int, int]:
    """Number of key blocks kept from a row of block probabilities sorted descending.

    Top-p: n_p = the smallest n whose cumulative sum C_n exceeds top_p (strictly),
    or every live block if no prefix does.  Hybrid: n = min(max(n_p, k_min), k_max, n_live).
    Reading for top_p >= 1: the weights of a row sum to exactly 1, so no prefix exceeds
    top_p and every live block is kept, however the float rounding of C_n comes out.
    Returns (n, n_p)."""
    P_sorted = np.asarray(P_sorted).astype(dtype)
    n_live = P_sorted.size
    C = np.cumsum(P_sorted, dtype=dtype)
    over = np.nonzero(C > dtype(top_p))[0] if top_p < 1 else np.zeros(0, dtype=np.int64)
    n_p = int(over[0]) + 1 if over.size else n_live
    n = min(max(n_p, k_min), k_max, n_live)
    return n, n_p


def _clamp(n_p, k_min, k_max, n_live):
    return min(max(n_p, k_min), k_max, n_live)


def select_row(qbar_row: np.ndarray, kbar: np.ndarray, live: np.ndarray, scale: float,
               top_p: float, k_min: int, k_max: int, dtype=np.float32):
    """Selection of one live query block.

    Readings: block score = scale * <mean Q of the query block, mean K of the key block>
    with scale = 1/sqrt(d); softmax over the live key blocks; sort descending with ties
    broken toward the lower key-block index; hybrid count (hybrid_count); no block is
    forced in.  Returns (ascending selected key-block indices, near_tie flag)."""
    J = np.nonzero(live)[0]
    q = np.asarray(qbar_row).astype(dtype)
    K = np.asarray(kbar[J]).astype(dtype)
    logits = (K @ q) * dtype(scale)
    e = np.exp(logits - logits.max())
    P = (e / e.sum(dtype=dtype)).astype(dtype)
    order = np.argsort(-P, kind="stable")
    Ps = P[order]
    n, n_p = hybrid_count(Ps, top_p, k_min, k_max, dtype)
    sel = np.sort(J[order[:n]])
    # near-tie: a decision within the relative margin that another rounding could flip
    Cs = np.cumsum(Ps.astype(np.float64))
    near = False
    if n < Ps.size and (float(Ps[n - 1]) - float(Ps[n])) <= NEAR_TIE * float(Ps[n - 1]):
        near = True
    if top_p < 1 and abs(Cs[n_p - 1] - top_p) < NEAR_TIE and _clamp(n_p + 1, k_min, k_max, Ps.size) != n:
        near = True
    if top_p < 1 and n_p >= 2 and abs(Cs[n_p - 2] - top_p) < NEAR_TIE and \
            _clamp(n_p - 1, k_min, k_max, Ps.size) != n:
        near = True
    return sel.astype(np.int32), near


def select_blocks(qbar: np.ndarray, kbar: np.ndarray, bvalid: np.ndarray, scale: float,
                  top_p: float, k_min: int, k_max: int, rows: Optional[Sequence[int]] = None,
                  dtype=np.float32):
    """Selected key-block lists for every (b, h, query block) (or the given rows).

    Returns sel: dict (b, h, I) -> ascending int32 array (empty for dead query blocks),
    and near: dict (b, h, I) -> bool."""
    B, Hh, nb, C = qbar.shape
    sel, near = {}, {}
    for b in range(B):
        for h in range(Hh):
            live = bvalid[b, h] > 0
            it = range(nb) if rows is None else rows
            for I in it:
                if not live[I]:
                    sel[(b, h, I)] = np.zeros(0, dtype=np.int32)
                    near[(b, h, I)] = False
                    continue
                sel[(b, h, I)], near[(b, h, I)] = select_row(
                    qbar[b, h, I], kbar[b, h], live, scale, top_p, k_min, k_max, dtype)
    return sel, near


def select_blocks_all(qbar: np.ndarray, kbar: np.ndarray, bvalid: np.ndarray, scale: float,
                      top_p: float, k_min: int, k_max: int, dtype=np.float32):
    """select_blocks over every row, with each head's score matrix formed at once (same
    arithmetic as select_row, in matrix form: one matmul, row-wise softmax, row-wise
    stable descending sort, row-wise cumulative sums)."""
    B, Hh, nb, C = qbar.shape
    sel, near = {}, {}
    for b in range(B):
        for h in range(Hh):
            live = bvalid[b, h] > 0
            J = np.nonzero(live)[0]
            Ilive = np.nonzero(live)[0]
            K = np.asarray(kbar[b, h, J]).astype(dtype)
            Qm = np.asarray(qbar[b, h, Ilive]).astype(dtype)
            logits = (Qm @ K.T) * dtype(scale)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            P = (e / e.sum(axis=1, keepdims=True, dtype=dtype)).astype(dtype)
            order = np.argsort(-P, axis=1, kind="stable")
            Ps = np.take_along_axis(P, order, axis=1)
            Cs = np.cumsum(Ps, axis=1, dtype=dtype)
            Cd = np.cumsum(Ps.astype(np.float64), axis=1)
            nl = J.size
            for r, I in enumerate(Ilive):
                over = np.nonzero(Cs[r] > dtype(top_p))[0] if top_p < 1 else np.zeros(0, dtype=np.int64)
                n_p = int(over[0]) + 1 if over.size else nl
                n = _clamp(n_p, k_min, k_max, nl)
                sel[(b, h, int(I))] = np.sort(J[order[r, :n]]).astype(np.int32)
                nr = False
                if n < nl and (float(Ps[r, n - 1]) - float(Ps[r, n])) <= NEAR_TIE * float(Ps[r, n - 1]):
                    nr = True
                if top_p < 1 and abs(Cd[r, n_p - 1] - top_p) < NEAR_TIE and _clamp(n_p + 1, k_min, k_max, nl) != n:
                    nr = True
                if top_p < 1 and n_p >= 2 and abs(Cd[r, n_p - 2] - top_p) < NEAR_TIE and \
                        _clamp(n_p - 1, k_min, k_max, nl) != n:
                    nr = True
                near[(b, h, int(I))] = nr
            for I in np.nonzero(~live)[0]:
                sel[(b, h, int(I))] = np.zeros(0, dtype=np.int32)
                near[(b, h, int(I))] = False
    return sel, near


def selection_arrays(sel: Dict, B: int, Hh: int, nb: int, k_max: int):
    """ELL form of a full selection: idx [B,Hh,nb,k_max] (-1 padded) and cnt [B,Hh,nb]."""
    idx = np.full((B, Hh, nb, k_max), -1, dtype=np.int32)
    cnt = np.zeros((B, Hh, nb), dtype=np.int32)
    for (b, h, I), s in sel.items():
        idx[b, h, I, :s.size] = s
        cnt[b, h, I] = s.size
    return idx, cnt


def reverse_index_sorted(idx: np.ndarray, cnt: np.ndarray):
    """reverse_index by one stable sort of the (I, J) pairs on J per head (pairs are
    listed in ascending I, so each key block's query blocks stay ascending)."""
    B, Hh, nb, k_max = idx.shape
    rev_ptr = np.zeros((B, Hh, nb + 1), dtype=np.int32)
    rev_idx = np.full((B, Hh, nb * k_max), -1, dtype=np.int32)
    pos = np.arange(k_max)[None, :]
    for b in range(B):
        for h in range(Hh):
            m = pos < cnt[b, h][:, None]
            I = np.broadcast_to(np.arange(nb)[:, None], (nb, k_max))[m]
            J = idx[b, h][m]
            o = np.argsort(J, kind="stable")
            rev_idx[b, h, :o.size] = I[o]
            rev_ptr[b, h, 1:] = np.cumsum(np.bincount(J, minlength=nb))
    return rev_ptr, rev_idx


def reverse_index(idx: np.ndarray, cnt: np.ndarray):
    """Transpose of the selection: for every key block J, the query blocks that chose
    it, ascending.  rev_ptr [B,Hh,nb+1], rev_idx [B,Hh,nb*k_max] (-1 padded)."""
    B, Hh, nb, k_max = idx.shape
    rev_ptr = np.zeros((B, Hh, nb + 1), dtype=np.int32)
    rev_idx = np.full((B, Hh, nb * k_max), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hh):
            cols: List[List[int]] = [[] for _ in range(nb)]
            for I in range(nb):
                for J in idx[b, h, I, :cnt[b, h, I]]:
                    cols[int(J)].append(I)
            pos = 0
            for J in range(nb):
                rev_ptr[b, h, J] = pos
                rev_idx[b, h, pos:pos + len(cols[J])] = cols[J]
                pos += len(cols[J])
            rev_ptr[b, h, nb] = pos
    return rev_ptr, rev_idx


# =================================================================================
# Block-sparse attention (Figure 2 caption: attention restricted to the selected
# blocks).  Reading: exact softmax attention in which query row i of block I attends to
# every valid key row of every selected block and to nothing else; padding query rows
# output zeros.  LSE_i = ln sum_j exp(scale q_i.k_j).
# =================================================================================

def _rows(x, b, h, B_, vol, n):
    return x[b, h, B_ * vol: B_ * vol + n]


def sparse_attn_fwd(qp, kp, vp, bvalid, sel: Dict, scale: float, vol: int,
                    blocks: Optional[Sequence[Tuple[int, int, int]]] = None, dtype=np.float64):
    """O' [B,Hh,Npad,C] and LSE [B,Hh,Npad] in float64 (rows of unlisted blocks stay 0).
    Reading: a valid query row with nothing to attend (an empty list, or listed blocks
    without valid rows) has no softmax; it outputs 0 with LSE 0, as padding rows do.
    dtype: the precision of the arithmetic (float64 for parity; float32 only for timing)."""
    qp, kp, vp = (np.asarray(a, dtype=dtype) for a in (qp, kp, vp))
    B, Hh, Np, C = qp.shape
    O = np.zeros((B, Hh, Np, vp.shape[-1]), dtype=dtype)
    L = np.zeros((B, Hh, Np), dtype=dtype)
    it = blocks if blocks is not None else [(b, h, I) for b in range(B) for h in range(Hh) for I in range(Np // vol)]
    for (b, h, I) in it:
        n = int(bvalid[b, h, I])
        js = [J for J in sel[(b, h, I)] if bvalid[b, h, J] > 0]
        if n == 0 or not js:
            continue
        q = _rows(qp, b, h, I, vol, n)
        K = np.concatenate([_rows(kp, b, h, J, vol, int(bvalid[b, h, J])) for J in js])
        V = np.concatenate([_rows(vp, b, h, J, vol, int(bvalid[b, h, J])) for J in js])
        s = (q @ K.T) * scale
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        O[b, h, I * vol: I * vol + n] = (e / z) @ V
        L[b, h, I * vol: I * vol + n] = (m + np.log(z))[:, 0]
    return O, L


def _transpose_selection(sel: Dict) -> Dict:
    """(b, h, J) -> ascending array of the query blocks I whose selection holds J."""
    cols: Dict[Tuple[int, int, int], List[int]] = {}
    for (b, h, I) in sorted(sel):
        for J in sel[(b, h, I)]:
            cols.setdefault((b, h, int(J)), []).append(I)
    return {k: np.array(v, dtype=np.int32) for k, v in cols.items()}


def sparse_attn_bwd(qp, kp, vp, op, dop, lse, bvalid, sel: Dict, scale: float, vol: int,
                    q_blocks: Optional[Sequence[Tuple[int, int, int]]] = None,
                    k_blocks: Optional[Sequence[Tuple[int, int, int]]] = None, dtype=np.float64):
    """Gradients of sum(O' * dO') w.r.t. Q', K', V' with the selection held fixed
    (reading: the statistics, shapes and selection are piecewise constant, so no
    gradient flows through them).
        D_i = dO_i . O_i,  P_ij = exp(scale q_i.k_j - LSE_i),  dV_j = sum_i P_ij dO_i,
        dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i),
        dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
    dQ is accumulated per query block over its selected key blocks, dK/dV per key block
    over the query blocks that selected it.  q_blocks / k_blocks limit the work to the
    listed blocks (all by default); other rows stay 0.  Returns float64 dQ', dK', dV'
    (dtype: the precision of the arithmetic, float64 for parity; float32 only for timing)."""
    qp, kp, vp, op, dop = (np.asarray(a, dtype=dtype) for a in (qp, kp, vp, op, dop))
    B, Hh, Np, C = qp.shape
    nb = Np // vol
    dQ, dK, dV = np.zeros_like(qp), np.zeros_like(kp), np.zeros_like(vp)
    lse = np.asarray(lse, dtype=dtype)

    def rows(x, b, h, I):
        return x[b, h, I * vol: I * vol + int(bvalid[b, h, I])]

    def grads_of_rows(q, do, o, li, k, v):
        """P and dS of query rows (q, dO, O, LSE) against key rows (k, v)."""
        Di = (do * o).sum(axis=1, keepdims=True)
        P = np.exp((q @ k.T) * scale - li[:, None])
        return P, P * (do @ v.T - Di)

    allq = [(b, h, I) for b in range(B) for h in range(Hh) for I in range(nb)]
    for (b, h, I) in (allq if q_blocks is None else q_blocks):
        js = sel.get((b, h, I), ())
        if bvalid[b, h, I] == 0 or len(js) == 0:
            continue
        k = np.concatenate([rows(kp, b, h, int(J)) for J in js])
        v = np.concatenate([rows(vp, b, h, int(J)) for J in js])
        q = rows(qp, b, h, I)
        P, dS = grads_of_rows(q, rows(dop, b, h, I), rows(op, b, h, I), rows(lse, b, h, I), k, v)
        dQ[b, h, I * vol: I * vol + q.shape[0]] = scale * (dS @ k)
    if k_blocks is None:
        cols = _transpose_selection(sel)
    else:  # only the requested key blocks: which query blocks list J (lists are ascending)
        def lists(s, J):
            i = int(np.searchsorted(s, J))
            return i < len(s) and s[i] == J
        empty = np.zeros(0, dtype=np.int32)
        cols = {(b, h, J): np.array([I for I in range(nb) if lists(sel.get((b, h, I), empty), J)], dtype=np.int32)
                for (b, h, J) in k_blocks}
    for (b, h, J) in (allq if k_blocks is None else k_blocks):
        Is = [int(I) for I in cols.get((b, h, J), ()) if bvalid[b, h, I] > 0]
        m = int(bvalid[b, h, J])
        if m == 0 or not Is:
            continue
        cat = lambda x: np.concatenate([rows(x, b, h, I) for I in Is])  # noqa: E731
        q, do = cat(qp), cat(dop)
        P, dS = grads_of_rows(q, do, cat(op), cat(lse), rows(kp, b, h, J), rows(vp, b, h, J))
        dV[b, h, J * vol: J * vol + m] = P.T @ do
        dK[b, h, J * vol: J * vol + m] = scale * (dS.T @ q)
    return dQ, dK, dV


def dense_attn_fwd(q, k, v, scale: float):
    """Full softmax attention on unpermuted tokens, float64: O [B,Hh,N,C], LSE [B,Hh,N]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    T = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    s = (q @ T(k)) * scale
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[..., 0]


def dense_attn_bwd(q, k, v, o, do, lse, scale: float):
    """Gradients of full softmax attention, float64 (same formulas as sparse_attn_bwd
    with every key selected)."""
    q, k, v, o, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, o, do))
    T = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    P = np.exp((q @ T(k)) * scale - lse[..., None])
    D = (do * o).sum(axis=-1)[..., None]
    dS = P * ((do @ T(v)) - D)
    dq = scale * (dS @ k)
    dk = scale * (T(dS) @ q)
    dv = T(P) @ do
    return dq, dk, dv


# =================================================================================
# The whole chain: zones -> statistics -> shapes -> permutation -> pooling ->
# selection -> block-sparse attention -> inverse permutation (Figure 2 caption).
# =================================================================================

def prism_forward(q, k, v, a2v, grid, zone, cands, top_p, k_min, k_max, scale=None,
                  shape_params: ShapeParams = ShapeParams(), dtype=np.float32,
                  features: str = "v", global_variance: bool = False, shape_id=None, mixed=None):
    """The whole forward chain.  The options are the block-shape ablations of Table 9:
    features "q" / "k" take the query / key features instead of the values for the
    variance; global_variance takes it across all channels jointly; shape_id, when
    given, replaces the statistics and shape assignment (random or fixed shapes, whose
    draws are inputs).  Top-k only / Top-p only (Table 7) are plain parameter choices:
    top_p = 1 with k_min = k_max = k, or k_min = 1 with k_max >= the live block count.
    mixed = (tau_128, tau_256): cands mixes block volumes; shapes by assign_shapes_multi,
    blocks identified by their first 64-slot unit (block_heads) and everything downstream
    run with vol = 64."""
    q, k, v, a2v = (np.asarray(a, dtype=np.float64) for a in (q, k, v, a2v))
    B, Hh, N, C = q.shape
    scale = 1.0 / math.sqrt(C) if scale is None else scale
    vol = 64 if mixed is not None else candidate_volume(cands)
    if shape_id is None:
        feat = {"v": v, "q": q, "k": k}[features]
        stats = zone_stats(feat, a2v, grid, zone, global_variance=global_variance)
        if mixed is not None:
            sid, margin = assign_shapes_multi(stats.astype(np.float32), zone_activity(feat, grid, zone), cands, zone,
                                              shape_params, mixed[0], mixed[1], dtype)
        else:
            sid, margin = assign_shapes(stats.astype(np.float32), cands, zone, shape_params, dtype)
    else:
        stats, sid = None, np.asarray(shape_id, dtype=np.int32)
        margin = np.full(sid.shape, np.inf)
    tok = slot_map(grid, zone, cands, sid)
    bv = block_heads(tok, sid, cands, zone) if mixed is not None else block_valid(tok, vol)
    qp, kp, vp = permute(q, tok), permute(k, tok), permute(v, tok)
    qbar, kbar = pool_blocks(qp, bv, vol), pool_blocks(kp, bv, vol)
    sel, near = select_blocks(qbar.astype(np.float32), kbar.astype(np.float32), bv, scale,
                              top_p, k_min, k_max, dtype=dtype)
    op, lse = sparse_attn_fwd(qp, kp, vp, bv, sel, scale, vol)
    o = unpermute(op, tok, N)
    return dict(stats=stats, shape_id=sid, shape_margin=margin, tok=tok, bvalid=bv, qp=qp, kp=kp,
                vp=vp, qbar=qbar, kbar=kbar, sel=sel, sel_near=near, op=op, lse=lse, o=o,
                scale=scale, vol=vol, N=N)


def prism_backward(fwd: Dict, do) -> Dict:
    do = np.asarray(do, dtype=np.float64)
    tok, N, vol = fwd["tok"], fwd["N"], fwd["vol"]
    dop = permute(do, tok)
    dqp, dkp, dvp = sparse_attn_bwd(fwd["qp"], fwd["kp"], fwd["vp"], fwd["op"], dop, fwd["lse"],
                                    fwd["bvalid"], fwd["sel"], fwd["scale"], vol)
    return dict(dop=dop, dqp=dqp, dkp=dkp, dvp=dvp,
                dq=unpermute(dqp, tok, N), dk=unpermute(dkp, tok, N), dv=unpermute(dvp, tok, N))


def selected_pair_flops(bvalid: np.ndarray, sel: Dict, d: int) -> float:
    """Algorithmic fwd+bwd flops of the selected blocks: 14 d per valid (query, key) pair
    (forward 4 d: two matmuls; backward 10 d: five matmuls)."""
    tot = 0
    for (b, h, I), js in sel.items():
        if js.size:
            tot += int(bvalid[b, h, I]) * int(bvalid[b, h, js].sum())
    return 14.0 * d * tot
