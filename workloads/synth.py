"""Seeded synthetic inputs for the Prism attention path.

This module only draws inputs.  It holds none of the method's arithmetic: no zone
statistics, no shape choice, no permutation, no pooling, no block selection and no
block-sparse attention.  It does evaluate the model's own dense audio-to-video (A2V)
cross-attention, because the method reads that layer's output as an input (abstract:
shapes follow the feature norms of the A2V cross-attention output).

Recipe (all streams are numpy PCG64, one independent stream per (seed, tag, b, h)):
  tag 0  per-(b,h) zone anisotropy (zoned fields): dominant axis ~ U{t,h,w},
         ratio rho ~ logU[1, rho_hi], one pair per zone in zone raster order.
  tag 1/2/3  Q/K/V field parameters then noise.  Per channel c and sinusoid m:
         global fields: per-axis frequency logU[f_lo, f_hi] with a random sign;
         zoned fields: one base frequency f0 logU[f_lo, f_hi] and a random sign per axis.
         Phase ~ U(0, 2pi).  Value = A * sum_m sin(2pi * <f, x> + phase) + N(0, noise_std).
  tag 4/5  audio keys / values K_a, V_a ~ N(0, 1), shape [n_audio, d].
  tag 6  blobs (per b): centre uniform in the (t, h, w) box, sigma ~ U[lo, hi],
         window start ~ U{0 .. n_audio - window}.
  tag 7  upstream gradient dO ~ N(0, 1).
A2V logits of video token x against audio token j are q_x . k_j / sqrt(d) plus
beta * sum_b G_b(x) * [j in window_b], G_b = exp(-|x - mu_b|^2 / (2 sigma_b^2)); the
A2V output is softmax_j(logits) @ V_a.  It is computed from the un-gained Q field.
Fields are evaluated in float32 (phases reduced modulo one cycle in float64), then
rounded to nearest-even bfloat16 for the bf16 workloads; Q is multiplied by the
workload's q_gain before rounding.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np
import torch

from .configs import Workload

TAG_ZONES, TAG_Q, TAG_K, TAG_V, TAG_KA, TAG_VA, TAG_BLOBS, TAG_DO = range(8)


def _rng(seed: int, tag: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(tag), int(b), int(h)]))


def _log_uniform(rng: np.random.Generator, lo: float, hi: float, size) -> np.ndarray:
    return np.exp(rng.uniform(math.log(lo), math.log(hi), size=size))


def token_coords(grid) -> np.ndarray:
    """(t, h, w) of every token in t-major raster order n = (t*H + h)*W + w, int64 [N, 3]."""
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.int64)


def _zone_multipliers(w: Workload, seed: int, b: int, h: int, coords: np.ndarray) -> np.ndarray:
    """Per-token frequency multiplier [N, 3]: rho on the zone's dominant axis, 1 elsewhere."""
    T, H, W = w.grid
    zt, zh, zw = w.zone
    nzt, nzh, nzw = -(-T // zt), -(-H // zh), -(-W // zw)
    nz = nzt * nzh * nzw
    rng = _rng(seed, TAG_ZONES, b, h)
    axis = rng.integers(0, 3, size=nz)
    rho = _log_uniform(rng, 1.0, w.field.rho_hi, nz)
    zid = ((coords[:, 0] // zt) * nzh + coords[:, 1] // zh) * nzw + coords[:, 2] // zw
    mult = np.ones((coords.shape[0], 3), dtype=np.float64)
    mult[np.arange(coords.shape[0]), axis[zid]] = rho[zid]
    return mult


def _field(w: Workload, seed: int, tag: int, b: int, h: int, coords: np.ndarray,
           mult: Optional[np.ndarray]) -> torch.Tensor:
    """One head's smooth field plus noise, float32 [N, d]."""
    f = w.field
    d, M = w.d, f.M
    rng = _rng(seed, tag, b, h)
    if f.kind == "global":
        freq = _log_uniform(rng, f.f_lo, f.f_hi, (d, M, 3))
    else:
        f0 = _log_uniform(rng, f.f_lo, f.f_hi, (d, M))
        freq = np.repeat(f0[:, :, None], 3, axis=2)
    sign = rng.choice(np.array([-1.0, 1.0]), size=(d, M, 3))
    phase = rng.uniform(0.0, 2.0 * math.pi, size=(d, M))
    noise = rng.standard_normal((coords.shape[0], d), dtype=np.float32) * np.float32(f.noise_std)

    F = torch.from_numpy((freq * sign).reshape(d * M, 3))           # float64 [dM, 3]
    Y = coords.astype(np.float64)
    if mult is not None:
        Y = Y * mult
    Y = torch.from_numpy(Y)
    ph = torch.from_numpy(phase.reshape(1, d * M).astype(np.float32))
    out = torch.empty((coords.shape[0], d), dtype=torch.float32)
    step = 8192
    for s in range(0, coords.shape[0], step):
        cyc = Y[s:s + step] @ F.T                                   # float64 cycles
        cyc = (cyc - torch.floor(cyc)).to(torch.float32)
        val = torch.sin(cyc * np.float32(2.0 * math.pi) + ph)
        out[s:s + step] = val.view(-1, d, M).sum(dim=2) * np.float32(f.amplitude)
    out += torch.from_numpy(noise)
    return out


def _blobs(w: Workload, seed: int, b: int):
    rng = _rng(seed, TAG_BLOBS, b, 0)
    T, H, W = w.grid
    bl = w.blobs
    mu = rng.uniform(0.0, 1.0, size=(bl.n, 3)) * np.array([T, H, W], dtype=np.float64)
    sigma = rng.uniform(bl.sigma_lo, bl.sigma_hi, size=bl.n)
    start = rng.integers(0, w.n_audio - bl.window + 1, size=bl.n)
    return mu, sigma, start


def _a2v(w: Workload, seed: int, b: int, h: int, q: torch.Tensor, coords: np.ndarray) -> torch.Tensor:
    """Dense A2V cross-attention output for one head, float32 [N, d]."""
    d, Na = w.d, w.n_audio
    ka = torch.from_numpy(_rng(seed, TAG_KA, b, h).standard_normal((Na, d), dtype=np.float32))
    va = torch.from_numpy(_rng(seed, TAG_VA, b, h).standard_normal((Na, d), dtype=np.float32))
    mu, sigma, start = _blobs(w, seed, b)
    bl = w.blobs
    X = coords.astype(np.float64)
    bias_tok = np.zeros((coords.shape[0], bl.n), dtype=np.float64)
    for i in range(bl.n):
        r2 = ((X - mu[i]) ** 2).sum(axis=1)
        bias_tok[:, i] = bl.beta * np.exp(-r2 / (2.0 * sigma[i] ** 2))
    win = np.zeros((bl.n, Na), dtype=np.float64)
    for i in range(bl.n):
        win[i, start[i]:start[i] + bl.window] = 1.0
    bias = torch.from_numpy((bias_tok @ win).astype(np.float32))    # [N, Na]
    out = torch.empty((coords.shape[0], d), dtype=torch.float32)
    inv = np.float32(1.0 / math.sqrt(d))
    step = 16384
    for s in range(0, coords.shape[0], step):
        logits = (q[s:s + step] @ ka.T) * inv + bias[s:s + step]
        out[s:s + step] = torch.softmax(logits, dim=1) @ va
    return out


def make_inputs(w: Workload, seed: int, heads: Optional[Iterable[int]] = None,
                q_gain: Optional[float] = None, with_grad: bool = True) -> Dict[str, torch.Tensor]:
    """Seeded inputs on the CPU.  Returns q, k, v, a2v (and do) as [B, Hs, N, d] tensors
    in the workload's dtype, where Hs counts the requested heads (all by default).
    Requesting a subset of heads gives exactly those heads of the full draw."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    gain = w.q_gain if q_gain is None else q_gain
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    coords = token_coords(w.grid)
    B, N, d = w.B, w.N, w.d
    names = ["q", "k", "v", "a2v"] + (["do"] if with_grad else [])
    out = {n: torch.empty((B, len(heads), N, d), dtype=dt) for n in names}
    for b in range(B):
        for hi, h in enumerate(heads):
            mult = _zone_multipliers(w, seed, b, h, coords) if w.field.kind == "zoned" else None
            q = _field(w, seed, TAG_Q, b, h, coords, mult)
            out["a2v"][b, hi] = _a2v(w, seed, b, h, q, coords).to(dt)
            out["q"][b, hi] = (q * np.float32(gain)).to(dt)
            out["k"][b, hi] = _field(w, seed, TAG_K, b, h, coords, mult).to(dt)
            out["v"][b, hi] = _field(w, seed, TAG_V, b, h, coords, mult).to(dt)
            if with_grad:
                g = _rng(seed, TAG_DO, b, h).standard_normal((N, d), dtype=np.float32)
                out["do"][b, hi] = torch.from_numpy(g).to(dt)
    return out
