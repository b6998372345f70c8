"""The synthetic workloads: sizes, candidate shapes and selection parameters.

Every entry is a plain description of a workload.  Nothing here computes any part of
the Prism method; the numbers are the workload recipe (grid, zone size, candidate
block shapes, Top-k/Top-p parameters, recipe of the synthetic fields).

Shape notation follows the block-shape proportion table of the thelatestinai page
(Table 11 caption): a shape is written b_T b_H b_W, e.g. "824" is b_T=8, b_H=2, b_W=4.
Within one candidate set every shape holds the same number of tokens (C_64, C_128,
C_256 in Tables 9 and 11).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

Shape = Tuple[int, int, int]

# 16-token candidate set of the tiny fp32 workload.
CANDS_16: List[Shape] = [(1, 4, 4), (2, 2, 4), (2, 4, 2), (4, 2, 2)]
# 64-token candidate set used by every bf16 workload (list order = tie-break order).
CANDS_64: List[Shape] = [
    (1, 8, 8), (2, 4, 8), (2, 8, 4), (4, 4, 4),
    (1, 4, 16), (1, 16, 4), (4, 2, 8), (4, 8, 2),
]


# The 128- and 256-token candidate sets of the block-shape proportion table (Table 11
# codes b_T b_H b_W, list order = the table's column order).  In the 4x16x16 zones of the
# bf16 workloads only shapes with b_T <= 4 tile a zone: 288, 448, 484 and 488.
CANDS_128: List[Shape] = [(2, 8, 8), (8, 2, 8), (8, 8, 2), (4, 4, 8), (4, 8, 4), (8, 4, 4)]
CANDS_256: List[Shape] = [(4, 8, 8), (8, 4, 8), (8, 8, 4)]


@dataclass(frozen=True)
class FieldRecipe:
    """Recipe of the smooth Q/K/V fields: a sum of M sinusoids per (b, h, channel).

    kind == "global": each sinusoid's per-axis frequency is drawn log-uniform on
    [f_lo, f_hi] (cycles per token), with a random sign per axis.
    kind == "zoned": each sinusoid draws one base frequency f0 log-uniform on
    [f_lo, f_hi]; each (b, h, zone) draws a dominant axis and a ratio rho
    log-uniform on [1, rho_hi]; inside that zone the dominant axis runs at f0*rho
    and the other two at f0.
    """

    kind: str
    M: int
    f_lo: float
    f_hi: float
    rho_hi: float = 8.0
    amplitude: float = 1.0
    noise_std: float = 0.1


@dataclass(frozen=True)
class BlobRecipe:
    """Sound-producing regions that drive the audio-to-video coupling."""

    n: int
    sigma_lo: float
    sigma_hi: float
    beta: float = 8.0      # logit boost of the blob's audio window
    window: int = 4        # audio tokens per window


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    d: int
    grid: Tuple[int, int, int]       # (T, H, W) video latent grid
    zone: Tuple[int, int, int]       # (zt, zh, zw) macro-zone extents
    cands: Tuple[Shape, ...]
    n_audio: int
    dtype: str                       # "f32" or "bf16"
    field: FieldRecipe
    blobs: BlobRecipe
    top_p: float
    k_min: int
    k_max: int
    q_gain: float = 1.0              # scalar gain on Q (density calibration)
    density_target: Tuple[float, float] | None = None

    @property
    def N(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def vol(self) -> int:
        bt, bh, bw = self.cands[0]
        return bt * bh * bw


WORKLOADS: List[Workload] = [
    Workload(
        name="tiny-fp32", B=1, heads=2, d=64, grid=(4, 8, 8), zone=(2, 4, 8),
        cands=tuple(CANDS_16), n_audio=32, dtype="f32",
        field=FieldRecipe("global", M=4, f_lo=1 / 32, f_hi=1 / 4),
        blobs=BlobRecipe(n=1, sigma_lo=2.0, sigma_hi=2.0),
        top_p=0.9, k_min=2, k_max=8,
    ),
    Workload(
        name="480p-like", B=1, heads=12, d=128, grid=(8, 30, 52), zone=(4, 16, 16),
        cands=tuple(CANDS_64), n_audio=200, dtype="bf16",
        field=FieldRecipe("global", M=8, f_lo=1 / 32, f_hi=1 / 4),
        blobs=BlobRecipe(n=2, sigma_lo=3.0, sigma_hi=3.0),
        top_p=0.9, k_min=8, k_max=64,
    ),
    Workload(
        name="720p-like", B=1, heads=24, d=128, grid=(21, 45, 80), zone=(4, 16, 16),
        cands=tuple(CANDS_64), n_audio=500, dtype="bf16",
        field=FieldRecipe("zoned", M=8, f_lo=1 / 64, f_hi=1 / 16),
        blobs=BlobRecipe(n=3, sigma_lo=3.0, sigma_hi=6.0),
        top_p=0.9, k_min=16, k_max=256,
    ),
    Workload(
        name="1080p-like", B=1, heads=8, d=128, grid=(21, 68, 120), zone=(4, 16, 16),
        cands=tuple(CANDS_64), n_audio=500, dtype="bf16",
        field=FieldRecipe("zoned", M=8, f_lo=1 / 64, f_hi=1 / 16),
        blobs=BlobRecipe(n=3, sigma_lo=3.0, sigma_hi=6.0),
        top_p=0.85, k_min=32, k_max=512,
        q_gain=0.8052, density_target=(0.10, 0.15),     # from oracle/calibrate_gain.py 3
    ),
    Workload(
        name="2k-like", B=1, heads=4, d=128, grid=(21, 90, 160), zone=(4, 16, 16),
        cands=tuple(CANDS_64), n_audio=500, dtype="bf16",
        field=FieldRecipe("zoned", M=8, f_lo=1 / 32, f_hi=1 / 8),
        blobs=BlobRecipe(n=3, sigma_lo=3.0, sigma_hi=6.0),
        top_p=0.85, k_min=32, k_max=768,
        q_gain=1.5092, density_target=(0.09, 0.11),     # from oracle/calibrate_gain.py 4
    ),
    # Forward-only inference at the 2K, 10 s scale (Table 13 caption: about 870K tokens at
    # 2K, 10 s, 24 fps, run on 4 GPUs): 61 latent frames x 90 x 160, the same 4-head share
    # and field recipe as the 2K-like workload, audio scaled to the clip (1,500 tokens),
    # Top-k ceiling raised so that a 10 % density is not clamped.
    Workload(
        name="2k-10s-inference", B=1, heads=4, d=128, grid=(61, 90, 160), zone=(4, 16, 16),
        cands=tuple(CANDS_64), n_audio=1500, dtype="bf16",
        field=FieldRecipe("zoned", M=8, f_lo=1 / 32, f_hi=1 / 8),
        blobs=BlobRecipe(n=3, sigma_lo=3.0, sigma_hi=6.0),
        top_p=0.85, k_min=32, k_max=2048,
        q_gain=1.6818, density_target=(0.09, 0.11),     # from oracle/calibrate_gain.py 5
    ),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def shape_code(s: Shape) -> str:
    """b_T b_H b_W written as one string, e.g. (8, 2, 4) -> "824", (1, 4, 16) -> "1x4x16"."""
    if all(v < 10 for v in s):
        return "".join(str(v) for v in s)
    return "x".join(str(v) for v in s)
