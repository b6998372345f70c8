"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks an oracle function against something other than itself: a value the
pages print, a closed form, a brute-force enumeration, a textbook special case computed
by an independent routine, or central finite differences.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import prism_oracle as O
from workloads import CANDS_16, CANDS_64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SP = O.ShapeParams()


def _grid_field(grid, fn, C=1):
    """X [1, 1, N, C] with X[n, c] = fn(t, h, w, c) in token raster order."""
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    cols = [fn(t, h, w, c).ravel() for c in range(C)]
    return np.stack(cols, axis=1)[None, None].astype(np.float64)


def _shape_of(stats, cands=CANDS_64, zone=(4, 16, 16), dtype=np.float32):
    sid, margin = O.assign_shapes(stats, cands, zone, SP, dtype)
    return [cands[i] for i in sid.ravel()], margin.ravel()


# ------------------------------------------------------------------ pages' values
def test_table11_shape_codes_have_equal_volume_per_set():
    sets, rows = {}, []
    for line in open(os.path.join(GOLDEN, "table11_shape_codes.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "ROW":
            rows.append([float(x) for x in f[2:]])
        else:
            sets[f[0]] = (int(f[1]), [O.parse_shape_code(c) for c in f[2:]])
    assert O.parse_shape_code("824") == (8, 2, 4)
    for name, (vol, shapes) in sets.items():
        assert O.candidate_volume(shapes) == vol, name
    # mixing two sets must be rejected
    with pytest.raises(ValueError):
        O.candidate_volume(sets["C_64"][1] + sets["C_128"][1])
    for r in rows:
        assert abs(sum(r) - 100.0) < 1e-9
    assert O.candidate_volume(CANDS_64) == 64 and O.candidate_volume(CANDS_16) == 16
    # the 128- and 256-token workload sets are exactly the table's codes, in its order
    from workloads import CANDS_128, CANDS_256
    assert CANDS_128 == sets["C_128"][1] and CANDS_256 == sets["C_256"][1]


# ------------------------------------------------------------------ zones
def test_zone_view_tiles_every_token_once():
    grid, zone = (5, 7, 9), (2, 4, 4)
    N = 5 * 7 * 9
    X = (np.arange(N, dtype=np.float64) + 1.0)[None, None, :, None]
    Xz, mask = O.zone_view(X, grid, zone)
    vals = Xz[0, 0, ..., 0][mask]
    assert sorted(vals.tolist()) == list(range(1, N + 1))
    assert (Xz[0, 0, ..., 0][~mask] == 0).all()
    assert Xz.shape[2] == 3 * 2 * 3


def test_semivariance_of_sinusoids_matches_closed_form():
    # One 4x16x16 zone.  Channel 0 varies along t with period 3 (3 pairs = 1 period),
    # channel 1 along h with period 5 (15 pairs = 3 periods), channel 2 along w with
    # period 15; over whole periods gamma = A^2 sin^2(omega/2) on that axis, 0 elsewhere.
    grid = zone = (4, 16, 16)
    A = [2.0, 0.7, 1.3]
    om = [2 * math.pi / 3, 2 * math.pi / 5, 2 * math.pi / 15]
    ph = [0.3, 1.1, 2.0]

    def fn(t, h, w, c):
        x = (t, h, w)[c]
        return A[c] * np.sin(om[c] * x + ph[c])

    V = _grid_field(grid, fn, C=3)
    Vz, mask = O.zone_view(V[0, 0], grid, zone)
    g = O.directional_semivariance(Vz, mask)[0]          # [3 axes, 3 channels]
    for c in range(3):
        for d in range(3):
            want = A[c] ** 2 * math.sin(om[c] / 2) ** 2 if d == c else 0.0
            assert abs(g[d, c] - want) < 1e-12, (d, c, g[d, c], want)


def test_video_share_of_separable_field_matches_closed_form():
    grid = zone = (4, 16, 16)
    w1, w2 = 2 * math.pi / 3, 2 * math.pi / 5
    V = _grid_field(grid, lambda t, h, w, c: np.sin(w1 * t) + 0.5 * np.sin(w2 * h + 0.4), C=2)
    a2v = np.ones_like(V)
    st = O.zone_stats(V, a2v, grid, zone)[0, 0, 0]
    gt, gh = math.sin(w1 / 2) ** 2, 0.25 * math.sin(w2 / 2) ** 2
    assert abs(st[0] - gt / (gt + gh)) < 1e-9
    assert abs(st[1] - gh / (gt + gh)) < 1e-9
    assert abs(st[2]) < 1e-9
    assert abs(st[0] + st[1] + st[2] - 1.0) < 1e-9


def test_global_variance_share_matches_closed_form():
    # Channel 0 varies along t only (amplitude 2, period 3), channel 1 along h only
    # (amplitude 0.5, period 5).  Per channel the shares are (1,0,0) and (0,1,0), so their
    # mean is (1/2, 1/2, 0) whatever the amplitudes; jointly across channels the axes weigh
    # by each channel's semivariance A^2 sin^2(omega/2), which the global variant must give.
    grid = zone = (4, 16, 16)
    w1, w2 = 2 * math.pi / 3, 2 * math.pi / 5
    V = _grid_field(grid, lambda t, h, w, c: 2.0 * np.sin(w1 * t + 0.2) if c == 0 else 0.5 * np.sin(w2 * h + 0.9),
                    C=2)
    a2v = np.ones_like(V)
    per = O.zone_stats(V, a2v, grid, zone)[0, 0, 0]
    glo = O.zone_stats(V, a2v, grid, zone, global_variance=True)[0, 0, 0]
    assert np.allclose(per[:3], [0.5, 0.5, 0.0], atol=1e-9)
    gt, gh = 4.0 * math.sin(w1 / 2) ** 2, 0.25 * math.sin(w2 / 2) ** 2
    assert np.allclose(glo[:3], [gt / (gt + gh), gh / (gt + gh), 0.0], atol=1e-9)
    assert np.array_equal(per[3:], glo[3:])           # the audio statistics do not change


def test_a2v_norm_special_cases_and_bruteforce():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 7, 4))
    va = rng.standard_normal((1, 2, 5, 4))
    # one audio key: every query's output is that key's value row
    a1 = O.a2v_norm(q, rng.standard_normal((1, 2, 1, 4)), va[:, :, :1])
    assert np.allclose(a1, np.linalg.norm(va[:, :, 0], axis=-1)[..., None].repeat(7, axis=-1), atol=1e-12)
    # identical keys: uniform weights, output = mean value row
    ka = np.repeat(rng.standard_normal((1, 2, 1, 4)), 5, axis=2)
    a2 = O.a2v_norm(q, ka, va)
    assert np.allclose(a2, np.linalg.norm(va.mean(axis=2), axis=-1)[..., None].repeat(7, axis=-1), atol=1e-12)
    # explicit loops
    ka = rng.standard_normal((1, 2, 5, 4))
    a3 = O.a2v_norm(q, ka, va, scale=0.3)
    for h in range(2):
        for x in range(7):
            w = [math.exp(0.3 * float(q[0, h, x] @ ka[0, h, j])) for j in range(5)]
            o = sum(wj * va[0, h, j] for j, wj in enumerate(w)) / sum(w)
            assert abs(a3[0, h, x] - math.sqrt(float(o @ o))) < 1e-12


def test_zone_stats_from_norm_map_equals_from_rows():
    rng = np.random.default_rng(5)
    grid, zone = (5, 6, 7), (2, 4, 4)
    N = 5 * 6 * 7
    V = rng.standard_normal((1, 2, N, 3))
    A = rng.standard_normal((1, 2, N, 4))
    a = np.linalg.norm(A, axis=-1)[..., None]
    for gv in (False, True):
        assert np.allclose(O.zone_stats(V, A, grid, zone, global_variance=gv),
                           O.zone_stats(V, a, grid, zone, global_variance=gv), rtol=1e-13, atol=1e-13)


def test_zone_activity_closed_form():
    # channel 0 varies along t (amplitude 2, period 3), channel 1 along h (amplitude 0.5,
    # period 5): activity = mean over the 2 channels of each axis's semivariance, summed
    grid = zone = (4, 16, 16)
    w1, w2 = 2 * math.pi / 3, 2 * math.pi / 5
    V = _grid_field(grid, lambda t, h, w, c: 2.0 * np.sin(w1 * t + 0.2) if c == 0 else 0.5 * np.sin(w2 * h + 0.9),
                    C=2)
    act = O.zone_activity(V, grid, zone)[0, 0, 0]
    want = (4.0 * math.sin(w1 / 2) ** 2 + 0.25 * math.sin(w2 / 2) ** 2) / 2
    assert abs(act - want) < 1e-12
    assert O.zone_activity(np.ones_like(V), grid, zone)[0, 0, 0] == 0.0


def _multi_stats(rows):
    """stats rows [r_t, r_h, r_w, g_t, g_h, g_w, m, n] for one head, as [1, 1, nZ, 8]."""
    return np.array(rows, dtype=np.float64)[None, None]


def test_assign_multi_volume_classes_and_fallback():
    from workloads import CANDS_128, CANDS_256
    cands = CANDS_64 + CANDS_128 + CANDS_256
    zone = (4, 16, 16)
    iso = [1 / 3, 1 / 3, 1 / 3, 1.0, 1.0, 1.0]
    # four zones, equal audio norm (gate 0): activities 0.2, 0.75, 1.5, 1.55 of a mean 1
    st = _multi_stats([iso + [1.0, 1024]] * 4)
    vact = np.array([[[0.2, 0.75, 1.5, 1.55]]])
    sid, margin = O.assign_shapes_multi(st, vact, cands, zone)
    vols = [int(np.prod(cands[i])) for i in sid[0, 0]]
    assert vols == [256, 128, 64, 64]
    # isotropic guidance picks the most cubic shape of each volume that tiles the zone
    assert cands[sid[0, 0, 0]] == (4, 8, 8) and cands[sid[0, 0, 2]] == (4, 4, 4)
    # the audio gate lifts a smooth zone to the finest blocks: m_z = 2x the head mean
    st2 = _multi_stats([iso + [3.0, 1024], iso + [1.0, 1024], iso + [1.0, 1024], iso + [1.0, 1024]])
    sid2, _ = O.assign_shapes_multi(st2, vact, cands, zone)
    assert int(np.prod(cands[sid2[0, 0, 0]])) == 64            # act = 0.2 + 1
    # no 256-token shape tiles the zone -> 128 (and without 128 shapes -> 64)
    sid3, _ = O.assign_shapes_multi(st, vact, CANDS_64 + CANDS_128 + [(8, 4, 8)], zone)
    assert int(np.prod((CANDS_64 + CANDS_128 + [(8, 4, 8)])[sid3[0, 0, 0]])) == 128
    sid4, _ = O.assign_shapes_multi(st, vact, CANDS_64 + [(8, 4, 8)], zone)
    assert int(np.prod((CANDS_64 + [(8, 4, 8)])[sid4[0, 0, 0]])) == 64
    # an activity on a threshold is a near-tie
    _, m5 = O.assign_shapes_multi(st, np.array([[[0.5, 1.0, 1.5, 1.0]]]), cands, zone)
    assert m5[0, 0, 0] < O.NEAR_TIE and m5[0, 0, 1] < O.NEAR_TIE


def test_mixed_volume_slot_map_and_dense_equivalence():
    """Zones with 64-, 128- and 256-token blocks on a ragged grid: every token in exactly
    one slot, block heads carry whole-block counts, and with every block selected the chain
    reproduces dense attention."""
    from workloads import CANDS_128, CANDS_256
    cands = CANDS_64 + CANDS_128 + CANDS_256
    rng = np.random.default_rng(4)
    grid, zone = (6, 20, 18), (4, 16, 16)
    N = 6 * 20 * 18
    nZ = O.num_zones(grid, zone)
    sid = np.array([[[3, 11, 14, 8, 0, 14, 12, 1]]], dtype=np.int32)[:, :, :nZ]      # 64/128/256 mixed
    tok = O.slot_map(grid, zone, cands, sid)
    assert sorted(tok[0, 0][tok[0, 0] >= 0].tolist()) == list(range(N))
    bv = O.block_heads(tok, sid, cands, zone)
    assert bv.sum() == N and bv.max() <= 256
    for z in range(nZ):
        g = int(np.prod(cands[sid[0, 0, z]])) // 64
        heads = bv[0, 0, z * 16:(z + 1) * 16]
        assert (heads.reshape(-1, g)[:, 1:] == 0).all()
    q, k, v, a2v = (rng.standard_normal((1, 1, N, 8)) for _ in range(4))
    f = O.prism_forward(q, k, v, a2v, grid, zone, cands, 1.0, 10 ** 6, 10 ** 6, scale=0.4, dtype=np.float64,
                        shape_id=sid, mixed=(O.TAU_128, O.TAU_256))
    want, _ = O.dense_attn_fwd(q, k, v, 0.4)
    assert np.allclose(f["o"], want, atol=1e-12)


def test_zone_stats_vectorised_equals_bruteforce_on_ragged_grid():
    rng = np.random.default_rng(7)
    grid, zone = (5, 6, 7), (2, 4, 4)
    N = 5 * 6 * 7
    V = rng.standard_normal((1, 2, N, 3))
    A = rng.standard_normal((1, 2, N, 4))
    a = O.zone_stats(V, A, grid, zone)
    b = O.zone_stats_bruteforce(V, A, grid, zone)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    assert a[..., 7].sum() == 2 * N
    ag = O.zone_stats(V, A, grid, zone, global_variance=True)
    bg = O.zone_stats_bruteforce(V, A, grid, zone, global_variance=True)
    assert np.allclose(ag, bg, rtol=1e-12, atol=1e-12)


def test_audio_norm_statistics_closed_form():
    grid = zone = (4, 16, 16)
    # a2v rows of norm 3 (all tokens): m_z = 3, increments zero.
    A = np.zeros((1, 1, 4 * 16 * 16, 2))
    A[..., 0] = 3.0
    st = O.zone_stats(np.zeros_like(A), A, grid, zone)[0, 0, 0]
    assert abs(st[6] - 3.0) < 1e-12 and np.allclose(st[3:6], 0)
    # a norm ramp a = 2h along h: gamma_h = 1/2 * 2^2 = 2, nothing along t, w.
    A = _grid_field(grid, lambda t, h, w, c: 2.0 * h + 0 * c, C=1)
    st = O.zone_stats(np.zeros_like(A), A, grid, zone)[0, 0, 0]
    assert np.allclose(st[3:6], [0.0, 2.0, 0.0], atol=1e-12)
    assert abs(st[6] - 15.0) < 1e-12


# ------------------------------------------------------------------ shapes
def _stats_row(rv, ga=(0, 0, 0), m=1.0, n=1024):
    return np.array([[[list(rv) + list(ga) + [m, n]]]], dtype=np.float64)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_shape_special_cases(dtype):
    # flat zone -> cube; variation along one axis only -> the block is thinnest there.
    cases = {(0, 0, 0): (4, 4, 4), (1, 0, 0): (1, 8, 8), (0, 1, 0): (4, 2, 8), (0, 0, 1): (4, 8, 2),
             (0, 0.5, 0.5): (4, 4, 4)}
    for rv, want in cases.items():
        got, _ = _shape_of(_stats_row(rv), dtype=dtype)
        assert got[0] == want, (rv, got, want)


def test_shape_from_fields_single_axis():
    grid = zone = (4, 16, 16)
    flat = np.ones((1, 1, 1024, 4))
    fields = {
        0: (lambda t, h, w, c: np.sin(2.1 * t + c), (1, 8, 8)),
        1: (lambda t, h, w, c: np.sin(1.3 * h + c), (4, 2, 8)),
        2: (lambda t, h, w, c: np.sin(1.3 * w + c), (4, 8, 2)),
    }
    for _, (fn, want) in fields.items():
        V = _grid_field(grid, fn, C=4)
        st = O.zone_stats(V, flat, grid, zone)
        got, _ = _shape_of(st)
        assert got[0] == want
    st = O.zone_stats(np.full((1, 1, 1024, 4), 0.25), flat, grid, zone)
    assert _shape_of(st)[0][0] == (4, 4, 4)


def test_shape_is_equivariant_under_h_w_swap():
    rng = np.random.default_rng(3)
    grid = zone = (4, 16, 16)
    swap = {c: (c[0], c[2], c[1]) for c in CANDS_64}
    for trial in range(20):
        V = rng.standard_normal((4, 16, 16, 8)).cumsum(axis=rng.integers(0, 3)) * rng.uniform(0.1, 2)
        V = V * np.linspace(0.2, 2.0, 16)[None, None, :, None] ** rng.uniform(0, 3)
        Vt = V.transpose(0, 2, 1, 3)
        flat = np.ones((1, 1, 1024, 2))
        s1 = O.zone_stats(V.reshape(1, 1, 1024, 8), flat, grid, zone)
        s2 = O.zone_stats(Vt.reshape(1, 1, 1024, 8), flat, grid, zone)
        (c1,), (m1,) = _shape_of(s1, dtype=np.float64)
        (c2,), (m2,) = _shape_of(s2, dtype=np.float64)
        if m1 > 1e-6:
            assert swap[c1] == c2


def test_ideal_extents_preserve_volume_and_order():
    rng = np.random.default_rng(0)
    g = rng.uniform(1e-3, 1.0, size=(100, 3))
    lam = O.ideal_log_extents(g, 64, 0.5, np.float64)
    assert np.allclose(lam.sum(axis=1), 6.0, atol=1e-12)
    for i in range(100):
        o = np.argsort(g[i])
        assert lam[i, o[0]] >= lam[i, o[1]] >= lam[i, o[2]]     # faster variation -> thinner
    # hand value: g = (1/2, 1/4, 1/4) -> log2 g = (-1, -2, -2), mean -5/3
    lam = O.ideal_log_extents(np.array([[0.5, 0.25, 0.25]]), 64, 0.5, np.float64)[0]
    assert np.allclose(lam, [2 - 1 / 3, 2 + 1 / 6, 2 + 1 / 6], atol=1e-12)


def test_gate_closed_form():
    # zones with mean norms 1, 1, 3, 1 of equal size: head mean 1.5, ratios 2/3, 2/3, 2, 2/3
    st = np.zeros((1, 1, 4, 8))
    st[0, 0, :, 0:3] = (0.0, 0.0, 1.0)          # video alone would pick 4x8x2
    st[0, 0, :, 3:6] = (0.0, 5.0, 0.0)          # audio varies along h
    st[0, 0, :, 6] = (1.0, 1.0, 3.0, 1.0)
    st[0, 0, :, 7] = 256
    abar, vhat, g = O.shape_guidance(st, SP, np.float64)
    assert np.allclose(abar[0, 0], [0, 0, 1, 0])
    assert np.allclose(vhat[0, 0, 2], [0, 1, 0], atol=1e-9)
    got, _ = _shape_of(st)
    assert got == [(4, 8, 2), (4, 8, 2), (4, 2, 8), (4, 8, 2)]
    # gate halfway: ratio 1.5 -> a-bar = 0.5
    st[0, 0, :, 6] = (1.0, 1.0, 2.0, 0.0)        # mean 1, ratios 1, 1, 2, 0
    abar, _, _ = O.shape_guidance(st, SP, np.float64)
    assert np.allclose(abar[0, 0], [0, 0, 1, 0])
    st[0, 0, :, 6] = (1.0, 1.0, 1.5, 0.5)        # mean 1, ratio 1.5 -> 0.5
    abar, _, _ = O.shape_guidance(st, SP, np.float64)
    assert np.allclose(abar[0, 0], [0, 0, 0.5, 0])
    # uniform norms -> gate closed everywhere
    st[0, 0, :, 6] = 2.0
    abar, _, _ = O.shape_guidance(st, SP, np.float64)
    assert (abar == 0).all()


def test_infeasible_candidate_is_never_chosen():
    # tiny workload: zone 2x4x8 cannot hold the 4x2x2 candidate (b_T = 4 > 2)
    assert not O.feasible((4, 2, 2), (2, 4, 8))
    st = _stats_row((0.0, 1.0, 1.0))            # ideal is long along t
    sid, _ = O.assign_shapes(st, CANDS_16, (2, 4, 8), SP)
    assert CANDS_16[int(sid.ravel()[0])] != (4, 2, 2)


# ------------------------------------------------------------------ permutation
def test_slot_map_hand_example():
    grid, zone = (1, 2, 3), (1, 2, 4)
    cands = [(1, 2, 2), (1, 1, 4)]
    tok = O.slot_map(grid, zone, cands, np.array([[[0]]]))
    assert tok[0, 0].tolist() == [0, 1, 3, 4, 2, 5, -1, -1]
    tok = O.slot_map(grid, zone, cands, np.array([[[1]]]))
    assert tok[0, 0].tolist() == [0, 1, 2, -1, 3, 4, 5, -1]
    assert O.block_valid(tok, 4).tolist() == [[[3, 3]]]


def test_slot_map_tiles_each_zone_exactly():
    rng = np.random.default_rng(1)
    grid, zone = (8, 30, 52), (4, 16, 16)
    nZ = O.num_zones(grid, zone)
    sid = rng.integers(0, 8, size=(1, 3, nZ))
    tok = O.slot_map(grid, zone, CANDS_64, sid)
    N = 8 * 30 * 52
    T, H, W = grid
    for h in range(3):
        t = tok[0, h]
        v = t[t >= 0]
        assert sorted(v.tolist()) == list(range(N))
        for z in range(nZ):                      # each zone's slots hold exactly its tokens
            zt_ = t[z * 1024:(z + 1) * 1024]
            zt_ = zt_[zt_ >= 0]
            tt, hh, ww = zt_ // (H * W), (zt_ // W) % H, zt_ % W
            zid = ((tt // 4) * 2 + hh // 16) * 4 + ww // 16
            assert (zid == z).all()
            for blk in range(16):                # each block is a box of its shape
                bt, bh, bw = CANDS_64[sid[0, h, z]]
                s = t[z * 1024 + blk * 64: z * 1024 + blk * 64 + 64]
                s = s[s >= 0]
                if s.size:
                    ext = [np.ptp(s // (H * W)) + 1, np.ptp((s // W) % H) + 1, np.ptp(s % W) + 1]
                    assert ext[0] <= bt and ext[1] <= bh and ext[2] <= bw
                    assert ext[0] * ext[1] * ext[2] == s.size
        bv = O.block_valid(tok, 64)[0, h]
        assert bv.sum() == N and bv.max() == 64


def test_permute_unpermute_is_identity():
    rng = np.random.default_rng(2)
    grid, zone = (8, 30, 52), (4, 16, 16)
    N = 8 * 30 * 52
    x = rng.standard_normal((1, 2, N, 5)).astype(np.float32)
    sid = rng.integers(0, 8, size=(1, 2, O.num_zones(grid, zone)))
    tok = O.slot_map(grid, zone, CANDS_64, sid)
    y = O.permute(x, tok)
    assert (O.unpermute(y, tok, N) == x).all()
    assert (y[tok < 0] == 0).all()


def test_pooling_bruteforce():
    rng = np.random.default_rng(4)
    xp = rng.standard_normal((1, 2, 64, 3))
    bv = np.array([[[16, 5, 0, 9], [1, 16, 16, 2]]], dtype=np.int32)
    got = O.pool_blocks(xp, bv, 16)
    for h in range(2):
        for I in range(4):
            n = bv[0, h, I]
            want = np.zeros(3) if n == 0 else sum(xp[0, h, I * 16 + r] for r in range(n)) / n
            assert np.allclose(got[0, h, I], want, atol=1e-14)
    # blocks identified by their first 16-row unit that run past it (mixed volumes): a
    # 48-row block at unit 0 with 40 valid rows, a 16-row block at unit 3
    bv2 = np.array([[[40, 0, 0, 9], [33, 0, 0, 16]]], dtype=np.int32)
    got2 = O.pool_blocks(xp, bv2, 16)
    for h in range(2):
        for I in range(4):
            n = bv2[0, h, I]
            want = np.zeros(3) if n == 0 else sum(xp[0, h, I * 16 + r] for r in range(n)) / n
            assert np.allclose(got2[0, h, I], want, atol=1e-14)


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_hybrid_count_hand_rows(dtype):
    P = np.array([0.5, 0.25, 0.125, 0.125])
    assert O.hybrid_count(P, 0.9, 1, 4, dtype)[0] == 4       # .5 .75 .875 1.0
    assert O.hybrid_count(P, 0.75, 1, 4, dtype)[0] == 3      # strictly exceeds: .75 is not > .75
    assert O.hybrid_count(P, 0.7, 1, 4, dtype)[0] == 2
    assert O.hybrid_count(P, 1e-6, 1, 4, dtype)[0] == 1
    assert O.hybrid_count(P, 1e-6, 3, 4, dtype)[0] == 3      # Top-k floor
    assert O.hybrid_count(P, 0.9, 1, 2, dtype)[0] == 2       # Top-k ceiling
    assert O.hybrid_count(P, 1.0, 1, 9, dtype) == (4, 4)     # nothing exceeds 1 -> all live
    P = np.array([0.5, 0.3, 0.15, 0.05])
    assert O.hybrid_count(P, 0.9, 1, 8, dtype)[0] == 3


def test_top_p_one_keeps_every_live_block():
    """Top-p at p = 1 (Table 7 caption: the smallest set whose cumulative weight exceeds
    the threshold): weights that sum to 1 have no prefix exceeding 1, so every live block
    stays, also when the float32 running sum rounds above 1 before the last block, and the
    Top-k floor alone does not cut the row."""
    P = np.array([0.6, 0.4000001, 1e-9, 1e-9], dtype=np.float32)
    assert np.cumsum(P, dtype=np.float32)[1] > np.float32(1.0)      # the float32 sum overshoots at n = 2
    assert O.hybrid_count(P, 1.0, 1, 8, np.float32) == (4, 4)
    # a whole selection row: softmax of many logits, Top-p 1 with k_min 1 keeps all live blocks
    rng = np.random.default_rng(3)
    nb, d = 600, 16
    qb = rng.standard_normal((1, 1, nb, d)).astype(np.float32)
    kb = rng.standard_normal((1, 1, nb, d)).astype(np.float32)
    bv = np.full((1, 1, nb), 4, dtype=np.int32)
    bv[0, 0, ::7] = 0
    live = np.nonzero(bv[0, 0] > 0)[0]
    sel, near = O.select_blocks_all(qb, kb, bv, 0.25, 1.0, 1, nb)
    for I in live:
        assert sel[(0, 0, int(I))].tolist() == live.tolist()
        assert not near[(0, 0, int(I))]
    sel_r, _ = O.select_blocks(qb, kb, bv, 0.25, 1.0, 1, nb, rows=[int(live[0])])
    assert sel_r[(0, 0, int(live[0]))].tolist() == live.tolist()


def test_top_p_is_smallest_subset_by_bruteforce():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(2, 9))
        P = rng.dirichlet(np.full(n, rng.uniform(0.2, 2.0)))
        p = float(rng.uniform(0.05, 0.99))
        best = n
        for r in range(1, n + 1):
            if any(sum(P[list(c)]) > p + 1e-12 for c in itertools.combinations(range(n), r)):
                best = r
                break
        got = O.hybrid_count(np.sort(P)[::-1], p, 1, n, np.float64)[1]
        if all(abs(sum(sorted(P, reverse=True)[:r]) - p) > 1e-9 for r in range(1, n + 1)):
            assert got == best


def test_select_row_topk_and_topp_against_independent_sorts():
    rng = np.random.default_rng(6)
    d = 16
    for trial in range(50):
        nb = int(rng.integers(3, 40))
        K = rng.standard_normal((nb, d)) * rng.uniform(0.1, 3)
        q = rng.standard_normal(d)
        live = rng.uniform(size=nb) > 0.2
        live[0] = True
        J = np.nonzero(live)[0]
        s = K[J] @ q / 4.0
        P = np.exp(s - s.max())
        P /= P.sum()
        k = int(rng.integers(1, J.size + 1))
        sel, _ = O.select_row(q, K, live, 0.25, 1.0, k, k, np.float64)
        want = sorted(sorted(range(J.size), key=lambda i: (-P[i], J[i]))[:k])
        assert sel.tolist() == [int(J[i]) for i in want]
        p = float(rng.uniform(0.1, 0.95))
        sel, near = O.select_row(q, K, live, 0.25, p, 1, J.size, np.float64)
        order = sorted(range(J.size), key=lambda i: (-P[i], J[i]))
        acc, n = 0.0, J.size
        for r, i in enumerate(order):
            acc += P[i]
            if acc > p:
                n = r + 1
                break
        if not near:
            assert sel.tolist() == sorted(int(J[i]) for i in order[:n])


def test_select_flags_exact_tie_at_cut():
    K = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 0.0]])
    sel, near = O.select_row(np.array([2.0, 0.0]), K, np.ones(3, bool), 1.0, 0.3, 1, 3, np.float64)
    assert sel.tolist() == [0] and near          # blocks 0 and 1 tie; lower index wins


def test_reverse_index_bruteforce():
    rng = np.random.default_rng(8)
    nb, kmax = 12, 5
    sel = {}
    for I in range(nb):
        c = int(rng.integers(0, kmax + 1))
        sel[(0, 0, I)] = np.sort(rng.choice(nb, size=c, replace=False)).astype(np.int32)
    idx, cnt = O.selection_arrays(sel, 1, 1, nb, kmax)
    rp, ri = O.reverse_index(idx, cnt)
    for J in range(nb):
        want = [I for I in range(nb) if J in sel[(0, 0, I)].tolist()]
        assert ri[0, 0, rp[0, 0, J]:rp[0, 0, J + 1]].tolist() == want


# ------------------------------------------------------------------ attention
def _tiny_problem(seed=0, C=8):
    rng = np.random.default_rng(seed)
    grid, zone, cands = (4, 8, 8), (2, 4, 8), list(CANDS_16)
    N = 256
    q, k, v = (rng.standard_normal((1, 2, N, C)) for _ in range(3))
    sid = rng.integers(0, 3, size=(1, 2, O.num_zones(grid, zone)))
    tok = O.slot_map(grid, zone, cands, sid)
    return q, k, v, tok, N


def _all_selected(bv):
    B, Hh, nb = bv.shape
    return {(b, h, I): (np.nonzero(bv[b, h] > 0)[0].astype(np.int32) if bv[b, h, I] else np.zeros(0, np.int32))
            for b in range(B) for h in range(Hh) for I in range(nb)}


def test_all_blocks_selected_equals_textbook_dense_attention():
    q, k, v, tok, N = _tiny_problem()
    bv = O.block_valid(tok, 16)
    # p = 1 with k_min = k_max = every live block selects all live key blocks
    qp, kp, vp = O.permute(q, tok), O.permute(k, tok), O.permute(v, tok)
    qb, kb = O.pool_blocks(qp, bv, 16), O.pool_blocks(kp, bv, 16)
    nl = int((bv[0, 0] > 0).sum())
    sel, _ = O.select_blocks(qb, kb, bv, 0.3, 1.0, nl, nl, dtype=np.float64)
    op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, 0.3, 16)
    o = O.unpermute(op, tok, N)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3).numpy()
    assert np.allclose(o, want, atol=1e-12)
    lse_want = torch.logsumexp(0.3 * tq @ tk.transpose(-1, -2), dim=-1).numpy()
    assert np.allclose(O.unpermute(lse[..., None], tok, N)[..., 0], lse_want, atol=1e-12)
    od, ld = O.dense_attn_fwd(q, k, v, 0.3)
    assert np.allclose(od, want, atol=1e-12) and np.allclose(ld, lse_want, atol=1e-12)


@pytest.mark.parametrize("cands", [[(2, 8, 8), (4, 4, 8), (4, 8, 4)], [(4, 8, 8)]])
def test_large_blocks_all_selected_equal_dense_attention(cands):
    """128- and 256-token blocks (cut by the grid edge, so with padding) through the whole
    chain with every live block selected reproduce dense attention over the real tokens."""
    rng = np.random.default_rng(21)
    grid, zone = (6, 10, 12), (4, 16, 16)
    N = 6 * 10 * 12
    q, k, v = (rng.standard_normal((1, 2, N, 8)) for _ in range(3))
    a2v = rng.standard_normal((1, 2, N, 8))
    vol = O.candidate_volume(cands)
    f = O.prism_forward(q, k, v, a2v, grid, zone, cands, 1.0, 10 ** 6, 10 ** 6, scale=0.4, dtype=np.float64)
    assert f["vol"] == vol and f["bvalid"].max() <= vol
    tok = f["tok"]
    assert sorted(tok[0, 0][tok[0, 0] >= 0].tolist()) == list(range(N))
    want, _ = O.dense_attn_fwd(q, k, v, 0.4)
    assert np.allclose(f["o"], want, atol=1e-12)


def test_single_selected_block_is_attention_inside_that_block():
    q, k, v, tok, N = _tiny_problem(1)
    bv = O.block_valid(tok, 16)
    qp, kp, vp = O.permute(q, tok), O.permute(k, tok), O.permute(v, tok)
    sel = {(0, 0, 3): np.array([5], np.int32)}
    op, _ = O.sparse_attn_fwd(qp, kp, vp, bv, sel, 0.5, 16, blocks=[(0, 0, 3)])
    n, m = bv[0, 0, 3], bv[0, 0, 5]
    Q = torch.from_numpy(qp[0, 0, 48:48 + n])
    K = torch.from_numpy(kp[0, 0, 80:80 + m])
    V = torch.from_numpy(vp[0, 0, 80:80 + m])
    want = torch.softmax(0.5 * Q @ K.T, dim=1) @ V
    assert np.allclose(op[0, 0, 48:48 + n], want.numpy(), atol=1e-12)
    assert (op[0, 0, 48 + n:64] == 0).all()


def test_rows_with_nothing_to_attend_are_zero():
    """Reading of the attention over an empty key set: a block whose list is empty, or holds
    only blocks without valid rows, outputs 0 with LSE 0 and gets no gradient; the other
    blocks are unaffected (each equals softmax attention over its own keys)."""
    rng = np.random.default_rng(3)
    vol, C = 8, 4
    bv = np.array([[[8, 5, 0, 8]]], dtype=np.int32)
    qp, kp, vp, dop = (rng.standard_normal((1, 1, 4 * vol, C)) for _ in range(4))
    for x in (qp, kp, vp, dop):
        for I in range(4):
            x[0, 0, I * vol + bv[0, 0, I]:(I + 1) * vol] = 0.0
    sel = {(0, 0, 0): np.array([], np.int32), (0, 0, 1): np.array([2], np.int32),
           (0, 0, 2): np.array([], np.int32), (0, 0, 3): np.array([0, 2, 3], np.int32)}
    op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, 0.5, vol)
    assert (op[0, 0, :2 * vol] == 0).all() and (lse[0, 0, :2 * vol] == 0).all()
    Q = torch.from_numpy(qp[0, 0, 24:32])
    K = torch.from_numpy(np.concatenate([kp[0, 0, 0:8], kp[0, 0, 24:32]]))
    V = torch.from_numpy(np.concatenate([vp[0, 0, 0:8], vp[0, 0, 24:32]]))
    assert np.allclose(op[0, 0, 24:32], (torch.softmax(0.5 * Q @ K.T, dim=1) @ V).numpy(), atol=1e-12)
    assert np.allclose(lse[0, 0, 24:32], torch.logsumexp(0.5 * Q @ K.T, dim=1).numpy(), atol=1e-12)
    dq, dk, dv = O.sparse_attn_bwd(qp, kp, vp, op, dop, lse, bv, sel, 0.5, vol)
    assert (dq[0, 0, :2 * vol] == 0).all()
    assert (dk[0, 0, 8:24] == 0).all() and (dv[0, 0, 8:24] == 0).all()


def test_backward_matches_central_finite_differences():
    q, k, v, tok, N = _tiny_problem(2, C=4)
    bv = O.block_valid(tok, 16)
    rng = np.random.default_rng(9)
    qp, kp, vp = O.permute(q, tok), O.permute(k, tok), O.permute(v, tok)
    qb, kb = O.pool_blocks(qp, bv, 16), O.pool_blocks(kp, bv, 16)
    sel, _ = O.select_blocks(qb, kb, bv, 0.5, 0.6, 2, 5, dtype=np.float64)   # frozen mask
    dop = O.permute(rng.standard_normal(q.shape), tok)
    op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, 0.5, 16)
    dq, dk, dv = O.sparse_attn_bwd(qp, kp, vp, op, dop, lse, bv, sel, 0.5, 16)

    def loss(a, b_, c):
        return float((O.sparse_attn_fwd(a, b_, c, bv, sel, 0.5, 16)[0] * dop).sum())

    valid = np.nonzero(tok[0, 0] >= 0)[0]
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            s = int(rng.choice(valid))
            c = int(rng.integers(0, 4))
            args = [qp.copy(), kp.copy(), vp.copy()]
            args[which][0, 0, s, c] += h
            lp = loss(*args)
            args[which][0, 0, s, c] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[0, 0, s, c]) <= 1e-6 * max(1.0, abs(fd)), (which, s, c, fd, grad[0, 0, s, c])


def test_backward_all_selected_matches_autograd_dense():
    q, k, v, tok, N = _tiny_problem(3)
    bv = O.block_valid(tok, 16)
    rng = np.random.default_rng(10)
    do = rng.standard_normal(q.shape)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.4)
    (out * torch.from_numpy(do)).sum().backward()
    # dense oracle
    o, lse = O.dense_attn_fwd(q, k, v, 0.4)
    dq, dk, dv = O.dense_attn_bwd(q, k, v, o, do, lse, 0.4)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(a, t.grad.numpy(), atol=1e-10)
    # sparse oracle with every block selected
    qp, kp, vp = O.permute(q, tok), O.permute(k, tok), O.permute(v, tok)
    sel = _all_selected(bv)
    op, lsp = O.sparse_attn_fwd(qp, kp, vp, bv, sel, 0.4, 16)
    g = O.sparse_attn_bwd(qp, kp, vp, op, O.permute(do, tok), lsp, bv, sel, 0.4, 16)
    for a, t in zip(g, (tq, tk, tv)):
        assert np.allclose(O.unpermute(a, tok, N), t.grad.numpy(), atol=1e-10)
    # restricting the gradient to some blocks gives those blocks' rows unchanged
    gq = O.sparse_attn_bwd(qp, kp, vp, op, O.permute(do, tok), lsp, bv, sel, 0.4, 16,
                           q_blocks=[(0, 1, 2)], k_blocks=[(0, 0, 7)])
    assert np.allclose(gq[0][0, 1, 32:48], g[0][0, 1, 32:48])
    assert np.allclose(gq[1][0, 0, 112:128], g[1][0, 0, 112:128])
    assert np.allclose(gq[2][0, 0, 112:128], g[2][0, 0, 112:128])


def test_full_chain_tiny_workload_invariants():
    from workloads import workload
    from workloads.synth import make_inputs
    w = workload(0)
    x = make_inputs(w, seed=0)
    f = O.prism_forward(*(x[n].numpy() for n in ("q", "k", "v", "a2v")), w.grid, w.zone, list(w.cands),
                        w.top_p, w.k_min, w.k_max)
    assert (f["shape_id"] != 3).all()                       # 4x2x2 never fits a 2x4x8 zone
    nb = f["bvalid"].shape[-1]
    for (b, h, I), s in f["sel"].items():
        assert w.k_min <= s.size <= w.k_max
        assert (np.diff(s) > 0).all()
    assert np.isfinite(f["o"]).all()
    bw = O.prism_backward(f, x["do"].numpy())
    assert np.isfinite(bw["dq"]).all() and nb == 16


def test_vectorised_selection_and_reverse_match_row_forms():
    rng = np.random.default_rng(11)
    nb, d = 40, 16
    qb = rng.standard_normal((1, 2, nb, d)).astype(np.float32)
    kb = rng.standard_normal((1, 2, nb, d)).astype(np.float32)
    bv = rng.integers(0, 3, size=(1, 2, nb)).astype(np.int32) * 8
    s1, n1 = O.select_blocks(qb, kb, bv, 0.7, 0.8, 2, 9)
    s2, n2 = O.select_blocks_all(qb, kb, bv, 0.7, 0.8, 2, 9)
    assert s1.keys() == s2.keys()
    for k in s1:
        assert s1[k].tolist() == s2[k].tolist() and n1[k] == n2[k]
    idx, cnt = O.selection_arrays(s1, 1, 2, nb, 9)
    a, b = O.reverse_index(idx, cnt), O.reverse_index_sorted(idx, cnt)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def test_selected_pair_flops_closed_forms():
    """14 d flops per valid (query, key) token pair: with every live block selected the
    pair count is (valid tokens)^2 per head; a hand case with partial blocks."""
    rng = np.random.default_rng(9)
    B, Hh, nb, d = 1, 2, 9, 32
    bv = rng.integers(0, 5, size=(B, Hh, nb)).astype(np.int32)
    sel = {}
    for h in range(Hh):
        live = np.nonzero(bv[0, h] > 0)[0].astype(np.int32)
        for I in range(nb):
            sel[(0, h, I)] = live if bv[0, h, I] > 0 else np.zeros(0, np.int32)
    want = 14.0 * d * sum(int(bv[0, h].sum()) ** 2 for h in range(Hh))
    assert O.selected_pair_flops(bv, sel, d) == want
    bv2 = np.array([[[3, 0, 5]]], dtype=np.int32)
    sel2 = {(0, 0, 0): np.array([0, 2], np.int32), (0, 0, 1): np.zeros(0, np.int32), (0, 0, 2): np.array([2], np.int32)}
    assert O.selected_pair_flops(bv2, sel2, 8) == 14.0 * 8 * (3 * (3 + 5) + 5 * 5)
