"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function the header declares, and rejects invalid arguments before launching anything."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from oracle import prism_oracle as O
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")


@pytest.fixture(scope="module")
def lib():
    from content_adaptive_block_zone_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from content_adaptive_block_zone_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    from content_adaptive_block_zone_amd import _lib
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.PROTOTYPES, f"binding lacks {n}"
    assert set(_lib.PROTOTYPES) == set(names)


def test_struct_sizes_match_the_header():
    """The ctypes mirrors of the header's structs have the header's array sizes."""
    from content_adaptive_block_zone_amd import _lib
    m = re.search(r"#define\s+PRISM_MAX_SHAPES\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == _lib.MAX_SHAPES
    assert ctypes.sizeof(_lib.PrismShapes) == 4 * (2 + 3 * _lib.MAX_SHAPES)


def test_zone_and_block_counts_match_the_oracle(lib):
    from content_adaptive_block_zone_amd import api
    for w in WORKLOADS:
        g = api.make_grid(w.grid, w.zone)
        s = api.make_shapes(list(w.cands))
        nz = O.num_zones(w.grid, w.zone)
        assert api.prism_num_zones(g) == nz
        assert api.prism_num_blocks(g, s) == nz * (w.zone[0] * w.zone[1] * w.zone[2]) // w.vol


def test_host_helpers_reject_bad_geometry(lib):
    from content_adaptive_block_zone_amd import api
    assert api.prism_num_zones(api.make_grid((0, 8, 8), (2, 4, 8))) == -1
    assert api.prism_num_zones(api.make_grid((4, 8, 8), (64, 64, 64))) == -1        # zone too large
    mixed = api.make_shapes([(1, 4, 4), (2, 2, 2)])                                 # unequal volumes
    assert api.prism_num_blocks(api.make_grid((4, 8, 8), (2, 4, 8)), mixed) == -1
    nofit = api.make_shapes([(4, 2, 2)])                                            # never fits 2x4x8
    assert api.prism_num_blocks(api.make_grid((4, 8, 8), (2, 4, 8)), nofit) == -1
    assert api.prism_select_workspace_size(0, 1, 1, 64) == 0
    import torch
    assert api.prism_fwd_workspace_size(1, 2, 16, 16, 64, torch.float32) == 0
    assert api.prism_bwd_workspace_size(1, 4, 5760, 64, 128, torch.bfloat16) >= 4 * 5760 * 64 * 4


def test_attention_workspace_holds_the_schedules(lib):
    """The matrix-core path (bf16, 64-row blocks, d = 128) keeps in the workspace its
    workgroup schedules (one int32 per (head, block), sparse mode only) and, for the
    forward, the fp16 copy of V (2 bytes per element) with two per-head words (max |V|
    bits, inverse scale); the backward holds D (one float per row) and two schedules.
    Every part is rounded up to 256 bytes.  Other paths need no workspace for the forward
    and D alone for the backward."""
    import torch
    from content_adaptive_block_zone_amd import api
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hh, nb in ((1, 4, 5760), (2, 3, 77)):
        sched = a256(B * Hh * nb * 4)
        v16 = 2 * a256(B * Hh * 4) + a256(B * Hh * nb * 64 * 128 * 2)
        assert api.prism_fwd_workspace_size(B, Hh, nb, 64, 128, torch.bfloat16) == sched + v16
        assert api.prism_bwd_workspace_size(B, Hh, nb, 64, 128, torch.bfloat16) == a256(B * Hh * nb * 64 * 4) + 2 * sched
        assert api.prism_fwd_workspace_size(B, Hh, nb, 64, 64, torch.bfloat16) == 0           # generic path
        assert api.prism_fwd_workspace_size(B, Hh, nb, 16, 128, torch.bfloat16) == 0
        assert api.prism_bwd_workspace_size(B, Hh, nb, 64, 128, torch.float32) == a256(B * Hh * nb * 64 * 4)
    # dense: no schedule, the fp16 copy of V only
    assert api.prism_dense_fwd_workspace_size(1, 4, 1000, 128, torch.bfloat16) == 2 * 256 + a256(4 * 1000 * 128 * 2)


def test_select_workspace_is_linear_in_nb(lib):
    """Selection scores one chunk of query blocks at a time: as many per head as keep
    the chunk's scores ([B*Hh][CH][nb] float32) within 256 MB, in multiples of 64, never
    fewer than 512 (or nb).  With that chunk's selection bits (a row of words32(nb) words
    per query block), plus reverse counts and cursors (one int each per key block), the
    workspace grows linearly with nb, never as nb^2."""
    from content_adaptive_block_zone_amd import api
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    w32 = lambda x: (x + 31) // 32  # noqa: E731
    for BH, nb in ((4, 5760), (4, 15360), (2, 300), (4, 32768)):
        ch = min(nb, max(512, (256 << 20) // (BH * nb * 4) // 64 * 64))
        want = a256(BH * ch * nb * 4) + a256(BH * ch * w32(nb) * 4) + 2 * a256(BH * nb * 4)
        assert api.prism_select_pooled_workspace_size(1, BH, nb) == want
        assert api.prism_select_workspace_size(1, BH, nb, 128) == want + 2 * a256(BH * nb * 128 * 4)
    assert api.prism_select_pooled_workspace_size(1, 4, 32768) <= 2.01 * api.prism_select_pooled_workspace_size(1, 4, 16384)
    assert api.prism_select_pooled_workspace_size(1, 4, 15360) < (280 << 20)   # the scores: 256 MB at most


def _status(fn, *args):
    return fn(*args)


def test_calls_validate_before_launch(lib):
    """Every call with one bad argument returns its error code and a message; the fake
    pointers below are never dereferenced because validation fails first."""
    from content_adaptive_block_zone_amd import _lib, api
    P = ctypes.c_void_p(64)
    g = api.make_grid((4, 8, 8), (2, 4, 8))
    s = api.make_shapes([(1, 4, 4), (2, 2, 4), (2, 4, 2), (4, 2, 2)])
    sp = api.make_shape_params()
    sel = api.make_select_params(0.9, 2, 8)
    F32, BF16 = _lib.PRISM_F32, _lib.PRISM_BF16
    E = _lib

    cases = [
        ("prism_zone_stats", (None, P, F32, 1, 2, 64, g, P, None), E.PRISM_ERR_ARG),
        ("prism_zone_stats", (P, P, 7, 1, 2, 64, g, P, None), E.PRISM_ERR_DTYPE),
        ("prism_zone_stats", (P, P, F32, 1, 2, 48, g, P, None), E.PRISM_ERR_DTYPE),
        ("prism_zone_stats", (P, P, F32, 0, 2, 64, g, P, None), E.PRISM_ERR_ARG),
        ("prism_zone_stats", (P, P, F32, 1, 2, 64, api.make_grid((4, 8, 8), (64, 64, 2)), P, None),
         E.PRISM_ERR_SHAPE),
        ("prism_assign_shapes", (P, 1, 2, g, api.make_shapes([(1, 4, 4), (1, 2, 2)]), sp, P, None, None),
         E.PRISM_ERR_SHAPE),
        ("prism_assign_shapes", (P, 1, 2, g, s, api.make_shape_params(api.ShapeRule(tau_lo=2.0, tau_hi=1.0)),
                                 P, None, None), E.PRISM_ERR_ARG),
        ("prism_assign_shapes", (P, 1, 2, g, s, api.make_shape_params(api.ShapeRule(g_min=0.0)), P, None, None),
         E.PRISM_ERR_ARG),
        ("prism_permute", (P, P, F32, 1, 2, 64, g, s, P, 2, None, None), E.PRISM_ERR_ARG),
        ("prism_permute", (P, P, BF16, 1, 2, 4, g, s, P, 0, None, None), E.PRISM_ERR_DTYPE),
        ("prism_permute", (P, P, F32, 1, 2, 64, g, s, P, 0, None, None), E.PRISM_ERR_ARG),   # x aliases y
        ("prism_select_blocks", (P, P, F32, P, 1, 2, 16, 16, 64, 0.125, api.make_select_params(0.0, 2, 8),
                                 P, P, P, P, None, P, 1 << 30, None), E.PRISM_ERR_ARG),
        ("prism_select_blocks", (P, P, F32, P, 1, 2, 16, 16, 64, 0.125, api.make_select_params(0.9, 5, 4),
                                 P, P, P, P, None, P, 1 << 30, None), E.PRISM_ERR_ARG),
        ("prism_select_blocks", (P, P, F32, P, 1, 2, 16, 16, 64, 0.125, sel, P, P, P, P, None, P, 16, None),
         E.PRISM_ERR_ARG),                                                             # workspace too small
        ("prism_select_blocks", (P, P, F32, P, 1, 2, 40000, 16, 64, 0.125, sel, P, P, P, P, None, P, 1 << 44,
                                 None), E.PRISM_ERR_SHAPE),
        ("prism_select_blocks", (P, P, F32, P, 1, 2, 32769, 16, 64, 0.125, sel, P, P, P, P, None, P, 1 << 44,
                                 None), E.PRISM_ERR_SHAPE),                            # one past the limit
        ("prism_sparse_attn_fwd", (P, P, P, F32, P, P, P, 8, 1, 2, 16, 16, 96, 0.125, P, P, None, 0, None),
         E.PRISM_ERR_DTYPE),
        ("prism_sparse_attn_fwd", (P, P, P, F32, P, P, P, 8, 1, 2, 16, 128, 64, 0.125, P, P, None, 0, None),
         E.PRISM_ERR_SHAPE),
        ("prism_sparse_attn_fwd", (P, P, P, F32, P, P, P, 0, 1, 2, 16, 16, 64, 0.125, P, P, None, 0, None),
         E.PRISM_ERR_ARG),
        ("prism_sparse_attn_fwd", (P, P, P, BF16, P, P, P, 8, 1, 2, 16, 64, 128, 0.125, P, P, None, 0, None),
         E.PRISM_ERR_ARG),                                                             # schedule and the fp16 copy of V need a workspace
        ("prism_sparse_attn_fwd", (P, P, P, BF16, P, P, P, 8, 1, 2, 16, 64, 128, 0.125, P, P, P, 127, None),
         E.PRISM_ERR_ARG),                                                             # workspace too small
        ("prism_sparse_attn_bwd", (P, P, P, P, P, P, BF16, P, P, P, 8, P, P, 1, 2, 16, 64, 128, 0.125, P, P, P,
                                   P, 2 * 16 * 64 * 4, None, None), E.PRISM_ERR_ARG),  # D only, no room for schedules
        ("prism_sparse_attn_bwd", (P, P, P, P, P, P, F32, P, P, P, 8, P, P, 1, 2, 16, 16, 64, 0.125, P, P, P,
                                   P, 8, None, None), E.PRISM_ERR_ARG),
        ("prism_dense_attn_fwd", (P, P, P, F32, 1, 2, 0, 64, 0.125, P, P, None, 0, None), E.PRISM_ERR_ARG),
        ("prism_a2v_attn_norm", (P, P, P, F32, 1, 2, 64, 32, 128, 0.1, None, P, None), E.PRISM_ERR_DTYPE),
        ("prism_a2v_attn_norm", (P, P, P, BF16, 1, 2, 64, 0, 128, 0.1, None, P, None), E.PRISM_ERR_ARG),
        ("prism_a2v_attn_norm", (P, P, None, BF16, 1, 2, 64, 32, 128, 0.1, None, P, None), E.PRISM_ERR_ARG),
        ("prism_zone_stats_from_norm", (P, None, BF16, 1, 2, 128, g, 0, P, None), E.PRISM_ERR_ARG),
        ("prism_zone_stats_from_norm", (P, P, BF16, 1, 2, 48, g, 0, P, None), E.PRISM_ERR_DTYPE),
        ("prism_zone_stats_global", (P, P, F32, 0, 2, 64, g, P, None), E.PRISM_ERR_ARG),
        ("prism_blocks_to_tiles", (P, P, P, P, P, 1, 2, 16, 96, 4, P, P, P, P, P, P, 1 << 20, None),
         E.PRISM_ERR_SHAPE),                                                           # vol not a multiple of 64
        ("prism_blocks_to_tiles", (P, P, P, P, P, 1, 2, 16, 128, 4, P, P, P, P, P, P, 4, None),
         E.PRISM_ERR_ARG),                                                             # workspace too small
        ("prism_blocks_to_tiles", (P, None, P, P, P, 1, 2, 16, 128, 4, P, P, P, P, P, P, 1 << 20, None),
         E.PRISM_ERR_ARG),
        ("prism_dense_attn_bwd", (P, P, P, P, P, P, F32, 1, 2, 256, 64, float("nan"), P, P, P, P, 1 << 30,
                                  None, None), E.PRISM_ERR_ARG),
        ("prism_sparse_attn_bwd_noalloc", (P, P, P, P, P, P, BF16, P, P, P, 8, P, P, 1, 1, (1 << 17) + 1, 64, 128,
                                           0.1, P, P, P, None, None), E.PRISM_ERR_SHAPE),   # past the static scratch
        ("prism_sparse_attn_bwd_noalloc", (P, P, P, P, P, None, BF16, P, P, P, 8, P, P, 1, 1, 16, 64, 128,
                                           0.1, P, P, P, None, None), E.PRISM_ERR_ARG),
        ("prism_permute_pool", (P, P, F32, 1, 2, 64, g, s, P, None, None, None), E.PRISM_ERR_ARG),   # no pooled
        ("prism_permute_pool", (P, P, BF16, 1, 2, 24, g, s, P, None, P, None), E.PRISM_ERR_DTYPE),  # 48-byte rows
        ("prism_permute_pool", (P, P, F32, 1, 2, 64, g, s, P, None, P, None), E.PRISM_ERR_ARG),     # x aliases y
        ("prism_permute_pool", (P, ctypes.c_void_p(128), F32, 1, 2, 64, g,
                                api.make_shapes([(1, 4, 4), (2, 4, 4)], unit=16), P, None, P, None),
         E.PRISM_ERR_SHAPE),                                                           # mixed volumes
        ("prism_select_blocks_pooled", (P, P, P, 1, 2, 16, 64, 0.125, api.make_select_params(1.5, 2, 8), P, P, P,
                                        P, None, P, 1 << 30, None), E.PRISM_ERR_ARG),
        ("prism_select_blocks_pooled", (P, P, P, 1, 2, 16, 60, 0.125, sel, P, P, P, P, None, P, 1 << 30, None),
         E.PRISM_ERR_DTYPE),                                                           # d not a multiple of 16
        ("prism_select_blocks_pooled", (P, P, P, 1, 2, 16, 64, 0.125, sel, P, P, P, P, None, P, 8, None),
         E.PRISM_ERR_ARG),                                                             # workspace too small
        ("prism_select_blocks_pooled", (P, P, P, 1, 2, 32769, 64, 0.125, sel, P, P, P, P, None, P, 1 << 44, None),
         E.PRISM_ERR_SHAPE),
        # B*Hh heads x zones (or blocks) per head past 2^31 - 1: the 32-bit launch grids would wrap
        ("prism_zone_stats", (P, P, F32, 1 << 16, 1 << 14, 64, g, P, None), E.PRISM_ERR_SHAPE),
        ("prism_assign_shapes", (P, 1 << 16, 1 << 14, g, s, sp, P, None, None), E.PRISM_ERR_SHAPE),
        ("prism_permute", (P, ctypes.c_void_p(128), F32, 1 << 16, 1 << 12, 64, g, s, P, 0, None, None),
         E.PRISM_ERR_SHAPE),
        ("prism_select_blocks_pooled", (P, P, P, 1 << 16, 1 << 8, 1 << 8, 64, 0.125, sel, P, P, P, P, None, P,
                                        1 << 62, None), E.PRISM_ERR_SHAPE),
        ("prism_bench_stream_read", (P, None, 1 << 20, P, None), E.PRISM_ERR_ARG),
        ("prism_bench_stream_read", (P, P, 1000, P, None), E.PRISM_ERR_ARG),            # not a multiple of 16
        ("prism_bench_stream_read", (P, P, 0, P, None), E.PRISM_ERR_ARG),
    ]
    for name, args, want in cases:
        st = getattr(lib, name)(*args)
        assert st == want, (name, args, st, lib.prism_last_error())
        assert lib.prism_last_error().decode(), name


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from content_adaptive_block_zone_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_layer_rejects_invalid_shape_ids(lib):
    """Given shapes (the random / fixed ablations) are checked on the host: an id outside
    the candidate list, or a candidate that does not tile the zone, raises before any
    launch (the shape check runs before the layer touches the GPU)."""
    import torch
    from content_adaptive_block_zone_amd.pipeline import PrismLayer
    L = PrismLayer(1, 2, 64, (4, 8, 8), (2, 4, 8), [(1, 4, 4), (2, 2, 4), (2, 4, 2), (4, 2, 2)], 0.9, 2, 8,
                   dtype=torch.float32, device="cpu")
    ok = torch.zeros(1, 2, L.nZ, dtype=torch.int32)
    L.check_shape_ids(ok)
    with pytest.raises(ValueError, match="lie in"):
        L.check_shape_ids(ok + 4)
    with pytest.raises(ValueError, match="do not tile"):
        L.check_shape_ids(ok + 3)                  # 4x2x2 has b_T = 4 > zone extent 2
    with pytest.raises(ValueError, match="expected"):
        L.check_shape_ids(torch.zeros(1, 1, L.nZ, dtype=torch.int32))
