"""Python face of libprism: one function per C-ABI call, same names, taking torch
tensors.  Each wrapper only checks the tensors' dtype/device/contiguity/shape and
passes raw device pointers plus torch's current stream to the library; every step of
the computation runs in the library's HIP kernels."""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (PRISM_BF16, PRISM_F32, PrismGrid, PrismSelectParams, PrismShapeParams, PrismShapes,
                   check, load)

Shape = Tuple[int, int, int]


@dataclass(frozen=True)
class ShapeRule:
    """Constants of the shape rule (documented defaults)."""
    alpha: float = 0.5
    tau_lo: float = 1.0
    tau_hi: float = 2.0
    g_min: float = 1e-3
    eps: float = 1e-12


def make_grid(grid: Sequence[int], zone: Sequence[int]) -> PrismGrid:
    return PrismGrid(*[int(x) for x in grid], *[int(x) for x in zone])


def make_shapes(cands: Sequence[Shape], unit: Optional[int] = None) -> PrismShapes:
    """Candidate table.  vol is the first candidate's volume, or `unit` for a list that
    mixes volumes (each a multiple of the unit)."""
    s = PrismShapes()
    s.n = len(cands)
    s.vol = int(unit) if unit is not None else (int(cands[0][0] * cands[0][1] * cands[0][2]) if cands else 0)
    for i, (bt, bh, bw) in enumerate(cands):
        s.bt[i], s.bh[i], s.bw[i] = int(bt), int(bh), int(bw)
    return s


def make_shape_params(rule: ShapeRule = ShapeRule()) -> PrismShapeParams:
    return PrismShapeParams(rule.alpha, rule.tau_lo, rule.tau_hi, rule.g_min, rule.eps)


def make_select_params(top_p: float, k_min: int, k_max: int) -> PrismSelectParams:
    return PrismSelectParams(float(top_p), int(k_min), int(k_max))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, shape=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _same_dtype(*ts):
    d = ts[0].dtype
    for t in ts[1:]:
        if t.dtype != d:
            raise TypeError("tensors must share one dtype")
    return _dt(ts[0])


# ------------------------------------------------------------------ host-only helpers
def prism_num_zones(grid: PrismGrid) -> int:
    return int(load().prism_num_zones(grid))


def prism_num_blocks(grid: PrismGrid, shapes: PrismShapes) -> int:
    return int(load().prism_num_blocks(grid, shapes))


def prism_select_workspace_size(B: int, Hh: int, nb: int, d: int) -> int:
    return int(load().prism_select_workspace_size(B, Hh, nb, d))


def _dtc(dtype) -> int:
    return PRISM_BF16 if dtype == torch.bfloat16 else PRISM_F32


def prism_fwd_workspace_size(B: int, Hh: int, nb: int, vol: int, d: int, dtype=torch.bfloat16) -> int:
    return int(load().prism_fwd_workspace_size(B, Hh, nb, vol, d, _dtc(dtype)))


def prism_bwd_workspace_size(B: int, Hh: int, nb: int, vol: int, d: int, dtype=torch.bfloat16) -> int:
    return int(load().prism_bwd_workspace_size(B, Hh, nb, vol, d, _dtc(dtype)))


def prism_dense_fwd_workspace_size(B: int, Hh: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    return int(load().prism_dense_fwd_workspace_size(B, Hh, N, d, _dtc(dtype)))


def prism_dense_bwd_workspace_size(B: int, Hh: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    return int(load().prism_dense_bwd_workspace_size(B, Hh, N, d, _dtc(dtype)))


def prism_last_error() -> str:
    return load().prism_last_error().decode(errors="replace")


# ------------------------------------------------------------------ the six calls
def _zone_stats(name: str, v: torch.Tensor, a2v: torch.Tensor, grid: PrismGrid, stats: torch.Tensor,
                stream) -> None:
    B, Hh, N, d = v.shape
    nZ = prism_num_zones(grid)
    dt = _same_dtype(v, a2v)
    check(getattr(load(), name)(_ptr(v, shape=(B, Hh, N, d), name="v"),
                                _ptr(a2v, shape=(B, Hh, N, d), name="a2v"), dt, B, Hh, d, grid,
                                _ptr(stats, torch.float32, (B, Hh, nZ, 8), "stats"), _stream(stream)), name)


def prism_zone_stats(v: torch.Tensor, a2v: torch.Tensor, grid: PrismGrid, stats: torch.Tensor,
                     stream=None) -> None:
    _zone_stats("prism_zone_stats", v, a2v, grid, stats, stream)


def prism_zone_stats_global(v: torch.Tensor, a2v: torch.Tensor, grid: PrismGrid, stats: torch.Tensor,
                            stream=None) -> None:
    _zone_stats("prism_zone_stats_global", v, a2v, grid, stats, stream)


def prism_a2v_attn_norm(q: torch.Tensor, ka: torch.Tensor, va: torch.Tensor, scale: float, a2v_norm: torch.Tensor,
                        o: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, N, d = q.shape
    Na = ka.shape[2]
    dt = _same_dtype(q, ka, va)
    check(load().prism_a2v_attn_norm(_ptr(q, shape=(B, Hh, N, d), name="q"), _ptr(ka, shape=(B, Hh, Na, d), name="ka"),
                                     _ptr(va, shape=(B, Hh, Na, d), name="va"), dt, B, Hh, N, Na, d, float(scale),
                                     None if o is None else _ptr(o, q.dtype, (B, Hh, N, d), "o"),
                                     _ptr(a2v_norm, torch.float32, (B, Hh, N), "a2v_norm"), _stream(stream)),
          "prism_a2v_attn_norm")


def prism_zone_stats_from_norm(v: torch.Tensor, a2v_norm: torch.Tensor, grid: PrismGrid, stats: torch.Tensor,
                               global_variance: bool = False, stream=None) -> None:
    B, Hh, N, d = v.shape
    nZ = prism_num_zones(grid)
    check(load().prism_zone_stats_from_norm(_ptr(v, shape=(B, Hh, N, d), name="v"),
                                            _ptr(a2v_norm, torch.float32, (B, Hh, N), "a2v_norm"), _dt(v), B, Hh,
                                            d, grid, int(bool(global_variance)),
                                            _ptr(stats, torch.float32, (B, Hh, nZ, 8), "stats"), _stream(stream)),
          "prism_zone_stats_from_norm")


STATS_GLOBAL_VARIANCE, STATS_FROM_NORM = 1, 2


def prism_zone_stats_ex(v: torch.Tensor, aux: torch.Tensor, grid: PrismGrid, stats: torch.Tensor, flags: int = 0,
                        vact: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, N, d = v.shape
    nZ = prism_num_zones(grid)
    if flags & STATS_FROM_NORM:
        a = _ptr(aux, torch.float32, (B, Hh, N), "a2v_norm")
    else:
        _same_dtype(v, aux)
        a = _ptr(aux, shape=(B, Hh, N, d), name="a2v")
    check(load().prism_zone_stats_ex(_ptr(v, shape=(B, Hh, N, d), name="v"), a, _dt(v), B, Hh, d, grid, int(flags),
                                     _ptr(stats, torch.float32, (B, Hh, nZ, 8), "stats"),
                                     _ptr(vact, torch.float32, (B, Hh, nZ), "vact"), _stream(stream)),
          "prism_zone_stats_ex")


def prism_assign_shapes_multi(stats: torch.Tensor, vact: torch.Tensor, grid: PrismGrid, shapes: PrismShapes,
                              params: PrismShapeParams, tau_128: float, tau_256: float, shape_id: torch.Tensor,
                              margin: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, nZ, _ = stats.shape
    check(load().prism_assign_shapes_multi(_ptr(stats, torch.float32, name="stats"),
                                           _ptr(vact, torch.float32, (B, Hh, nZ), "vact"), B, Hh, grid, shapes, params,
                                           float(tau_128), float(tau_256),
                                           _ptr(shape_id, torch.int32, (B, Hh, nZ), "shape_id"),
                                           _ptr(margin, torch.float32, (B, Hh, nZ), "margin"), _stream(stream)),
          "prism_assign_shapes_multi")


def prism_block_heads(unit_valid: torch.Tensor, shape_id: torch.Tensor, grid: PrismGrid, shapes: PrismShapes,
                      block_valid: torch.Tensor, stream=None) -> None:
    B, Hh, nb = unit_valid.shape
    check(load().prism_block_heads(_ptr(unit_valid, torch.int32, name="unit_valid"),
                                   _ptr(shape_id, torch.int32, name="shape_id"), B, Hh, grid, shapes,
                                   _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), _stream(stream)),
          "prism_block_heads")


def prism_assign_shapes(stats: torch.Tensor, grid: PrismGrid, shapes: PrismShapes, params: PrismShapeParams,
                        shape_id: torch.Tensor, margin: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, nZ, _ = stats.shape
    check(load().prism_assign_shapes(_ptr(stats, torch.float32, name="stats"), B, Hh, grid, shapes, params,
                                     _ptr(shape_id, torch.int32, (B, Hh, nZ), "shape_id"),
                                     _ptr(margin, torch.float32, (B, Hh, nZ), "margin"), _stream(stream)),
          "prism_assign_shapes")


def prism_permute(x: torch.Tensor, y: torch.Tensor, grid: PrismGrid, shapes: PrismShapes,
                  shape_id: torch.Tensor, inverse: bool = False, block_valid: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    B, Hh = x.shape[:2]
    d = x.shape[-1]
    dt = _same_dtype(x, y)
    nb = prism_num_blocks(grid, shapes)
    npad, n = nb * shapes.vol, grid.T * grid.H * grid.W
    src_rows, dst_rows = (npad, n) if inverse else (n, npad)
    check(load().prism_permute(_ptr(x, shape=(B, Hh, src_rows, d), name="x"),
                               _ptr(y, shape=(B, Hh, dst_rows, d), name="y"), dt, B, Hh, d, grid, shapes,
                               _ptr(shape_id, torch.int32, (B, Hh, prism_num_zones(grid)), "shape_id"),
                               int(bool(inverse)),
                               _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), _stream(stream)),
          "prism_permute")


def prism_permute_pool(x: torch.Tensor, y: torch.Tensor, grid: PrismGrid, shapes: PrismShapes,
                       shape_id: torch.Tensor, pooled: torch.Tensor, block_valid: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """Forward permutation that also writes each block's mean valid row (float32 [B, Hh, nb, d])."""
    B, Hh, n, d = x.shape
    dt = _same_dtype(x, y)
    nb = prism_num_blocks(grid, shapes)
    check(load().prism_permute_pool(_ptr(x, shape=(B, Hh, grid.T * grid.H * grid.W, d), name="x"),
                                    _ptr(y, shape=(B, Hh, nb * shapes.vol, d), name="y"), dt, B, Hh, d, grid, shapes,
                                    _ptr(shape_id, torch.int32, (B, Hh, prism_num_zones(grid)), "shape_id"),
                                    _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"),
                                    _ptr(pooled, torch.float32, (B, Hh, nb, d), "pooled"), _stream(stream)),
          "prism_permute_pool")


def prism_select_pooled_workspace_size(B: int, Hh: int, nb: int) -> int:
    return int(load().prism_select_pooled_workspace_size(B, Hh, nb))


def prism_select_blocks_pooled(qbar: torch.Tensor, kbar: torch.Tensor, block_valid: torch.Tensor, scale: float,
                               params: PrismSelectParams, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                               rev_ptr: torch.Tensor, rev_idx: torch.Tensor, workspace: torch.Tensor,
                               sel_margin: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, nb, d = qbar.shape
    km = params.k_max
    check(load().prism_select_blocks_pooled(
        _ptr(qbar, torch.float32, name="qbar"), _ptr(kbar, torch.float32, qbar.shape, "kbar"),
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), B, Hh, nb, d, float(scale), params,
        _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"), _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"),
        _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"), _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"),
        _ptr(sel_margin, torch.float32, (B, Hh, nb), "sel_margin"), _ptr(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "prism_select_blocks_pooled")


def prism_select_blocks(qp: torch.Tensor, kp: torch.Tensor, block_valid: torch.Tensor, vol: int, scale: float,
                        params: PrismSelectParams, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                        rev_ptr: torch.Tensor, rev_idx: torch.Tensor, workspace: torch.Tensor,
                        sel_margin: Optional[torch.Tensor] = None, stream=None) -> None:
    B, Hh, npad, d = qp.shape
    nb = npad // vol
    dt = _same_dtype(qp, kp)
    km = params.k_max
    check(load().prism_select_blocks(
        _ptr(qp, name="qp"), _ptr(kp, shape=qp.shape, name="kp"), dt,
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), B, Hh, nb, vol, d, float(scale), params,
        _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"), _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"),
        _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"), _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"),
        _ptr(sel_margin, torch.float32, (B, Hh, nb), "sel_margin"), _ptr(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "prism_select_blocks")


def prism_tiles_workspace_size(B: int, Hh: int, nb: int, vol: int) -> int:
    return int(load().prism_tiles_workspace_size(B, Hh, nb, vol))


def prism_blocks_to_tiles(block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx, vol: int, tile_valid, tile_idx, tile_cnt,
                          tile_rev_ptr, tile_rev_idx, workspace, stream=None) -> None:
    B, Hh, nb = block_valid.shape
    km = sel_idx.shape[-1]
    g = vol // 64
    nt, kt = nb * g, km * g
    check(load().prism_blocks_to_tiles(
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"),
        _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"), _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"),
        _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"), B, Hh, nb, vol, km,
        _ptr(tile_valid, torch.int32, (B, Hh, nt), "tile_valid"), _ptr(tile_idx, torch.int32, (B, Hh, nt, kt), "tile_idx"),
        _ptr(tile_cnt, torch.int32, (B, Hh, nt), "tile_cnt"), _ptr(tile_rev_ptr, torch.int32, (B, Hh, nt + 1), "tile_rev_ptr"),
        _ptr(tile_rev_idx, torch.int32, (B, Hh, nt * kt), "tile_rev_idx"), _ptr(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "prism_blocks_to_tiles")


def prism_tiles_mixed_workspace_size(B: int, Hh: int, nb: int) -> int:
    return int(load().prism_tiles_mixed_workspace_size(B, Hh, nb))


def prism_blocks_to_tiles_mixed(block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx, max_units: int, tile_idx, tile_cnt,
                                tile_rev_ptr, tile_rev_idx, workspace, stream=None) -> None:
    B, Hh, nb = block_valid.shape
    km = sel_idx.shape[-1]
    kt = km * max_units
    check(load().prism_blocks_to_tiles_mixed(
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"),
        _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"), _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"),
        _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"), B, Hh, nb, km, int(max_units),
        _ptr(tile_idx, torch.int32, (B, Hh, nb, kt), "tile_idx"), _ptr(tile_cnt, torch.int32, (B, Hh, nb), "tile_cnt"),
        _ptr(tile_rev_ptr, torch.int32, (B, Hh, nb + 1), "tile_rev_ptr"),
        _ptr(tile_rev_idx, torch.int32, (B, Hh, nb * kt), "tile_rev_idx"), _ptr(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "prism_blocks_to_tiles_mixed")


def prism_sparse_attn_fwd(qp, kp, vp, block_valid, sel_idx, sel_cnt, vol: int, scale: float, op, lse,
                          workspace=None, stream=None) -> None:
    B, Hh, npad, d = qp.shape
    nb = npad // vol
    km = sel_idx.shape[-1]
    dt = _same_dtype(qp, kp, vp, op)
    if workspace is None:
        need = prism_fwd_workspace_size(B, Hh, nb, vol, d, qp.dtype)
        workspace = torch.empty(need, dtype=torch.uint8, device=qp.device) if need else None
    check(load().prism_sparse_attn_fwd(
        _ptr(qp, name="qp"), _ptr(kp, shape=qp.shape, name="kp"), _ptr(vp, shape=qp.shape, name="vp"), dt,
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"),
        _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"), _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"),
        km, B, Hh, nb, vol, d, float(scale), _ptr(op, shape=qp.shape, name="op"),
        _ptr(lse, torch.float32, (B, Hh, npad), "lse"), _ptr(workspace, torch.uint8, name="workspace"),
        0 if workspace is None else workspace.numel(), _stream(stream)), "prism_sparse_attn_fwd")


def prism_sparse_attn_bwd(qp, kp, vp, op, dop, lse, block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx, vol: int,
                          scale: float, dqp, dkp, dvp, workspace, marks=None, stream=None) -> None:
    B, Hh, npad, d = qp.shape
    nb = npad // vol
    km = sel_idx.shape[-1]
    dt = _same_dtype(qp, kp, vp, op, dop, dqp, dkp, dvp)
    keep = _event_array(marks)
    mk = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    check(load().prism_sparse_attn_bwd(
        _ptr(qp, name="qp"), _ptr(kp, shape=qp.shape, name="kp"), _ptr(vp, shape=qp.shape, name="vp"),
        _ptr(op, shape=qp.shape, name="op"), _ptr(dop, shape=qp.shape, name="dop"),
        _ptr(lse, torch.float32, (B, Hh, npad), "lse"), dt, _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"),
        _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"), _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"), km,
        _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"), _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"),
        B, Hh, nb, vol, d, float(scale), _ptr(dqp, shape=qp.shape, name="dqp"), _ptr(dkp, shape=qp.shape, name="dkp"),
        _ptr(dvp, shape=qp.shape, name="dvp"), _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(),
        mk, _stream(stream)), "prism_sparse_attn_bwd")


def prism_sparse_attn_bwd_noalloc(qp, kp, vp, op, dop, lse, block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx,
                                  vol: int, scale: float, dqp, dkp, dvp, marks=None, stream=None) -> None:
    """prism_sparse_attn_bwd without a workspace argument: the library's static scratch."""
    B, Hh, npad, d = qp.shape
    nb = npad // vol
    km = sel_idx.shape[-1]
    dt = _same_dtype(qp, kp, vp, op, dop, dqp, dkp, dvp)
    keep = _event_array(marks)
    mk = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    check(load().prism_sparse_attn_bwd_noalloc(
        _ptr(qp, name="qp"), _ptr(kp, shape=qp.shape, name="kp"), _ptr(vp, shape=qp.shape, name="vp"),
        _ptr(op, shape=qp.shape, name="op"), _ptr(dop, shape=qp.shape, name="dop"),
        _ptr(lse, torch.float32, (B, Hh, npad), "lse"), dt, _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"),
        _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"), _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"), km,
        _ptr(rev_ptr, torch.int32, (B, Hh, nb + 1), "rev_ptr"), _ptr(rev_idx, torch.int32, (B, Hh, nb * km), "rev_idx"),
        B, Hh, nb, vol, d, float(scale), _ptr(dqp, shape=qp.shape, name="dqp"), _ptr(dkp, shape=qp.shape, name="dkp"),
        _ptr(dvp, shape=qp.shape, name="dvp"), mk, _stream(stream)), "prism_sparse_attn_bwd_noalloc")


def prism_dense_attn_fwd(q, k, v, scale: float, o, lse, workspace=None, stream=None) -> None:
    B, Hh, N, d = q.shape
    dt = _same_dtype(q, k, v, o)
    check(load().prism_dense_attn_fwd(_ptr(q, name="q"), _ptr(k, shape=q.shape, name="k"),
                                      _ptr(v, shape=q.shape, name="v"), dt, B, Hh, N, d, float(scale),
                                      _ptr(o, shape=q.shape, name="o"), _ptr(lse, torch.float32, (B, Hh, N), "lse"),
                                      _ptr(workspace, torch.uint8, name="workspace"),
                                      0 if workspace is None else workspace.numel(), _stream(stream)),
          "prism_dense_attn_fwd")


def prism_dense_attn_bwd(q, k, v, o, do, lse, scale: float, dq, dk, dv, workspace, marks=None, stream=None) -> None:
    B, Hh, N, d = q.shape
    dt = _same_dtype(q, k, v, o, do, dq, dk, dv)
    keep = _event_array(marks)
    mk = None if keep is None else ctypes.cast(keep, ctypes.c_void_p)
    check(load().prism_dense_attn_bwd(
        _ptr(q, name="q"), _ptr(k, shape=q.shape, name="k"), _ptr(v, shape=q.shape, name="v"),
        _ptr(o, shape=q.shape, name="o"), _ptr(do, shape=q.shape, name="do"),
        _ptr(lse, torch.float32, (B, Hh, N), "lse"), dt, B, Hh, N, d, float(scale),
        _ptr(dq, shape=q.shape, name="dq"), _ptr(dk, shape=q.shape, name="dk"), _ptr(dv, shape=q.shape, name="dv"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), mk, _stream(stream)),
        "prism_dense_attn_bwd")


def _event_array(marks):
    """C array of 4 hipEvent_t handles for the optional `marks` argument.  `marks` holds
    torch.cuda.Event objects (already recorded once, so that their handles exist) or raw
    integer handles."""
    if marks is None:
        return None
    if len(marks) != 4:
        raise ValueError("marks needs 4 events")
    hs = [m.cuda_event if isinstance(m, torch.cuda.Event) else int(m) for m in marks]
    if any(h == 0 for h in hs):
        raise ValueError("record each event once before passing it as a mark")
    return (ctypes.c_void_p * 4)(*hs)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# ------------------------------------------------------------------ measurement kernels
def prism_bench_mfma_peak(workgroups: int, iters: int, clocks: torch.Tensor, sink: torch.Tensor,
                          stream=None) -> None:
    """clocks int64 [workgroups, 2] (shader cycles, 100 MHz ticks), sink float32 [workgroups]."""
    check(load().prism_bench_mfma_peak(int(workgroups), int(iters),
                                       _ptr(clocks, torch.int64, (workgroups, 2), "clocks"),
                                       _ptr(sink, torch.float32, (workgroups,), "sink"), _stream(stream)),
          "prism_bench_mfma_peak")


PRISM_BENCH_STREAM_SINK = 8192


def prism_bench_stream_read(a: torch.Tensor, b: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Reads every byte of a and of b (same size, a multiple of 16 bytes); sink int32
    [PRISM_BENCH_STREAM_SINK] receives per-wavefront checksums."""
    nbytes = a.numel() * a.element_size()
    if b.numel() * b.element_size() != nbytes:
        raise ValueError("a and b must hold the same number of bytes")
    check(load().prism_bench_stream_read(_ptr(a, name="a"), _ptr(b, name="b"), nbytes,
                                         _ptr(sink, torch.int32, (PRISM_BENCH_STREAM_SINK,), "sink"),
                                         _stream(stream)), "prism_bench_stream_read")


def prism_bench_tile_gather(qp, kp, vp, block_valid, sel_idx, sel_cnt, vol: int, op, workspace, stream=None) -> None:
    B, Hh, npad, d = qp.shape
    nb = npad // vol
    km = sel_idx.shape[-1]
    dt = _same_dtype(qp, kp, vp, op)
    check(load().prism_bench_tile_gather(
        _ptr(qp, name="qp"), _ptr(kp, shape=qp.shape, name="kp"), _ptr(vp, shape=qp.shape, name="vp"), dt,
        _ptr(block_valid, torch.int32, (B, Hh, nb), "block_valid"), _ptr(sel_idx, torch.int32, (B, Hh, nb, km), "sel_idx"),
        _ptr(sel_cnt, torch.int32, (B, Hh, nb), "sel_cnt"), km, B, Hh, nb, vol, d, _ptr(op, shape=qp.shape, name="op"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(stream)), "prism_bench_tile_gather")
