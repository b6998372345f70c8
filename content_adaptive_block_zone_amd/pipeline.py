"""One Prism attention layer as a sequence of C-ABI calls.

PrismLayer owns the device buffers (allocated once with torch) and calls the library in
the method's order (Figure 2 caption): zone statistics -> shape assignment -> permute
Q, K, V -> pooling + hybrid selection (+ reverse index) -> block-sparse attention ->
inverse permute of O; the backward permutes dO, runs the sparse backward and inverse
permutes dQ, dK, dV.  Everything is enqueued on torch's current stream."""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from . import api
from .api import ShapeRule

Shape = Tuple[int, int, int]


def random_shape_ids(B: int, Hh: int, grid: Sequence[int], zone: Sequence[int], cands: Sequence[Shape],
                     seed: int) -> torch.Tensor:
    """Seeded uniform draw of a feasible candidate per (batch, head, zone): the random-shape
    ablation of Table 9.  The draw happens here, on the host, and enters the layer as an
    input (PrismLayer.forward(..., shape_id=...)).  int32 [B, Hh, nZ] on the CPU."""
    T, H, W = grid
    zt, zh, zw = zone
    nZ = -(-T // zt) * -(-H // zh) * -(-W // zw)
    ok = [i for i, (bt, bh, bw) in enumerate(cands) if zt % bt == 0 and zh % bh == 0 and zw % bw == 0]
    if not ok:
        raise ValueError("no candidate shape fits the zone")
    g = torch.Generator().manual_seed(int(seed))
    pick = torch.randint(len(ok), (B, Hh, nZ), generator=g)
    return torch.tensor(ok, dtype=torch.int32)[pick]


class PrismLayer:
    """One layer's buffers and call sequence.

    Ablation settings (Table 9 caption): `features` picks the tensor whose directional
    variance guides the shapes ("v" by default, or "q" / "k"); `variance` = "global"
    takes it across all channels jointly instead of per channel.  Fixed shapes are a
    one-candidate set; random shapes come in through forward(shape_id=...).  Top-k only
    and Top-p only (Table 7) are selection parameters (top_p = 1 with k_min = k_max, or
    k_min = 1 with k_max >= the block count).

    mixed = (tau_128, tau_256) takes a candidate list that mixes 64-, 128- and 256-token
    shapes (Tables 9 and 11: C_64, C_128, C_256) and picks each zone's volume by those
    thresholds on its activity (prism_assign_shapes_multi); blocks are then identified by
    their first 64-row unit and the attention runs on 64-row tiles."""

    def __init__(self, B: int, Hh: int, d: int, grid: Sequence[int], zone: Sequence[int],
                 cands: Sequence[Shape], top_p: float, k_min: int, k_max: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", scale: Optional[float] = None,
                 rule: ShapeRule = ShapeRule(), features: str = "v", variance: str = "channel",
                 mixed: Optional[Tuple[float, float]] = None):
        if features not in ("v", "q", "k") or variance not in ("channel", "global"):
            raise ValueError(f"features must be v, q or k and variance channel or global, got {features}, {variance}")
        self.features, self.variance = features, variance
        self.mixed = None if mixed is None else (float(mixed[0]), float(mixed[1]))
        self.B, self.Hh, self.d = B, Hh, d
        self.dtype, self.device = dtype, torch.device(device)
        self.grid = api.make_grid(grid, zone)
        self.shapes = api.make_shapes(cands, unit=64 if mixed is not None else None)
        self.shape_params = api.make_shape_params(rule)
        self.sel_params = api.make_select_params(top_p, k_min, k_max)
        self.scale = api.default_scale(d) if scale is None else float(scale)
        self.vol = self.shapes.vol
        self.N = int(grid[0] * grid[1] * grid[2])
        self.nZ = api.prism_num_zones(self.grid)
        self.nb = api.prism_num_blocks(self.grid, self.shapes)
        if self.nZ < 0 or self.nb < 0:
            raise ValueError(api.prism_last_error())
        self.Npad = self.nb * self.vol
        self.k_max = int(k_max)
        dev, i32, f32 = self.device, torch.int32, torch.float32
        e = lambda *s, dt=dtype: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        B_, H_ = B, Hh
        self.stats = e(B_, H_, self.nZ, 8, dt=f32)
        self.shape_id = e(B_, H_, self.nZ, dt=i32)
        self.shape_margin = e(B_, H_, self.nZ, dt=f32)
        self.bvalid = e(B_, H_, self.nb, dt=i32)
        self.qp, self.kp, self.vp = (e(B_, H_, self.Npad, d) for _ in range(3))
        self.op = e(B_, H_, self.Npad, d)
        self.lse = e(B_, H_, self.Npad, dt=f32)
        self.sel_idx = e(B_, H_, self.nb, self.k_max, dt=i32)
        self.sel_cnt = e(B_, H_, self.nb, dt=i32)
        self.sel_margin = e(B_, H_, self.nb, dt=f32)
        self.rev_ptr = e(B_, H_, self.nb + 1, dt=i32)
        self.rev_idx = e(B_, H_, self.nb * self.k_max, dt=i32)
        # Uniform block volume: pooling is fused into the permutation of Q and K
        # (prism_permute_pool) and the selection starts from the pooled means.  Mixed volumes
        # pool whole blocks that span several units, inside prism_select_blocks.
        self.fused_pool = mixed is None
        if self.fused_pool:
            self.qbar = e(B_, H_, self.nb, d, dt=f32)
            self.kbar = e(B_, H_, self.nb, d, dt=f32)
            self.ws_sel = e(api.prism_select_pooled_workspace_size(B, Hh, self.nb), dt=torch.uint8)
        else:
            self.ws_sel = e(api.prism_select_workspace_size(B, Hh, self.nb, d), dt=torch.uint8)
        self.ws_fwd = e(max(1, api.prism_fwd_workspace_size(B, Hh, self.nb, self.vol, d, dtype)), dt=torch.uint8)
        self.ws_bwd = e(api.prism_bwd_workspace_size(B, Hh, self.nb, self.vol, d, dtype), dt=torch.uint8)
        self.o = e(B_, H_, self.N, d)
        self._grad_bufs = None
        self._ws_sel_slots = None
        # Blocks of more than 64 tokens run the attention on 64-row tiles (vol/64 per block).
        self.g = self.vol // 64 if self.vol > 64 else 1
        if self.mixed is not None:
            # blocks identified by their first 64-row unit; units are the attention tiles
            self.max_units = max(bt * bh * bw for (bt, bh, bw) in cands) // 64
            kt = self.k_max * self.max_units
            self.vact = e(B_, H_, self.nZ, dt=f32)
            self.unit_valid = e(B_, H_, self.nb, dt=i32)
            self.tile_idx = e(B_, H_, self.nb, kt, dt=i32)
            self.tile_cnt = e(B_, H_, self.nb, dt=i32)
            self.tile_rev_ptr = e(B_, H_, self.nb + 1, dt=i32)
            self.tile_rev_idx = e(B_, H_, self.nb * kt, dt=i32)
            self.ws_tiles = e(api.prism_tiles_mixed_workspace_size(B, Hh, self.nb), dt=torch.uint8)
        elif self.vol > 64:
            if self.vol % 64:
                raise ValueError(f"block volume {self.vol} above 64 must be a multiple of 64")
            nt, kt = self.nb * self.g, self.k_max * self.g
            self.tile_valid = e(B_, H_, nt, dt=i32)
            self.tile_idx = e(B_, H_, nt, kt, dt=i32)
            self.tile_cnt = e(B_, H_, nt, dt=i32)
            self.tile_rev_ptr = e(B_, H_, nt + 1, dt=i32)
            self.tile_rev_idx = e(B_, H_, nt * kt, dt=i32)
            self.ws_tiles = e(api.prism_tiles_workspace_size(B, Hh, self.nb, self.vol), dt=torch.uint8)
            self.ws_fwd = e(max(1, api.prism_fwd_workspace_size(B, Hh, nt, 64, d, dtype)), dt=torch.uint8)
            self.ws_bwd = e(api.prism_bwd_workspace_size(B, Hh, nt, 64, d, dtype), dt=torch.uint8)

    def _grads(self):
        if self._grad_bufs is None:
            e = lambda *s: torch.empty(s, dtype=self.dtype, device=self.device)  # noqa: E731
            B, H, P, N, d = self.B, self.Hh, self.Npad, self.N, self.d
            self._grad_bufs = dict(dop=e(B, H, P, d), dqp=e(B, H, P, d), dkp=e(B, H, P, d), dvp=e(B, H, P, d),
                                   dq=e(B, H, N, d), dk=e(B, H, N, d), dv=e(B, H, N, d))
        return self._grad_bufs

    # ---- stages (each is exactly one library call)
    def _stats_flags(self, from_norm: bool) -> int:
        return ((api.STATS_GLOBAL_VARIANCE if self.variance == "global" else 0) |
                (api.STATS_FROM_NORM if from_norm else 0))

    def zone_stats(self, feat, a2v):
        if self.mixed is not None:
            api.prism_zone_stats_ex(feat, a2v, self.grid, self.stats, self._stats_flags(False), self.vact)
            return
        fn = api.prism_zone_stats_global if self.variance == "global" else api.prism_zone_stats
        fn(feat, a2v, self.grid, self.stats)

    def zone_stats_from_norm(self, feat, a2v_norm):
        if self.mixed is not None:
            api.prism_zone_stats_ex(feat, a2v_norm, self.grid, self.stats, self._stats_flags(True), self.vact)
            return
        api.prism_zone_stats_from_norm(feat, a2v_norm, self.grid, self.stats, self.variance == "global")

    def a2v_norm(self, q, ka, va, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Per-token norm of the audio-to-video cross-attention softmax(q ka^T/sqrt(d)) va,
        float32 [B, Hh, N] (the layer's own dense cross-attention kernel)."""
        if out is None:
            out = torch.empty(q.shape[:3], dtype=torch.float32, device=self.device)
        api.prism_a2v_attn_norm(q, ka, va, self.scale, out)
        return out

    def assign_shapes(self):
        if self.mixed is not None:
            api.prism_assign_shapes_multi(self.stats, self.vact, self.grid, self.shapes, self.shape_params,
                                          self.mixed[0], self.mixed[1], self.shape_id, self.shape_margin)
            return
        api.prism_assign_shapes(self.stats, self.grid, self.shapes, self.shape_params, self.shape_id,
                                self.shape_margin)

    def permute_qkv(self, q, k, v):
        """Q, K, V into slot order; block_valid (block heads, when volumes are mixed) from Q's
        pass; with a uniform volume also the pooled means of Q and K."""
        if self.mixed is not None:
            self.permute(q, self.qp, block_valid=self.unit_valid)
            api.prism_block_heads(self.unit_valid, self.shape_id, self.grid, self.shapes, self.bvalid)
            self.permute(k, self.kp)
        else:
            api.prism_permute_pool(q, self.qp, self.grid, self.shapes, self.shape_id, self.qbar, self.bvalid)
            api.prism_permute_pool(k, self.kp, self.grid, self.shapes, self.shape_id, self.kbar)
        self.permute(v, self.vp)

    def permute(self, x, y, inverse=False, block_valid=None):
        api.prism_permute(x, y, self.grid, self.shapes, self.shape_id, inverse, block_valid)

    def select(self, from_slots: bool = False):
        """Scores, hybrid cut and reverse index.  With a uniform volume this starts from the
        pooled means that permute_qkv wrote (qbar, kbar); from_slots=True pools Q' and K'
        inside the selection instead (prism_select_blocks), for Q' and K' filled by other
        means."""
        if from_slots and self.fused_pool:
            if getattr(self, "_ws_sel_slots", None) is None:
                self._ws_sel_slots = torch.empty(api.prism_select_workspace_size(self.B, self.Hh, self.nb, self.d),
                                                 dtype=torch.uint8, device=self.device)
            api.prism_select_blocks(self.qp, self.kp, self.bvalid, self.vol, self.scale, self.sel_params,
                                    self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx, self._ws_sel_slots,
                                    self.sel_margin)
        elif self.fused_pool:
            api.prism_select_blocks_pooled(self.qbar, self.kbar, self.bvalid, self.scale, self.sel_params,
                                           self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx, self.ws_sel,
                                           self.sel_margin)
        else:
            api.prism_select_blocks(self.qp, self.kp, self.bvalid, self.vol, self.scale, self.sel_params,
                                    self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx, self.ws_sel,
                                    self.sel_margin)
        if self.mixed is not None:
            api.prism_blocks_to_tiles_mixed(self.bvalid, self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx,
                                            self.max_units, self.tile_idx, self.tile_cnt, self.tile_rev_ptr,
                                            self.tile_rev_idx, self.ws_tiles)
        elif self.vol > 64:
            api.prism_blocks_to_tiles(self.bvalid, self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx, self.vol,
                                      self.tile_valid, self.tile_idx, self.tile_cnt, self.tile_rev_ptr,
                                      self.tile_rev_idx, self.ws_tiles)

    def _attn_lists(self):
        """(valid counts, lists, counts, reverse pointers, reverse lists, rows per unit) the
        attention runs on: the blocks themselves, or their 64-row tiles."""
        if self.mixed is not None:
            return (self.unit_valid, self.tile_idx, self.tile_cnt, self.tile_rev_ptr, self.tile_rev_idx, 64)
        if self.vol > 64:
            return (self.tile_valid, self.tile_idx, self.tile_cnt, self.tile_rev_ptr, self.tile_rev_idx, 64)
        return (self.bvalid, self.sel_idx, self.sel_cnt, self.rev_ptr, self.rev_idx, self.vol)

    def attn_fwd(self):
        bv, idx, cnt, _, _, vol = self._attn_lists()
        api.prism_sparse_attn_fwd(self.qp, self.kp, self.vp, bv, idx, cnt, vol, self.scale, self.op, self.lse,
                                  self.ws_fwd)

    def attn_bwd(self, marks=None):
        g = self._grads()
        bv, idx, cnt, rp, ri, vol = self._attn_lists()
        api.prism_sparse_attn_bwd(self.qp, self.kp, self.vp, self.op, g["dop"], self.lse, bv, idx, cnt, rp, ri, vol,
                                  self.scale, g["dqp"], g["dkp"], g["dvp"], self.ws_bwd, marks)

    # ---- whole layer
    def forward(self, q, k, v, a2v=None, shape_id: Optional[torch.Tensor] = None,
                a2v_norm: Optional[torch.Tensor] = None):
        """a2v: the A2V cross-attention output [B, Hh, N, d]; or a2v_norm: its per-token
        norm [B, Hh, N] (see a2v_norm()); or shape_id: given shapes, no statistics."""
        if shape_id is None:
            feat = {"v": v, "q": q, "k": k}[self.features]
            if a2v_norm is not None:
                self.zone_stats_from_norm(feat, a2v_norm)
            else:
                self.zone_stats(feat, a2v)
            self.assign_shapes()
        else:
            self.check_shape_ids(shape_id)
            self.shape_id.copy_(shape_id)
        self.permute_qkv(q, k, v)
        self.select()
        self.attn_fwd()
        self.permute(self.op, self.o, inverse=True)
        return self.o

    def check_shape_ids(self, shape_id: torch.Tensor) -> None:
        """Given shapes (ablations) must name a candidate that tiles the zone; raises
        otherwise (the permutation would map no token for such a zone)."""
        ids = shape_id.detach().to("cpu", torch.int64).reshape(-1)
        n = int(self.shapes.n)
        if tuple(shape_id.shape) != (self.B, self.Hh, self.nZ):
            raise ValueError(f"shape_id has shape {tuple(shape_id.shape)}, expected {(self.B, self.Hh, self.nZ)}")
        if ids.numel() and (int(ids.min()) < 0 or int(ids.max()) >= n):
            raise ValueError(f"shape ids must lie in [0, {n}), got [{int(ids.min())}, {int(ids.max())}]")
        g = self.grid
        bad = [c for c in range(n) if g.zt % self.shapes.bt[c] or g.zh % self.shapes.bh[c] or g.zw % self.shapes.bw[c]]
        if bad and bool(torch.isin(ids, torch.tensor(bad)).any()):
            raise ValueError(f"shape ids {bad} name candidates that do not tile the {g.zt}x{g.zh}x{g.zw} zone")

    def backward(self, do, marks=None):
        g = self._grads()
        self.permute(do, g["dop"])
        self.attn_bwd(marks)
        self.permute(g["dqp"], g["dq"], inverse=True)
        self.permute(g["dkp"], g["dk"], inverse=True)
        self.permute(g["dvp"], g["dv"], inverse=True)
        return g["dq"], g["dk"], g["dv"]

    @classmethod
    def for_workload(cls, w, device="cuda", heads: Optional[int] = None, **kw):
        """A layer sized for a workload; keyword arguments override its cands, top_p,
        k_min, k_max or set the ablation options."""
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        args = dict(cands=list(w.cands), top_p=w.top_p, k_min=w.k_min, k_max=w.k_max)
        args.update(kw)
        return cls(w.B, w.heads if heads is None else heads, w.d, w.grid, w.zone, dtype=dt, device=device, **args)
