"""Benchmark of one Prism attention layer (forward + backward) on one MI355X.

A step is one pass of the whole path over the 2K-like workload (B=1, 4-head slice of a
40-head layer, d=128, grid 21x90x160 = 302,400 tokens, 64-token shapes, Top-p 0.85,
Top-k 32..768): zone statistics, shape assignment, permutation of Q/K/V, pooling +
hybrid selection + reverse index, sparse attention forward, inverse permutation of O,
permutation of dO, sparse attention backward, inverse permutation of dQ/dK/dV.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line.  `value` is effective TFLOP/s of the whole step: 14*d flops per
selected valid (query, key) token pair (forward 4d, backward 10d) divided by the step
time.  Also reported: ms per step (= per layer), attention-only TFLOP/s, per-stage
times, the dense comparator's time on the same inputs and the speedup over it, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def selection_sums(L):
    """Sums over heads of the selection, all in valid token rows:
    tok_pairs = sum_I n_I * sum_{J in sel(I)} n_J      (valid (query, key) token pairs)
    key_rows  = sum_I sum_{J in sel(I)} n_J            (key rows streamed, query-major kernels)
    qry_rows  = sum_I cnt_I * n_I                      (query rows streamed, key-major kernel)
    rows      = sum_I n_I                              (valid rows)"""
    import torch
    idx = L.sel_idx.long()                                           # [B, Hh, nb, k_max]
    bv = L.bvalid.long()                                             # [B, Hh, nb]
    nJ = torch.gather(bv, 2, idx.clamp(min=0).reshape(L.B, L.Hh, -1)).reshape(idx.shape)
    keys = (nJ * (idx >= 0)).sum(dim=-1)                             # [B, Hh, nb]
    return dict(tok_pairs=int((keys * bv).sum().item()), key_rows=int(keys.sum().item()),
                qry_rows=int((L.sel_cnt.long() * bv).sum().item()), rows=int(bv.sum().item()),
                block_pairs=int(L.sel_cnt.long().sum().item()))


def kernel_bytes(sums, d):
    """Algorithmic HBM bytes of one launch of each attention kernel (bf16 tensors, fp32 LSE/D):
    every selected pair streams the valid rows of the other block's two tiles once; each owner
    block reads its own tiles and writes its outputs once."""
    e = 2
    return {
        "sparse_attn_fwd": sums["key_rows"] * 2 * d * e + sums["rows"] * (2 * d * e + 4),
        "sparse_attn_bwd_dkdv": sums["qry_rows"] * (2 * d * e + 8) + sums["rows"] * 4 * d * e,
        "sparse_attn_bwd_dq": sums["key_rows"] * 2 * d * e + sums["rows"] * (3 * d * e + 8),
    }


# kernel (bench name) -> symbol of its HIP kernel
KERNEL_SYMBOL = {"sparse_attn_fwd": "k_fwd", "sparse_attn_bwd_dkdv": "k_dkdv32", "sparse_attn_bwd_dq": "k_dq32"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernels_2k_like_traffic.txt")
# Counter calibration: one elementwise pass y = -x over 256 MiB of fp32 (reads and writes
# 256 MiB each); FETCH_SIZE and WRITE_SIZE are scaled by what they report for it.
COPY_MIB = 256


def attn_source_sha256():
    """Hash of the attention kernels' source file: recorded counter traffic is reported
    only while the kernels are the ones it was measured on."""
    import hashlib
    with open(os.path.join(ROOT, "content_adaptive_block_zone_amd", "csrc", "attn_mfma.hip"), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha, traffic = None, {}
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) == 2 and f[0] == "source_sha256":
            sha = f[1]
        elif len(f) == 3 and f[0] == "traffic_bytes_per_launch":
            traffic[f[1]] = int(f[2])
    if sha != attn_source_sha256():
        return None
    return traffic.get(kernel)


def summarize_profile(stats_dir, fetch_dir, write_dir, commands):
    """Text summary of a `rocprofv3 --kernel-trace --stats` run of the benchmark and of its
    FETCH_SIZE / WRITE_SIZE counter runs, with the traffic per launch of each attention
    kernel scaled by what the counters read for the plain copy (written to stdout)."""
    import csv
    import glob
    lines = ["# Commands (one MI355X, repository at /root/repo; rocprofv3 runs from /tmp)"]
    lines += [f"#   {c}" for c in commands]
    lines.append("")
    st = glob.glob(os.path.join(stats_dir, "*kernel_stats.csv"))[0]
    lines.append("## Kernel time (rocprofv3 --kernel-trace --stats)")
    lines.append(f"{'kernel':44s} {'calls':>6s} {'avg ms':>10s} {'total %':>8s}")
    import re
    for r in csv.DictReader(open(st)):
        m = re.search(r"::(k_\w+)", r["Name"])
        n = m.group(1) if m else r["Name"][:44]
        lines.append(f"{n:44s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:10.4f} {float(r['Percentage']):8.2f}")
    lines.append("")
    per = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        f = glob.glob(os.path.join(d, "*counter_collection*.csv"))[0]
        acc = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != cname:
                continue
            m = re.search(r"::(k_\w+)", r["Kernel_Name"])
            n = m.group(1) if m else ("neg_kernel (calibration)" if "neg_kernel" in r["Kernel_Name"]
                                      else r["Kernel_Name"][:44])
            a = acc.setdefault(n, [0.0, set()])
            a[0] += float(r["Counter_Value"])
            a[1].add(r["Dispatch_Id"])
        per[cname] = {n: v[0] / len(v[1]) for n, v in acc.items()}   # KiB per dispatch
    copy = [n for n in per["FETCH_SIZE"] if n == "neg_kernel (calibration)"]
    if len(copy) != 1:
        raise SystemExit("no calibration pass in the counter runs (run the benchmark with --copy-mib 256)")
    cn = copy[0]
    ref_kib = COPY_MIB * 1024.0
    sf = ref_kib / per["FETCH_SIZE"][cn]
    sw = ref_kib / per["WRITE_SIZE"][cn]
    lines.append("## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)")
    lines.append(f"calibration: {cn} of {COPY_MIB} MiB reads FETCH_SIZE {per['FETCH_SIZE'][cn]:.0f} KiB and "
                 f"WRITE_SIZE {per['WRITE_SIZE'][cn]:.0f} KiB per dispatch -> scale fetch x{sf:.3f}, write x{sw:.3f}")
    lines.append(f"{'kernel':44s} {'FETCH KiB':>14s} {'WRITE KiB':>12s} {'scaled GB':>10s}")
    for n in sorted(per["FETCH_SIZE"]):
        if not n.startswith("k_"):
            continue
        fk, wk = per["FETCH_SIZE"][n], per["WRITE_SIZE"].get(n, 0.0)
        tb = (fk * sf + wk * sw) * 1024.0
        lines.append(f"{n:44s} {fk:14.0f} {wk:12.0f} {tb / 1e9:10.3f}")
    lines.append("")
    lines.append("## Machine-readable (read by bench.py for roofline.traffic)")
    lines.append(f"source_sha256 {attn_source_sha256()}")
    for bench_name, sym in KERNEL_SYMBOL.items():
        if sym in per["FETCH_SIZE"]:
            tb = (per["FETCH_SIZE"][sym] * sf + per["WRITE_SIZE"].get(sym, 0.0) * sw) * 1024.0
            lines.append(f"traffic_bytes_per_launch {bench_name} {int(round(tb))}")
    print("\n".join(lines))


def parse_ablation(spec: str, w):
    """Layer settings for an ablation run (Table 7: Top-k only / Top-p only; Table 9:
    fixed or random shapes, query/key features, global variance), comma-separated:
    topk=F (top_p = 1, k = F * live blocks), topp=P (k_min = 1, k_max = nb),
    fixed=BTxBHxBW, random[=SEED], features=q|k, variance=global; block volumes (Tables 9
    and 11): sets=C128 | C256 (one larger set), mixed[=TAU128:TAU256] (C_64 + C_128 +
    C_256 chosen per zone by the activity thresholds).
    Returns (PrismLayer keyword arguments, shape ids or None)."""
    from content_adaptive_block_zone_amd.pipeline import random_shape_ids
    kw, ids = {}, None
    if not spec:
        return kw, ids
    T, H, W = w.grid
    zt, zh, zw = w.zone
    nZ = -(-T // zt) * -(-H // zh) * -(-W // zw)
    nb = nZ * (zt * zh * zw) // w.vol
    for item in spec.split(","):
        key, _, val = item.partition("=")
        if key == "topk":
            k = max(1, int(round(float(val) * nb)))
            kw.update(top_p=1.0, k_min=k, k_max=k)
        elif key == "topp":
            kw.update(top_p=float(val), k_min=1, k_max=nb)
        elif key == "fixed":
            kw.update(cands=[tuple(int(e) for e in val.split("x"))])
        elif key == "random":
            ids = random_shape_ids(w.B, w.heads, w.grid, w.zone, list(w.cands), int(val or 0))
        elif key == "sets":
            from workloads import CANDS_128, CANDS_256
            kw.update(cands={"C128": CANDS_128, "C256": CANDS_256}[val])
        elif key == "mixed":
            from workloads import CANDS_128, CANDS_256
            t128, t256 = (float(t) for t in val.split(":")) if val else (1.0, 0.5)
            kw.update(cands=list(w.cands) + CANDS_128 + CANDS_256, mixed=(t128, t256))
        elif key == "features":
            kw.update(features=val)
        elif key == "variance":
            kw.update(variance=val)
        else:
            raise SystemExit(f"unknown ablation setting {item!r}")
    return kw, ids


def density(L):
    import torch
    live = (L.bvalid > 0).sum(dim=-1).double()                      # [B, Hh]
    per_head = L.sel_cnt.double().sum(dim=-1) / (live * live)
    return float(per_head.mean().item())


def run_gpu(args):
    import torch

    from content_adaptive_block_zone_amd import _lib, api
    from content_adaptive_block_zone_amd.pipeline import PrismLayer
    from workloads import workload
    from workloads.synth import make_inputs

    _lib.load()
    w = workload(args.workload)
    t0 = time.time()
    x = make_inputs(w, seed=args.workload, with_grad=not args.forward_only)
    log(f"[bench] inputs of {w.name} generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    q, k, v, a2v = (x[n].to(dev) for n in ("q", "k", "v", "a2v"))
    do = x["do"].to(dev) if "do" in x else None
    kw, shape_ids = parse_ablation(args.ablation, w)
    L = PrismLayer.for_workload(w, device=dev, **kw)
    if shape_ids is not None:
        shape_ids = shape_ids.to(dev)
    feat = {"v": v, "q": q, "k": k}[L.features]
    stream = torch.cuda.current_stream()

    fwd_only = args.forward_only

    def stats_and_shapes():
        if shape_ids is None:
            L.zone_stats(feat, a2v)
            L.assign_shapes()
        else:
            L.shape_id.copy_(shape_ids)

    def step(ev=None):
        if ev is None:
            L.forward(q, k, v, a2v, shape_id=shape_ids)
            if not fwd_only:
                L.backward(do)
            return
        stats_and_shapes()
        L.permute_qkv(q, k, v)
        ev["select0"].record(stream)
        L.select()
        ev["fwd0"].record(stream)
        L.attn_fwd()
        ev["fwd1"].record(stream)
        L.permute(L.op, L.o, inverse=True)
        if fwd_only:
            return
        g = L._grads()
        L.permute(do, g["dop"])
        L.attn_bwd(marks=ev["marks"])
        L.permute(g["dqp"], g["dq"], inverse=True)
        L.permute(g["dkp"], g["dk"], inverse=True)
        L.permute(g["dvp"], g["dv"], inverse=True)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    if args.copy_mib:
        # one plain elementwise pass of known size (y = -x): the counter runs scale
        # FETCH_SIZE and WRITE_SIZE by what they read for it
        src = torch.ones(args.copy_mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # events for the kernels timed inside the region (one set per step)
    def new_events():
        e = {n: torch.cuda.Event(enable_timing=True) for n in ("select0", "fwd0", "fwd1")}
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for m in marks:
            m.record(stream)                      # materialise the handles
        e["marks"] = marks
        return e

    evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1e3 * t_total / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step")

    t_select = sum(e["select0"].elapsed_time(e["fwd0"]) for e in evs) / len(evs)
    t_fwd = sum(e["fwd0"].elapsed_time(e["fwd1"]) for e in evs) / len(evs)
    if fwd_only:
        t_pre = t_dkdv = t_dq = 0.0
    else:
        t_pre = sum(e["marks"][0].elapsed_time(e["marks"][1]) for e in evs) / len(evs)
        t_dkdv = sum(e["marks"][1].elapsed_time(e["marks"][2]) for e in evs) / len(evs)
        t_dq = sum(e["marks"][2].elapsed_time(e["marks"][3]) for e in evs) / len(evs)

    sums = selection_sums(L)
    pairs = sums["tok_pairs"]
    dens = density(L)
    d = w.d
    f_sel = (4.0 if fwd_only else 14.0) * d * pairs
    value = f_sel / (ms_step * 1e-3) / 1e12
    t_attn = t_fwd + t_pre + t_dkdv + t_dq
    attn_tflops = f_sel / (t_attn * 1e-3) / 1e12

    # dominant kernel: the one with the largest share of the step.  At about 64 flop per
    # streamed byte these kernels sit far below MI355X's ridge point (2.5 PFLOP/s / 8 TB/s
    # = 312 flop/B), so their roofline is HBM bandwidth on algorithmic bytes.
    kb = kernel_bytes(sums, d)
    kern = {"sparse_attn_fwd": t_fwd, "sparse_attn_bwd_dkdv": t_dkdv, "sparse_attn_bwd_dq": t_dq}
    if fwd_only:
        kern = {"sparse_attn_fwd": t_fwd}
    dom = max(kern, key=lambda n: kern[n])
    t_dom = kern[dom]
    achieved = kb[dom] / (t_dom * 1e-3) / 1e9
    kflops = {"sparse_attn_fwd": 4.0 * d * pairs, "sparse_attn_bwd_dkdv": 8.0 * d * pairs,
              "sparse_attn_bwd_dq": 2.0 * d * pairs}

    # per-stage breakdown from one extra instrumented pass (outside the timed region)
    stage = {}
    names = ["zone_stats", "assign_shapes", "permute_qkv", "select", "attn_fwd", "unpermute_o", "permute_do",
             "attn_bwd", "unpermute_grads"]
    calls = [lambda: L.zone_stats(feat, a2v) if shape_ids is None else L.shape_id.copy_(shape_ids),
             lambda: L.assign_shapes() if shape_ids is None else None,
             lambda: L.permute_qkv(q, k, v),
             L.select, L.attn_fwd, lambda: L.permute(L.op, L.o, inverse=True)]
    if fwd_only:
        names = names[:len(calls)]
    else:
        g = L._grads()
        calls += [lambda: L.permute(do, g["dop"]), L.attn_bwd,
                  lambda: (L.permute(g["dqp"], g["dq"], inverse=True), L.permute(g["dkp"], g["dk"], inverse=True),
                           L.permute(g["dvp"], g["dv"], inverse=True))]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    ev[0].record(stream)
    for i, c in enumerate(calls):
        c()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    for i, n in enumerate(names):
        stage[n] = round(ev[i].elapsed_time(ev[i + 1]), 4)

    # dense comparator on the same (unpermuted) inputs
    dense = None
    if not args.no_dense:
        o_d = torch.empty_like(q)
        lse_d = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        wsf = torch.empty(max(1, api.prism_dense_fwd_workspace_size(w.B, w.heads, w.N, w.d)), dtype=torch.uint8,
                          device=dev)
        if not fwd_only:
            dq_d, dk_d, dv_d = (torch.empty_like(q) for _ in range(3))
            ws = torch.empty(api.prism_dense_bwd_workspace_size(w.B, w.heads, w.N, w.d), dtype=torch.uint8,
                             device=dev)

        def dense_step():
            api.prism_dense_attn_fwd(q, k, v, L.scale, o_d, lse_d, wsf)
            if not fwd_only:
                api.prism_dense_attn_bwd(q, k, v, o_d, do, lse_d, L.scale, dq_d, dk_d, dv_d, ws)

        dense_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_steps):
            dense_step()
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_steps
        dflops = (4.0 if fwd_only else 14.0) * d * w.N * w.N * w.B * w.heads
        dense = dict(ms=round(dense_ms, 3), tflops=round(dflops / (dense_ms * 1e-3) / 1e12, 2),
                     speedup=round(dense_ms / ms_step, 3))
        log(f"[bench] dense comparator: {dense}")

    res = dict(
        metric=("ms/layer & effective TFLOP/s, sparse attn fwd (inference) ; speedup vs dense" if fwd_only else
                "ms/layer & effective TFLOP/s, sparse attn fwd+bwd at 2K; speedup vs dense"),
        value=round(value, 3), unit="TFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_step, 3), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if w.dtype == "bf16" else "f32", data="synthetic",
        config=dict(workload=f"{w.name}: B={w.B}, {w.heads} heads, d={w.d}, grid {w.grid[0]}x{w.grid[1]}x{w.grid[2]} "
                             f"({w.N} tokens), zone {w.zone[0]}x{w.zone[1]}x{w.zone[2]}, {len(w.cands)} shapes of "
                             f"{w.vol} tokens, top-p {w.top_p}, top-k {w.k_min}..{w.k_max}",
                    B=w.B, heads=w.heads, d=w.d, tokens=w.N, nb=L.nb, npad=L.Npad, density=round(dens, 4),
                    selected_token_pairs=pairs, selected_block_pairs=sums["block_pairs"],
                    **({"ablation": args.ablation} if args.ablation else {})),
        ms_per_layer=round(ms_step, 3),
        attn_tflops=round(attn_tflops, 3),
        attn_ms=dict(fwd=round(t_fwd, 4), bwd_pre=round(t_pre, 4), bwd_dkdv=round(t_dkdv, 4), bwd_dq=round(t_dq, 4)),
        select_ms=round(t_select, 4),
        stage_ms=stage,
        dense=dense,
        speedup_vs_dense=None if dense is None else dense["speedup"],
        roofline=dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=MI355X_HBM_GBPS, unit="GB/s",
                      frac=round(achieved / MI355X_HBM_GBPS, 4), traffic=recorded_traffic(dom), avg_ms=round(t_dom, 4),
                      bytes_per_launch=kb[dom],
                      mfma_tflops=round(kflops[dom] / (t_dom * 1e-3) / 1e12, 2),
                      mfma_frac=round(kflops[dom] / (t_dom * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 4)),
        kernels={n: dict(ms=round(kern[n], 4), gbps=round(kb[n] / (kern[n] * 1e-3) / 1e9, 1),
                         frac_hbm=round(kb[n] / (kern[n] * 1e-3) / 1e9 / MI355X_HBM_GBPS, 4)) for n in kern},
    )
    return res, (w, x)


def cpu_baseline(w, x, budget_blocks: int, fwd_only: bool = False):
    """The oracle as it stands, on one head of the same inputs: the whole chain for that
    head with the attention restricted to `budget_blocks` query blocks (forward, and
    unless fwd_only the full backward of exactly those blocks' selected pairs)."""
    import numpy as np
    import threadpoolctl

    from oracle import prism_oracle as O

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    h = 0
    n = {k: t[:, h:h + 1].float().numpy().astype(np.float64) for k, t in x.items()}
    t0 = time.perf_counter()
    scale = 1.0 / math.sqrt(w.d)
    stats = O.zone_stats(n["v"], n["a2v"], w.grid, w.zone)
    sid, _ = O.assign_shapes(stats.astype(np.float32), list(w.cands), w.zone)
    tok = O.slot_map(w.grid, w.zone, list(w.cands), sid)
    bv = O.block_valid(tok, w.vol)
    qp, kp, vp = O.permute(n["q"], tok), O.permute(n["k"], tok), O.permute(n["v"], tok)
    qb, kb = O.pool_blocks(qp, bv, w.vol), O.pool_blocks(kp, bv, w.vol)
    live = np.nonzero(bv[0, 0] > 0)[0]
    rows = live[np.linspace(0, live.size - 1, budget_blocks).astype(int)]
    sel, _ = O.select_blocks(qb.astype(np.float32), kb.astype(np.float32), bv, scale, w.top_p, w.k_min,
                             w.k_max, rows=rows)
    blocks = [(0, 0, int(I)) for I in rows]
    op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, scale, w.vol, blocks=blocks)
    if not fwd_only:
        dop = O.permute(n["do"], tok)
        touched = sorted({(0, 0, int(J)) for s in sel.values() for J in s})
        O.sparse_attn_bwd(qp, kp, vp, op, dop, lse, bv, sel, scale, w.vol, q_blocks=blocks, k_blocks=touched)
    dt = time.perf_counter() - t0
    pairs = sum(int(bv[0, 0, I]) * int(bv[0, 0, s].sum()) for (_, _, I), s in sel.items())
    flops = (4.0 if fwd_only else 14.0) * w.d * pairs
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                seconds=round(dt, 2),
                sample=(f"head 0 of {w.name}: zone stats, shapes, permutation and pooling of the whole head, "
                        f"selection, forward{'' if fwd_only else ' and backward'} of {budget_blocks} query blocks "
                        f"({pairs} valid token pairs, {4 if fwd_only else 14}*d flops each), float64 numpy"))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--ablation", default="",
                    help="ablation settings, e.g. topk=0.15 | topp=0.5 | fixed=4x4x4 | random=1 | features=q | "
                         "variance=global (comma-separated)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the forward chain only (inference; e.g. --workload 5)")
    ap.add_argument("--dense-steps", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=200)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one elementwise pass y = -x over this many MiB after warm-up (counter calibration)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="print a text summary of rocprofv3 output directories and exit (no GPU)")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="command line recorded in the summary (repeatable)")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, args.profile_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every Prism step is independent per head, so a multi-GPU "
              "layer shards heads with no communication; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    res, (w, x) = run_gpu(args)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle sample ...")
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_blocks, args.forward_only)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
