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
KERNEL_SYMBOL = {"sparse_attn_fwd": "k_fwd<true>", "sparse_attn_bwd_dkdv": "k_dkdv32", "sparse_attn_bwd_dq": "k_dq32"}
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


def _rocpd(path):
    """The rocprofv3 database (rocpd SQLite) under a result directory."""
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "**", "*results.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {path}")
    return sqlite3.connect(dbs[0])


def _short(name):
    import re
    m = re.search(r"::(k_\w+)", name)
    if m:
        t = re.search(r"k_\w+(<[^>(]*>)?", name[m.start(1):])
        return t.group(0) if t else m.group(1)
    return "neg_kernel (calibration)" if "neg_kernel" in name else name[:44]


def summarize_profile(stats_dir, fetch_dir, write_dir, commands):
    """Text summary of a `rocprofv3 --kernel-trace --stats` run of the benchmark and, when
    given, of its FETCH_SIZE / WRITE_SIZE counter runs, with the traffic per launch of each
    attention kernel scaled by what the counters read for the plain copy (to stdout)."""
    lines = ["# Commands (one MI355X, repository root as working copy; rocprofv3 runs with TMPDIR=/tmp)"]
    lines += [f"#   {c}" for c in commands]
    lines.append("")
    db = _rocpd(stats_dir)
    lines.append("## Kernel time (rocprofv3 --kernel-trace --stats)")
    lines.append(f"{'kernel':44s} {'calls':>6s} {'avg ms':>10s} {'total %':>8s}")
    for name, calls, _tot, avg, pct in db.execute(
            "select name, total_calls, total_duration, average, percentage from top_kernels"):
        # the database's summary view gives durations in microseconds
        lines.append(f"{_short(name):44s} {int(calls):6d} {float(avg) / 1e3:10.4f} {float(pct):8.2f}")
    lines.append("")
    if fetch_dir and write_dir:
        per = {}
        for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            acc = {}
            for kname, disp, val in _rocpd(d).execute(
                    "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?",
                    (cname,)):
                a = acc.setdefault(_short(kname), [0.0, set()])
                a[0] += float(val)
                a[1].add(disp)
            per[cname] = {n: v[0] / len(v[1]) for n, v in acc.items()}   # KiB per dispatch
        cn = "neg_kernel (calibration)"
        if cn not in per["FETCH_SIZE"]:
            raise SystemExit("no calibration pass in the counter runs (run the benchmark with --copy-mib 256)")
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
            lines.append(f"{n:44s} {fk:14.0f} {wk:12.0f} {(fk * sf + wk * sw) * 1024.0 / 1e9:10.3f}")
        lines.append("")
        lines.append("## Machine-readable (read by bench.py for roofline.traffic)")
        lines.append(f"source_sha256 {attn_source_sha256()}")
        for bench_name, sym in KERNEL_SYMBOL.items():
            if sym in per["FETCH_SIZE"]:
                tb = (per["FETCH_SIZE"][sym] * sf + per["WRITE_SIZE"].get(sym, 0.0) * sw) * 1024.0
                lines.append(f"traffic_bytes_per_launch {bench_name} {int(round(tb))}")
    print("\n".join(lines))


def summarize_counters(sqa, sqb, l2, lat, pairs, commands):
    """Text summary of the four counter runs of the benchmark (two passes of SQ counters,
    L2 hits and misses, L2-to-fabric read requests with their in-flight level) for the
    attention kernels, per launch, averaged over the launches (to stdout)."""
    per = {}
    for d in (sqa, sqb, l2, lat):
        for kname, disp, cname, val in _rocpd(d).execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            k = per.setdefault(_short(kname), {})
            c = k.setdefault(cname, {})
            c[disp] = c.get(disp, 0.0) + float(val)
    avg = {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    lines = ["# Commands (one MI355X, repository root as working copy; rocprofv3 runs with TMPDIR=/tmp)"]
    lines += [f"#   {c}" for c in commands]
    lines += [f"# 2K-like workload ({pairs:,} selected block pairs), per launch, averaged over the launches.",
              "# GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles = GRBM_GUI_ACTIVE / 8.",
              "#   MFMA check    = SQ_INSTS_MFMA / (pairs x products per pair: 64 forward, 128 dK/dV, 96 dQ)",
              "#   MFMA busy     = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles)",
              "#   LDS active    = SQ_LDS_IDX_ACTIVE / (256 CUs x cycles)",
              "#   LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
              "#   wait any      = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave cycles waiting on a dependency)",
              "#   wait LDS      = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES",
              "#   L2 hit        = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)",
              "#   read latency  = TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum (mean cycles an L2 read miss is in flight)"]
    hdr = (f"{'kernel':12s} {'cycles':>10s} {'MFMA check':>10s} {'MFMA busy':>9s} {'LDS active':>10s} "
           f"{'LDS confl':>9s} {'wait any':>8s} {'wait LDS':>8s} {'LDS FIFO full':>13s} {'L2 hit':>6s} "
           f"{'read lat':>8s}")
    lines.append(hdr)
    raw = []
    for bench_name, sym in KERNEL_SYMBOL.items():
        a = avg.get(sym)
        if not a:
            continue
        g = lambda c: a.get(c, float("nan"))  # noqa: E731
        cyc = g("GRBM_GUI_ACTIVE") / 8.0
        mchk = g("SQ_INSTS_MFMA") / (pairs * MFMA_PER_PAIR[bench_name])
        hit = g("TCC_HIT_sum") / (g("TCC_HIT_sum") + g("TCC_MISS_sum"))
        lat = g("TCC_EA0_RDREQ_LEVEL_sum") / g("TCC_EA0_RDREQ_sum")
        lines.append(f"{sym:12s} {cyc:10.3e} {mchk:10.4f} {g('SQ_VALU_MFMA_BUSY_CYCLES') / (1024 * cyc):9.3f} "
                     f"{g('SQ_LDS_IDX_ACTIVE') / (256 * cyc):10.3f} "
                     f"{g('SQ_LDS_BANK_CONFLICT') / g('SQ_LDS_IDX_ACTIVE'):9.4f} "
                     f"{g('SQ_WAIT_INST_ANY') / g('SQ_WAVE_CYCLES'):8.3f} "
                     f"{g('SQ_WAIT_INST_LDS') / g('SQ_WAVE_CYCLES'):8.3f} {g('SQ_LDS_DATA_FIFO_FULL'):13.3e} "
                     f"{hit:6.3f} {lat:8.0f}")
        raw.append(f"# {sym}: " + ", ".join(f"{c} {v:.4e}" for c, v in sorted(a.items())))
    lines.append("")
    lines.append("# Raw counters per launch")
    lines += raw
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


MFMA_PER_PAIR = {"sparse_attn_fwd": 64, "sparse_attn_bwd_dkdv": 128, "sparse_attn_bwd_dq": 96}
"""32x32x16 matrix-core products (32768 flops each) issued per selected 64x64 block pair:
forward 64 (32 for S in bf16, 32 for P V in fp16), dK/dV 128 (S, dP, dV, dK), dQ 96 (S
and dP recomputed, then dQ)."""


def flush_cache(buf):
    """Read a buffer twice the size of the 256 MB last-level cache, so that the next kernel
    reads its inputs from HBM as it does inside the layer.  A read evicts the cache without
    leaving dirty lines behind (those of earlier work drain during the read itself).
    Enqueued only: the host does not wait for it."""
    return buf.max()


def dirty_cache(buf):
    """Overwrite a buffer twice the size of the last-level cache: the next kernel then
    starts while 512 MB of dirty lines drain to HBM (the state after a large write)."""
    buf.zero_()


def time_stages(L, calls, reps, flush_buf):
    """Per-stage GPU time: each stage enqueued `reps` times, each run preceded by a cache
    flush and bracketed by its own pair of events on the launch stream; the median over
    runs.  The host enqueues everything before synchronising once, so the GPU runs the
    work back to back and the events see kernel time, not host launch latency."""
    import torch
    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in calls:
        evs = []
        for _ in range(reps):
            flush_cache(flush_buf)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)
        out[name] = round(t[len(t) // 2], 4)
    return out


def mfma_peak(dev, reps=3):
    """The project's own matrix-core loop (prism_bench_mfma_peak): 512 workgroups of 4
    waves (2 per SIMD), four independent 32x32x16 bf16 products per wave and step.
    Returns (best TFLOP/s, mean shader clock in MHz over that run)."""
    import torch

    from content_adaptive_block_zone_amd import api
    wgs, iters = 512, 4096
    clocks = torch.zeros(wgs, 2, dtype=torch.int64, device=dev)
    sink = torch.zeros(wgs, dtype=torch.float32, device=dev)
    api.prism_bench_mfma_peak(wgs, 64, clocks, sink)       # warm-up
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.prism_bench_mfma_peak(wgs, iters, clocks, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        tf = wgs * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12
        c = clocks.double().cpu()
        mhz = float((c[:, 0] / c[:, 1].clamp(min=1)).mean()) * 100.0
        if best is None or tf > best[0]:
            best = (tf, mhz)
    return round(best[0], 1), round(best[1], 1)


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
    fused_a2v = args.a2v == "fused"
    if fused_a2v:
        # the model's audio-to-video cross-attention (video queries over audio keys and
        # values drawn N(0, 1)) run by the library's kernel, which writes its output rows
        # and the per-token norm; the statistics read the norm map instead of the rows
        ga = torch.Generator().manual_seed(1000 + args.workload)
        ka, va = (torch.randn(w.B, w.heads, w.n_audio, w.d, generator=ga).to(torch.bfloat16).to(dev) for _ in range(2))
        o_a2v = torch.empty_like(q)
        a2v_nrm = torch.empty(w.B, w.heads, w.N, dtype=torch.float32, device=dev)

    def stats_and_shapes():
        if shape_ids is None:
            if fused_a2v:
                api.prism_a2v_attn_norm(q, ka, va, L.scale, a2v_nrm, o=o_a2v)
                L.zone_stats_from_norm(feat, a2v_nrm)
            else:
                L.zone_stats(feat, a2v)
            L.assign_shapes()
        else:
            L.shape_id.copy_(shape_ids)

    def step(ev=None):
        if ev is None:
            if fused_a2v and shape_ids is None:
                api.prism_a2v_attn_norm(q, ka, va, L.scale, a2v_nrm, o=o_a2v)
                L.forward(q, k, v, a2v_norm=a2v_nrm)
            else:
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
    # tile flops: every selected pair counted as a whole 64 x 64 tile pair, padding included
    f_tile = (4.0 if fwd_only else 14.0) * d * 64 * 64 * sums["block_pairs"]
    f_dense_eq = (4.0 if fwd_only else 14.0) * d * w.N * w.N * w.B * w.heads

    # Roofline: the attention kernels are priced on the bf16 matrix-core peak, each on its
    # own algorithmic flops (forward 4d, dK/dV 8d, dQ 2d per valid token pair); the
    # dominant kernel is the one that takes longest.
    kb = kernel_bytes(sums, d)
    kern = {"sparse_attn_fwd": t_fwd, "sparse_attn_bwd_dkdv": t_dkdv, "sparse_attn_bwd_dq": t_dq}
    if fwd_only:
        kern = {"sparse_attn_fwd": t_fwd}
    kflops = {"sparse_attn_fwd": 4.0 * d * pairs, "sparse_attn_bwd_dkdv": 8.0 * d * pairs,
              "sparse_attn_bwd_dq": 2.0 * d * pairs}
    dom = max(kern, key=lambda n: kern[n])
    t_dom = kern[dom]
    achieved = kflops[dom] / (t_dom * 1e-3) / 1e12

    # per-stage kernel time, cold cache, queued back to back (outside the timed region)
    flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    calls = [("zone_stats", lambda: L.zone_stats(feat, a2v) if shape_ids is None else L.shape_id.copy_(shape_ids)),
             ("assign_shapes", lambda: L.assign_shapes() if shape_ids is None else None),
             ("permute_pool_qkv", lambda: L.permute_qkv(q, k, v)),
             ("select", L.select), ("attn_fwd", L.attn_fwd),
             ("unpermute_o", lambda: L.permute(L.op, L.o, inverse=True))]
    if not fwd_only:
        g = L._grads()
        calls += [("permute_do", lambda: L.permute(do, g["dop"])), ("attn_bwd", L.attn_bwd),
                  ("unpermute_grads", lambda: (L.permute(g["dqp"], g["dq"], inverse=True),
                                               L.permute(g["dkp"], g["dk"], inverse=True),
                                               L.permute(g["dvp"], g["dv"], inverse=True)))]
    a2v_info = None
    if fused_a2v:
        calls[0] = ("a2v_attn_norm", lambda: api.prism_a2v_attn_norm(q, ka, va, L.scale, a2v_nrm, o=o_a2v))
        calls.insert(1, ("zone_stats_from_norm", lambda: L.zone_stats_from_norm(feat, a2v_nrm)))
    stage = time_stages(L, calls, args.stage_reps, flush_buf)
    log(f"[bench] stages (ms, cold cache): {stage}")
    if fused_a2v:
        rows = time_stages(L, [("zone_stats_from_rows", lambda: L.zone_stats(feat, o_a2v))], args.stage_reps,
                           flush_buf)["zone_stats_from_rows"]
        a2v_info = dict(mode="fused", a2v_attn_ms=stage["a2v_attn_norm"],
                        zone_stats_from_norm_ms=stage["zone_stats_from_norm"], zone_stats_from_rows_ms=rows,
                        stats_ms_saved=round(rows - stage["zone_stats_from_norm"], 4),
                        stats_bytes_saved=int(w.B * w.heads * w.N * (w.d * 2 - 4)))
        log(f"[bench] a2v: {a2v_info}")
    del flush_buf

    # measured ceilings: the matrix-core peak and clock, and the forward's tile traffic alone
    ceil = None
    if not args.no_microbench:
        pk, mhz = mfma_peak(dev)
        gop = torch.empty_like(L.op)
        bv_t, idx_t, cnt_t, _, _, vol_t = L._attn_lists()
        api.prism_bench_tile_gather(L.qp, L.kp, L.vp, bv_t, idx_t, cnt_t, vol_t, gop, L.ws_fwd)
        torch.cuda.synchronize()
        gt = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            api.prism_bench_tile_gather(L.qp, L.kp, L.vp, bv_t, idx_t, cnt_t, vol_t, gop, L.ws_fwd)
            e1.record(stream)
            torch.cuda.synchronize()
            gt.append(e0.elapsed_time(e1))
        del gop
        g_ms = sorted(gt)[1]
        # The statistics stage against a contiguous read of its input bytes (V and the A2V
        # output): both with clean caches (median of 3 after an untimed call), and the read
        # again right after a 512 MB write (dirty lines then drain to HBM during the read).
        sink = torch.empty(api.PRISM_BENCH_STREAM_SINK, dtype=torch.int32, device=dev)
        fb = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)

        def med3(fn, flush=False):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                if flush:
                    dirty_cache(fb)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return sorted(ts)[1]
        sb = a2v if a2v.numel() * a2v.element_size() == feat.numel() * feat.element_size() else feat
        s_bytes = 2 * feat.numel() * feat.element_size()
        s_clean = med3(lambda: api.prism_bench_stream_read(feat, sb, sink))
        s_flush = med3(lambda: api.prism_bench_stream_read(feat, sb, sink), flush=True)
        z_clean = med3(lambda: L.zone_stats(feat, sb))
        del sink, fb
        ceil = dict(mfma_peak_tflops=pk, mfma_peak_frac_of_spec=round(pk / MI355X_BF16_DENSE_TFLOPS, 4),
                    shader_clock_mhz=mhz,
                    fwd_tile_gather_ms=round(g_ms, 4),
                    fwd_tile_gather_gbps=round(kb["sparse_attn_fwd"] / (g_ms * 1e-3) / 1e9, 1),
                    fwd_over_gather=round(t_fwd / g_ms, 3),
                    stats_read_bytes=int(s_bytes),
                    stats_stream_ms=round(s_clean, 4),
                    stats_stream_gbps=round(s_bytes / (s_clean * 1e-3) / 1e9, 1),
                    stats_stream_after_flush_ms=round(s_flush, 4),
                    zone_stats_clean_ms=round(z_clean, 4),
                    zone_stats_clean_gbps=round(s_bytes / (z_clean * 1e-3) / 1e9, 1),
                    zone_stats_over_stream=round(z_clean / s_clean, 3))
        log(f"[bench] ceilings: {ceil}")

    # dense comparator on the same (unpermuted) inputs, per kernel
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
        mk = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for m in mk:
            m.record(stream)

        def dense_step(marks=None):
            api.prism_dense_attn_fwd(q, k, v, L.scale, o_d, lse_d, wsf)
            if not fwd_only:
                api.prism_dense_attn_bwd(q, k, v, o_d, do, lse_d, L.scale, dq_d, dk_d, dv_d, ws, marks)

        dense_step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dense_step(mk)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(mk[3]) if not fwd_only else None
        dfl = d * w.N * w.N * w.B * w.heads
        if fwd_only:
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dense_step()
            e1.record(stream)
            torch.cuda.synchronize()
            dense_ms = e0.elapsed_time(e1)
            dk_ms = {"fwd": dense_ms}
        else:
            dk_ms = {"fwd": e0.elapsed_time(mk[0]), "bwd_pre": mk[0].elapsed_time(mk[1]),
                     "bwd_dkdv": mk[1].elapsed_time(mk[2]), "bwd_dq": mk[2].elapsed_time(mk[3])}
        dflops = {"fwd": 4.0 * dfl, "bwd_dkdv": 8.0 * dfl, "bwd_dq": 2.0 * dfl}
        tot_fl = (4.0 if fwd_only else 14.0) * dfl
        dense = dict(ms=round(dense_ms, 3), tflops=round(tot_fl / (dense_ms * 1e-3) / 1e12, 2),
                     mfma_frac=round(tot_fl / (dense_ms * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 4),
                     speedup=round(dense_ms / ms_step, 3),
                     kernels={n: dict(ms=round(t, 3),
                                      **({} if n not in dflops else dict(
                                          tflops=round(dflops[n] / (t * 1e-3) / 1e12, 1),
                                          mfma_frac=round(dflops[n] / (t * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS,
                                                          4))))
                              for n, t in dk_ms.items()})
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
        tile_tflops=round(f_tile / (ms_step * 1e-3) / 1e12, 3),
        dense_equivalent_tflops=round(f_dense_eq / (ms_step * 1e-3) / 1e12, 3),
        attn_ms=dict(fwd=round(t_fwd, 4), bwd_pre=round(t_pre, 4), bwd_dkdv=round(t_dkdv, 4), bwd_dq=round(t_dq, 4)),
        select_ms=round(t_select, 4),
        stage_ms=stage,
        **({"a2v": a2v_info} if a2v_info else {}),
        dense=dense,
        speedup_vs_dense=None if dense is None else dense["speedup"],
        roofline=dict(bound="mfma", kernel=dom, achieved=round(achieved, 2), peak=MI355X_BF16_DENSE_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
                      traffic=recorded_traffic(dom), avg_ms=round(t_dom, 4), flops_per_launch=kflops[dom],
                      attn_achieved=round(attn_tflops, 2),
                      attn_frac=round(attn_tflops / MI355X_BF16_DENSE_TFLOPS, 4),
                      traffic_model_gbps=round(kb[dom] / (t_dom * 1e-3) / 1e9, 1)),
        ceilings=ceil,
        kernels={n: dict(ms=round(kern[n], 4), tflops=round(kflops[n] / (kern[n] * 1e-3) / 1e12, 2),
                         mfma_frac=round(kflops[n] / (kern[n] * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 4),
                         mfma_issued_tflops=round(MFMA_PER_PAIR[n] * 32768.0 * sums["block_pairs"] /
                                                  (kern[n] * 1e-3) / 1e12, 2),
                         traffic_model_gbps=round(kb[n] / (kern[n] * 1e-3) / 1e9, 1)) for n in kern},
    )
    return res, (w, x)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, n_blocks: int, fwd_only: bool = False):
    """The oracle in float32 (its timing precision) on the host cores, every BLAS thread
    in use, over a bounded sample of the same workload, extrapolated to the whole layer.

    Sample: head 0 (the heads are alike in size and density) -- zone statistics, shapes,
    permutation of Q, K, V, pooling and the whole head's selection in full; the forward
    and dQ of n_blocks sampled query blocks; dK/dV of n_blocks sampled key blocks (their
    O' and LSE inputs are placeholders for the rows outside the sample: the oracle's work
    does not depend on their values).  Extrapolation: each attention part scales by the
    head's selected token pairs over the sample's, and everything by the number of
    heads."""
    import numpy as np
    import threadpoolctl

    from oracle import prism_oracle as O

    nproc = len(os.sched_getaffinity(0))
    f32 = np.float32
    with threadpoolctl.threadpool_limits(nproc):
        h = 0
        n = {k: t[:, h:h + 1].float().numpy() for k, t in x.items()}
        scale = 1.0 / math.sqrt(w.d)
        t0 = time.perf_counter()
        stats = O.zone_stats(n["v"], n["a2v"], w.grid, w.zone)
        sid, _ = O.assign_shapes(stats.astype(f32), list(w.cands), w.zone)
        tok = O.slot_map(w.grid, w.zone, list(w.cands), sid)
        bv = O.block_valid(tok, w.vol)
        qp, kp, vp = O.permute(n["q"], tok), O.permute(n["k"], tok), O.permute(n["v"], tok)
        qb, kb = O.pool_blocks(qp, bv, w.vol), O.pool_blocks(kp, bv, w.vol)
        sel, _ = O.select_blocks_all(qb.astype(f32), kb.astype(f32), bv, scale, w.top_p, w.k_min, w.k_max)
        t_pre = time.perf_counter() - t0
        live = np.nonzero(bv[0, 0] > 0)[0]
        rows = live[np.linspace(0, live.size - 1, n_blocks).astype(int)]
        qblk = [(0, 0, int(I)) for I in rows]

        def pairs_of(blocks):
            return sum(int(bv[0, 0, I]) * int(bv[0, 0, sel[(0, 0, I)]].sum()) for (_, _, I) in blocks)

        head_pairs = O.selected_pair_flops(bv, sel, 1) / 14.0
        t0 = time.perf_counter()
        op, lse = O.sparse_attn_fwd(qp, kp, vp, bv, sel, scale, w.vol, blocks=qblk, dtype=f32)
        t_fwd = time.perf_counter() - t0
        parts = dict(fwd=(t_fwd, pairs_of(qblk)))
        if not fwd_only:
            dop = O.permute(n["do"], tok)
            t0 = time.perf_counter()
            O.sparse_attn_bwd(qp, kp, vp, op, dop, lse, bv, sel, scale, w.vol, q_blocks=qblk, k_blocks=[], dtype=f32)
            parts["dq"] = (time.perf_counter() - t0, pairs_of(qblk))
            rev = O._transpose_selection(sel)
            kblk = [(0, 0, int(J)) for J in rows if (0, 0, int(J)) in rev]
            lse_ph = np.where(lse == 0, 30.0, lse)            # placeholder rows: P = exp(s - 30) stays finite
            t0 = time.perf_counter()
            O.sparse_attn_bwd(qp, kp, vp, op, dop, lse_ph, bv, sel, scale, w.vol, q_blocks=[], k_blocks=kblk,
                              dtype=f32)
            kpairs = sum(int(bv[0, 0, J]) * int(bv[0, 0, rev[(0, 0, J)]].sum()) for (_, _, J) in kblk)
            parts["dkdv"] = (time.perf_counter() - t0, kpairs)
    n_k = 0 if fwd_only else len(kblk)
    sample_s = t_pre + sum(t for t, _ in parts.values())
    head_s = t_pre + sum(t * head_pairs / max(p, 1) for t, p in parts.values())
    layer_s = head_s * w.heads * w.B
    f_layer = (4.0 if fwd_only else 14.0) * w.d * head_pairs * w.heads * w.B
    return dict(value=round(f_layer / layer_s / 1e12, 6), unit="TFLOP/s", cores=nproc, kind="oracle",
                cpu=cpu_model(), dtype="f32", extrapolated=True,
                layer_seconds_extrapolated=round(layer_s, 1), sample_seconds=round(sample_s, 2),
                sample=(f"oracle in float32 on {nproc} host threads: head 0 of {w.name} -- zone statistics, shapes, "
                        f"permutation, pooling and selection of the whole head ({t_pre:.1f} s); attention forward"
                        f"{'' if fwd_only else ', dQ'} of {n_blocks} query blocks"
                        f"{'' if fwd_only else f' and dK/dV of {n_k} key blocks'}"
                        f"; extrapolated to the layer by selected token pairs and heads ({w.heads} heads)"))


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
    ap.add_argument("--a2v", choices=("rows", "fused"), default="rows",
                    help="rows: the statistics read the A2V cross-attention output (an input); fused: the step runs "
                         "the A2V cross-attention kernel, which also writes the per-token norm, and the statistics "
                         "read the norm map")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-microbench", action="store_true",
                    help="skip the measured ceilings (matrix-core peak and clock, forward tile gather, statistics read)")
    ap.add_argument("--stage-reps", type=int, default=3, help="cold-cache runs per stage for stage_ms")
    ap.add_argument("--cpu-blocks", type=int, default=160)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one elementwise pass y = -x over this many MiB after warm-up (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("SQA", "SQB", "L2", "LAT", "PAIRS"),
                    help="print the counter summary of four rocprofv3 --pmc runs of the benchmark")
    ap.add_argument("--summarize-profile", nargs="+", metavar="DIR",
                    help="print a text summary of rocprofv3 output directories and exit (no GPU): STATS_DIR "
                         "[FETCH_DIR WRITE_DIR]")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="command line recorded in the summary (repeatable)")
    args = ap.parse_args()
    if args.summarize_counters:
        d = args.summarize_counters
        summarize_counters(d[0], d[1], d[2], d[3], int(d[4]), args.profile_command)
        return
    if args.summarize_profile:
        dirs = list(args.summarize_profile) + [None, None]
        summarize_profile(dirs[0], dirs[1], dirs[2], args.profile_command)
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
