#!/usr/bin/env python3
"""Benchmark of the CGTP convolution forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c1_768] [--dtype f32|f64]
                    [--pass fwd|bwd]

One step = one pass of the hot path over resident inputs: mask prepare (active CSR and
degree order), per-edge compaction and harmonics, and the fused convolution kernel(s).
The neighbour list is built once per workload (positions do not change between steps)
and timed separately.  Prints one JSON line.

Timing is MALL-honest: the weights (and outputs) rotate over enough distinct buffers
(>= 768 MB in total) that the 256 MB last-level cache cannot hold them between the
steps that reuse them; the warm-cache time (one buffer) is reported as an extra field.
Two timed passes of K steps each: the first, with nothing but the steps in the stream,
gives ms_per_step and the throughput; in the second the library stamps every fused
convolution launch with dispatch events on the same stream, which times the dominant
kernel live (the stamps add gaps around the launch, so they stay out of the first pass).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CGTP conv fwd edges/sec on 1 MI355X; % of HBM/FP32 roofline"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 768 << 20
KERNEL_SOURCES = ["conv_kernel.hpp", "cg_real.hpp", "common.hpp", "variants.hpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "clebsch_gordan_tensor_node_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, dtype: str = "f32"):
    """HBM bytes per conv launch from the committed counter summary, if it was taken on
    the current kernel sources (else None)."""
    tag = workload if dtype == "f32" else f"{workload}_{dtype}"
    path = os.path.join(ROOT, "profiles", f"conv_kernel_{tag}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, min_seconds: float):
    """The oracle as it stands, on this host, single-threaded, over whole workloads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    import workloads as WL

    pos, box, cell, rng = WL.positions(wl)
    rp, col, sh = O.neighbors(pos, box, wl.cutoff)
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    gate = WL.gate_values(wl, rng, len(col))
    reps, spent = 0, 0.0
    with threadpool_limits(1):
        while reps == 0 or (spent < min_seconds and reps < 20):
            t0 = time.perf_counter()
            O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask, gate)
            spent += time.perf_counter() - t0
            reps += 1
    return {"value": len(col) * reps / spent, "unit": "edges/s", "cores": 1, "kind": "oracle",
            "sample": f"whole {wl.name} workload ({len(col)} edges), {reps} run(s), {spent:.1f} s, "
                      f"numpy fp64, BLAS limited to 1 thread"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c1_768")
    ap.add_argument("--dtype", choices=["f32", "f64"], default="f32",
                    help="arithmetic type of the forward (f64: plans with l <= 3)")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="bwd: time the backward step (x, w and position gradients; fp32, l <= 3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-warm-cache", action="store_true",
                    help="skip the warm-cache timing pass (profiling runs: every conv launch then "
                         "uses a rotated weight buffer)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB --steps times "
                         "(the reference kernel for scaling HBM byte counters)")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "sharding by receiver rows over several GPUs is not built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if a.copy_calibrate:
        n = a.copy_calibrate << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": a.steps,
                          "read_bytes_per_copy": n, "write_bytes_per_copy": n}), flush=True)
        return 0

    import clebsch_gordan_tensor_node_amd as C
    import workloads as WL

    wl = WL.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pos, box, cell, rng = WL.positions(wl)
    pos_d = torch.from_numpy(pos).to(dev)

    # neighbour list on the GPU (timed apart: it synchronises to return E)
    C.neighbors_build(pos_d, box, wl.cutoff)
    t_nbr = []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        row_ptr, col, shift = C.neighbors_build(pos_d, box, wl.cutoff)
        t_nbr.append(time.perf_counter() - t0)
    n, e = wl.n_atoms, int(col.shape[0])

    f64 = a.dtype == "f64"
    elem = 8 if f64 else 4
    plan = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, fp64=f64)
    x, w, mask = WL.draw_payload(wl, rng, n, plan.f_in, e, plan.w_per_edge)
    gate = WL.gate_values(wl, rng, e)
    if f64:   # the same draws, exact in fp64
        x, w = x.astype(np.float64), w.astype(np.float64)
        gate = None if gate is None else gate.astype(np.float64)
        pos_d = pos_d.double()
        cell = None if cell is None else np.asarray(cell, dtype=np.float64)
    active = np.ones(e, dtype=bool)
    if mask is not None:
        active &= mask != 0
    if gate is not None:
        active &= gate != 0
    e_act = int(active.sum())
    gate_d = torch.from_numpy(gate).to(dev) if gate is not None else None
    x_d = torch.from_numpy(x).to(dev)
    mask_d = torch.from_numpy(mask).to(dev) if mask is not None else None
    w_bytes = w.nbytes
    k = min(64, max(3, math.ceil(ROTATE_BYTES / max(w_bytes, 1))))
    w0 = torch.from_numpy(w).to(dev)
    wbufs = [w0] + [w0.clone() for _ in range(k - 1)]
    outs = [torch.empty((n, plan.f_out), dtype=plan.dtype, device=dev) for _ in range(k)]
    ws = torch.empty(plan.workspace_size(n, e, mask is not None), dtype=torch.uint8, device=dev)
    if a.which == "bwd":
        return bench_backward(a, C, wl, plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs, mask_d, gate_d,
                              n, e, e_act, k, t_nbr)

    def step(s, evs=None):
        C.conv_forward(plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs[s % k], mask_d, out=outs[s % k],
                       workspace=ws, conv_events=evs, gate=gate_d)

    K, W = a.steps, a.warmup
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for ev in ev_b + ev_e:
        ev.record()                       # materialise the HIP events
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    # throughput: K whole steps with nothing else in the stream
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_beg.record()
    for s in range(K):
        step(W + s)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_beg.elapsed_time(t_end) / K
    # kernel duration: K more steps whose conv launches are stamped by dispatch events
    # (the stamps themselves add gaps around the launch, so they stay out of the
    # throughput pass)
    t_beg.record()
    for s in range(K):
        step(W + K + s, (ev_b[s], ev_e[s]))
    t_end.record()
    torch.cuda.synchronize()
    ms_step_stamped = t_beg.elapsed_time(t_end) / K
    conv_ms = float(np.mean([ev_b[s].elapsed_time(ev_e[s]) for s in range(K)]))

    # warm-cache figure: one weight buffer reused every step
    ms_warm = None
    if not a.no_warm_cache:
        torch.cuda.synchronize()
        t_beg.record()
        for s in range(K):
            C.conv_forward(plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs[0], mask_d, out=outs[0],
                           workspace=ws, gate=gate_d)
        t_end.record()
        torch.cuda.synchronize()
        ms_warm = t_beg.elapsed_time(t_end) / K

    # algorithmic bytes of the hot path, each moved once (b = 4 bytes per element in
    # fp32, 8 in fp64): the weights of the active edges (b W per active edge), the edge
    # list (4 col + 3 shift, + 1 mask byte when masked, + b gate bytes when gated, per
    # edge), the row pointers (4 (N + 1)), 3 b bytes of positions per node, and the node
    # features in and the outputs out (b F_in and b F_out per node)
    conv_bytes = (elem * plan.w_per_edge * e_act
                  + e * (4 + 3 + (1 if mask is not None else 0) + (elem if gate is not None else 0))
                  + 4 * (n + 1) + 3 * elem * n + elem * plan.f_in * n + elem * plan.f_out * n)
    achieved = conv_bytes / (conv_ms * 1e-3) / 1e9
    traffic = read_traffic(wl.name, a.dtype)

    out = {
        "metric": METRIC,
        "value": e / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n_atoms": n, "n_edges": e, "n_active_edges": e_act,
                   "cutoff": wl.cutoff, "irreps_in": wl.irreps_in, "irreps_sh": wl.irreps_sh,
                   "irreps_out": plan.irreps_out, "paths": plan.n_paths, "masked": wl.masked, "gated": wl.gated,
                   "description": wl.description},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "conv_kernel (fused CGTP conv)", "kernel_ms": conv_ms,
                     "alg_bytes_per_launch": conv_bytes},
        "node_updates_per_s": n / (ms_step * 1e-3),
        "active_edges_per_s": e_act / (ms_step * 1e-3),
        "ms_per_step_stamped_pass": ms_step_stamped,
        "warm_cache_ms_per_step": ms_warm,
        "rotation_buffers": k,
        "nbr_build_ms": 1e3 * float(np.median(t_nbr)),
        "jobs_variants": list(plan.schedule()),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def bench_backward(a, C, wl, plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs, mask_d, gate_d, n, e, e_act, k,
                   t_nbr):
    """K backward steps (x, w and position gradients) over rotated weight and gradient
    buffers; the roofline is taken over the whole step (every backward kernel)."""
    import numpy as np
    import torch

    dev = pos_d.device
    rng = np.random.default_rng(1234)
    g0 = torch.from_numpy(rng.standard_normal((n, plan.f_out)).astype(np.float32)).to(dev)
    gouts = [g0] + [g0.clone() for _ in range(k - 1)]
    gws = [torch.empty_like(wbufs[0]) for _ in range(k)]
    gx = torch.empty((n, plan.f_in), dtype=torch.float32, device=dev)
    gp = torch.empty((n, 3), dtype=torch.float32, device=dev)
    ws = torch.empty(plan.backward_workspace_size(n, e), dtype=torch.uint8, device=dev)
    lib = C._lib.load()
    cella = None if cell is None else np.ascontiguousarray(np.asarray(cell, dtype=np.float32).reshape(-1))
    cellp = None if cella is None else cella.ctypes.data_as(C._lib.FP)
    P = lambda t: None if t is None else __import__("ctypes").c_void_p(t.data_ptr())

    def step(s):
        stream = __import__("ctypes").c_void_p(torch.cuda.current_stream().cuda_stream)
        C.check(lib.cgtp_conv_backward(plan.handle, P(pos_d), n, cellp, P(row_ptr), P(col), P(shift), e,
                                       P(x_d), P(wbufs[s % k]), P(mask_d), P(gate_d), P(gouts[s % k]), P(gx),
                                       P(gws[s % k]), P(gp), P(ws), ws.numel(), stream))

    K, W = a.steps, a.warmup
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_beg.record()
    for s in range(K):
        step(W + s)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_beg.elapsed_time(t_end) / K
    # algorithmic bytes of the backward, each moved once: w of the active edges and the
    # w-gradient of every edge (4 W each), the edge list (as the forward), x and
    # grad_x (4 F_in per node each), grad_out (4 F_out per node), positions and their
    # gradient (12 + 12 per node), row pointers
    bwd_bytes = (4 * plan.w_per_edge * e_act + 4 * plan.w_per_edge * e
                 + e * (4 + 3 + (1 if mask_d is not None else 0) + (4 if gate_d is not None else 0))
                 + 4 * (n + 1) + 24 * n + 8 * plan.f_in * n + 4 * plan.f_out * n)
    achieved = bwd_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "CGTP conv backward edges/sec on 1 MI355X; % of HBM roofline",
        "value": e / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "pass": "backward (grad_x, grad_w, grad_pos)", "n_atoms": n,
                   "n_edges": e, "n_active_edges": e_act, "irreps_in": wl.irreps_in, "irreps_sh": wl.irreps_sh,
                   "paths": plan.n_paths, "masked": wl.masked, "gated": wl.gated},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "backward step (every backward kernel, per-kernel times in profiles/)",
                     "kernel_ms": ms_step, "alg_bytes_per_launch": bwd_bytes},
        "rotation_buffers": k,
        "nbr_build_ms": 1e3 * float(np.median(t_nbr)),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(wl, a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_backward(wl, min_seconds: float):
    """The oracle's conv_backward as it stands, single-threaded, over whole workloads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    import workloads as WL

    pos, box, cell, rng = WL.positions(wl)
    rp, col, sh = O.neighbors(pos, box, wl.cutoff)
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    gate = WL.gate_values(wl, rng, len(col))
    gout = np.random.default_rng(1234).standard_normal((wl.n_atoms, plan.f_out))
    reps, spent = 0, 0.0
    with threadpool_limits(1):
        while reps == 0 or (spent < min_seconds and reps < 10):
            t0 = time.perf_counter()
            O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout, mask, gate)
            spent += time.perf_counter() - t0
            reps += 1
    return {"value": len(col) * reps / spent, "unit": "edges/s", "cores": 1, "kind": "oracle",
            "sample": f"whole {wl.name} workload ({len(col)} edges), {reps} run(s), {spent:.1f} s, "
                      f"numpy fp64 conv_backward, BLAS limited to 1 thread"}


if __name__ == "__main__":
    sys.exit(main())
