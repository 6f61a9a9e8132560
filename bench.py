#!/usr/bin/env python3
"""Benchmark of the CGTP convolution forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload si_mask]
                    [--configs c1_768,c2_768,highl_768,si_mask] [--dtype f32|f64]
                    [--pass fwd|bwd]

One step = one pass of the hot path over resident inputs: mask prepare (active CSR and
degree order), per-edge compaction and harmonics, and the fused convolution kernel(s).
The neighbour list is built once per workload (positions do not change between steps)
and timed separately.  Prints one JSON line.

The headline workload is the Si diamond supercell with the BranchIP mask (4096 atoms,
114 688 edges: the largest graph and the most bytes among the workloads with a
bandwidth target); the `configs` block repeats the same measurement for the other
768-atom workloads, each with its own roofline.

Timing is MALL-honest: the weights (and outputs) rotate over enough distinct buffers
(>= 768 MB in total) that the 256 MB last-level cache cannot hold them between the
steps that reuse them; the warm-cache time (one buffer) is reported as an extra field.
Three kinds of timed passes of K steps each: (A) nothing but the steps in the stream,
run PASSES_A times, the least of which gives ms_per_step and the throughput (all are
reported); (B) every step bracketed by its own events, which
gives the per-step p10 / p50 / p90; (C) the library stamps every fused convolution
launch with dispatch events on the same stream, which times the dominant kernel live
(the stamps add gaps around the launch, so they stay out of pass A).

Roofline: the algorithmic bytes and floating-point operations of a launch (each input
moved once; the A-form operation count: per active edge and path, the coupling
A = C . Y once, then mul (2 nnz(A) + 2 (2 l3 + 1)) for the channels) against the
published MI355X peaks, 8 TB/s of HBM and 157.3 TFLOP/s of FP32 vector arithmetic; the
bound is whichever of the two takes longer at peak.
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
FP32_PEAK_TFLOPS = 157.3            # FP32 vector, packed (dual-issue) rate
FP32_UNPACKED_TFLOPS = 78.6         # one FP32 FMA per lane and cycle (packed FP32 is not generated)
FP64_PEAK_TFLOPS = 78.6
ROTATE_BYTES = 768 << 20
KERNEL_SOURCES = ["conv_kernel.hpp", "cg_real.hpp", "common.hpp", "variants.hpp"]
HEADLINE = "si_mask"
CONFIGS = "c1_768,c2_768,highl_768,si_mask"
HOST_THREADS_CAP = 16               # CPU share of one GPU on the measurement hosts
# Timed passes of K steps behind ms_per_step (the least of them is reported, every one
# beside it): on the measurement boxes a whole pass of a few tens of milliseconds now and
# then runs up to 2.5 times slower than the passes around it (about one pass in three in
# some sessions), with the kernels and the host enqueue (about 20 us a step, a sixth of
# the GPU's time) unchanged.
PASSES_A = 5


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


def host_threads() -> int:
    return max(1, min(HOST_THREADS_CAP, len(os.sched_getaffinity(0))))


# ------------------------------------------------------------------------------------
# algorithmic bytes and operations of one forward launch
# ------------------------------------------------------------------------------------

def alg_bytes(plan, n, e, e_act, elem, masked, gated):
    """Each input moved once (b = bytes per floating-point element): the weights of the
    active edges (b W per active edge), the edge list (4 col + 3 shift, + 1 mask byte
    when masked, + b gate bytes when gated, per edge), the row pointers (4 (N + 1)), 3 b
    bytes of positions per node, and the node features in and the outputs out (b F_in
    and b F_out per node)."""
    return (elem * plan.w_per_edge * e_act
            + e * (4 + 3 + (1 if masked else 0) + (elem if gated else 0))
            + 4 * (n + 1) + 3 * elem * n + elem * plan.f_in * n + elem * plan.f_out * n)


def alg_flops_per_edge(plan) -> float:
    """A-form floating-point operations per active edge: per path, A = C . Y (2 nnz(C));
    per path and channel, A applied to x_j (2 nnz(A)) and the weight scaling of the
    2 l3 + 1 outputs; the harmonics (about 6 per SH component)."""
    import numpy as np
    total = 0.0
    for k, row in enumerate(plan.paths()):
        l3, mul = int(row[4]), int(row[6])
        cg = plan.cg(k)
        nnz_c = int(np.count_nonzero(cg))
        nnz_a = int(np.count_nonzero(np.any(cg != 0, axis=1)))
        total += 2 * nnz_c + mul * (2 * nnz_a + 2 * (2 * l3 + 1))
    return total + 6 * (plan.l_sh_max + 1) ** 2


def roofline(bytes_, flops, seconds, dtype="f32"):
    """Bound: whichever of HBM bytes and FP arithmetic takes longer at the peaks."""
    fp_peak = FP64_PEAK_TFLOPS if dtype == "f64" else FP32_PEAK_TFLOPS
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_fp = flops / (fp_peak * 1e12)
    gbs = bytes_ / seconds / 1e9
    tfs = flops / seconds / 1e12
    r = {"bytes": bytes_, "flops": flops, "achieved_gbs": gbs, "achieved_tflops": tfs,
         "hbm_frac": gbs / HBM_PEAK_GBS, "fp_frac": tfs / fp_peak}
    if t_fp > t_hbm:
        r.update({"bound": "fp64" if dtype == "f64" else "fp32", "achieved": tfs, "peak": fp_peak,
                  "unit": "TFLOP/s", "frac": tfs / fp_peak})
        if dtype != "f64":
            r["frac_of_unpacked_fp32"] = tfs / FP32_UNPACKED_TFLOPS
    else:
        r.update({"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS})
    return r


# ------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ------------------------------------------------------------------------------------

def _oracle_inputs(wl):
    import oracle as O
    import workloads as WL
    pos, box, cell, rng = WL.positions(wl)
    rp, col, sh = O.neighbors(pos, box, wl.cutoff)
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    gate = WL.gate_values(wl, rng, len(col))
    return plan, pos, cell, rp, col, sh, x, w, mask, gate


def _oracle_rows(O, plan, pos, cell, rp, col, sh, x, w, mask, gate, r0, r1):
    """oracle.conv_forward on receivers r0 .. r1 - 1 only: a sub-graph whose receivers
    come first (0 .. nb - 1) and whose senders keep their ids shifted by nb; a receiver's
    output depends only on its own incoming edges, so the rows equal the full graph's."""
    import numpy as np
    n = len(pos)
    e0, e1 = int(rp[r0]), int(rp[r1])
    nb = r1 - r0
    srp = np.concatenate([rp[r0:r1 + 1] - e0, np.full(n, e1 - e0)]).astype(np.int64)
    out = O.conv_forward(plan, np.concatenate([pos[r0:r1], pos]), cell, srp, col[e0:e1] + nb, sh[e0:e1],
                         np.concatenate([x[r0:r1], x]), w[e0:e1], None if mask is None else mask[e0:e1],
                         None if gate is None else gate[e0:e1])
    return out[:nb]


def cpu_baseline(wl, min_seconds: float):
    """The oracle (fp64 numpy, unmodified) over whole workloads: on the host's cores
    (threads over disjoint blocks of receiver rows; numpy releases the interpreter lock
    in its array loops) and single-threaded."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    plan, pos, cell, rp, col, sh, x, w, mask, gate = _oracle_inputs(wl)
    n, e = len(pos), len(col)
    threads = host_threads()
    cuts = np.searchsorted(rp, np.linspace(0, e, 4 * threads + 1)).clip(0, n)
    cuts[0], cuts[-1] = 0, n
    blocks = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    run = lambda blk: _oracle_rows(O, plan, pos, cell, rp, col, sh, x, w, mask, gate, *blk)
    reps, spent = 0, 0.0
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        while reps == 0 or (spent < min_seconds / 2 and reps < 10):
            t0 = time.perf_counter()
            list(ex.map(run, blocks))
            spent += time.perf_counter() - t0
            reps += 1
    multi = e * reps / spent
    reps1, spent1 = 0, 0.0
    with threadpool_limits(1):
        while reps1 == 0 or (spent1 < min_seconds / 2 and reps1 < 10):
            t0 = time.perf_counter()
            O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask, gate)
            spent1 += time.perf_counter() - t0
            reps1 += 1
    return {"value": multi, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"whole {wl.name} workload ({e} edges), {reps} run(s) in {spent:.1f} s on {threads} "
                      f"threads ({len(blocks)} blocks of receiver rows), numpy fp64, unmodified oracle",
            "single_thread": {"value": e * reps1 / spent1, "unit": "edges/s", "cores": 1,
                              "sample": f"whole workload, {reps1} run(s) in {spent1:.1f} s, one thread"}}


# ------------------------------------------------------------------------------------
# the GPU measurement of one workload
# ------------------------------------------------------------------------------------

def _pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def timed_passes(step, first, K, passes=None):
    """PASSES_A timed passes of K steps each (step indices from `first` on), each
    bracketed by synchronisations and timed by a pair of events around the K steps;
    returns the milliseconds per step of each pass."""
    import torch
    out = []
    for p in range(passes or PASSES_A):
        torch.cuda.synchronize()
        b, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        for s in range(K):
            step(first + p * K + s)
        t.record()
        torch.cuda.synchronize()
        out.append(b.elapsed_time(t) / K)
    return out


def measure_forward(C, wl, dev, K, W, f64=False, warm_cache=True):
    """Passes A, B and C (module docstring) over one workload; returns a dict."""
    import numpy as np
    import torch

    import workloads as WL

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
    k = min(64, max(3, math.ceil(ROTATE_BYTES / max(w.nbytes, 1))))
    w0 = torch.from_numpy(w).to(dev)
    del w
    wbufs = [w0] + [w0.clone() for _ in range(k - 1)]
    outs = [torch.empty((n, plan.f_out), dtype=plan.dtype, device=dev) for _ in range(k)]
    ws = torch.empty(plan.workspace_size(n, e, mask is not None), dtype=torch.uint8, device=dev)

    def step(s, evs=None):
        C.conv_forward(plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs[s % k], mask_d, out=outs[s % k],
                       workspace=ws, conv_events=evs, gate=gate_d)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    ev_b, ev_e = [ev() for _ in range(K)], [ev() for _ in range(K)]
    st_b, st_e = [ev() for _ in range(K)], [ev() for _ in range(K)]
    for x_ in ev_b + ev_e + st_b + st_e:
        x_.record()                       # materialise the HIP events
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    # A: throughput, K whole steps with nothing else in the stream, PASSES_A times
    passes = timed_passes(step, W, K)
    ms_step = min(passes)
    # B: per-step distribution
    for s in range(K):
        st_b[s].record()
        step(W + PASSES_A * K + s)
        st_e[s].record()
    torch.cuda.synchronize()
    steps_ms = [st_b[s].elapsed_time(st_e[s]) for s in range(K)]
    # C: the convolution launches, stamped by dispatch events
    for s in range(K):
        step(W + (PASSES_A + 1) * K + s, (ev_b[s], ev_e[s]))
    torch.cuda.synchronize()
    conv = [ev_b[s].elapsed_time(ev_e[s]) for s in range(K)]
    conv_ms = float(np.mean(conv))
    ms_warm = None
    if warm_cache:   # one weight buffer reused every step
        ms_warm = min(timed_passes(lambda s: C.conv_forward(plan, pos_d, cell, row_ptr, col, shift, x_d, wbufs[0],
                                                            mask_d, out=outs[0], workspace=ws, gate=gate_d),
                                   0, K, passes=2))
    nbytes = alg_bytes(plan, n, e, e_act, elem, mask is not None, gate is not None)
    flops = alg_flops_per_edge(plan) * e_act
    res = {
        "plan": plan, "n": n, "e": e, "e_act": e_act, "k": k,
        "ms_per_step": ms_step, "ms_per_step_passes": passes,
        "ms_per_step_p10": _pct(steps_ms, 10), "ms_per_step_p50": _pct(steps_ms, 50),
        "ms_per_step_p90": _pct(steps_ms, 90),
        "conv_ms": conv_ms, "conv_ms_p10": _pct(conv, 10), "conv_ms_p50": _pct(conv, 50),
        "conv_ms_p90": _pct(conv, 90),
        "warm_ms": ms_warm, "nbr_ms": 1e3 * float(np.median(t_nbr)),
        "roofline": roofline(nbytes, flops, conv_ms * 1e-3, "f64" if f64 else "f32"),
        "step_roofline": roofline(nbytes, flops, ms_step * 1e-3, "f64" if f64 else "f32"),
    }
    del wbufs, outs, ws, w0
    torch.cuda.empty_cache()
    return res


def copy_bandwidth(dev, mib=1024, reps=10):
    """Achievable HBM bandwidth of a plain device copy (read + write bytes per second)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    b, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    for _ in range(reps):
        dst.copy_(src)
    t.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (b.elapsed_time(t) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_per_copy": 2 * n, "copies": reps, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--configs", default=CONFIGS,
                    help="comma-separated workloads measured in the extra configs block ('' for none)")
    ap.add_argument("--dtype", choices=["f32", "f64"], default="f32",
                    help="arithmetic type of the forward (f64: plans with l <= 4)")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="bwd: time the backward step (x, w and position gradients; fp32, l <= 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-warm-cache", action="store_true",
                    help="skip the warm-cache timing pass (profiling runs: every conv launch then "
                         "uses a rotated weight buffer)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB --steps times "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--gather-calibrate", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, gather every 5248-byte row of a MIB MiB table "
                         "once, in a random order, --steps times (checks that the copy's counter "
                         "scale holds for row gathers like the weight stream's)")
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

    if a.gather_calibrate:
        row = 1312   # floats per row: one si_mask edge's weights
        rows = (a.gather_calibrate << 20) // (4 * row)
        src = torch.ones((rows, row), dtype=torch.float32, device="cuda:0")
        idx = torch.from_numpy(np.random.default_rng(0).permutation(rows)).to("cuda:0")
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            torch.index_select(src, 0, idx, out=dst)
        torch.cuda.synchronize()
        n = rows * row * 4
        print(json.dumps({"gather_calibration_bytes": n, "gathers": a.steps, "read_bytes_per_gather": n,
                          "write_bytes_per_gather": n}), flush=True)
        return 0

    import clebsch_gordan_tensor_node_amd as C
    import workloads as WL

    wl = WL.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.which == "bwd":
        return bench_backward(a, C, wl, dev)

    K, W = a.steps, a.warmup
    f64 = a.dtype == "f64"
    r = measure_forward(C, wl, dev, K, W, f64=f64, warm_cache=not a.no_warm_cache)
    plan, n, e, e_act = r["plan"], r["n"], r["e"], r["e_act"]
    rl = dict(r["roofline"])
    rl.update({"traffic": read_traffic(wl.name, a.dtype), "kernel": "conv_kernel (fused CGTP conv)",
               "kernel_ms": r["conv_ms"], "kernel_ms_p10": r["conv_ms_p10"], "kernel_ms_p50": r["conv_ms_p50"],
               "kernel_ms_p90": r["conv_ms_p90"], "alg_bytes_per_launch": rl["bytes"],
               "alg_flops_per_launch": rl["flops"]})
    out = {
        "metric": METRIC,
        "value": e / (r["ms_per_step"] * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n_atoms": n, "n_edges": e, "n_active_edges": e_act,
                   "edges_counted": "every edge of the receiver CSR, masked ones included (active edges/s "
                                    "is reported beside it)",
                   "cutoff": wl.cutoff, "irreps_in": wl.irreps_in, "irreps_sh": wl.irreps_sh,
                   "irreps_out": plan.irreps_out, "paths": plan.n_paths, "masked": wl.masked, "gated": wl.gated,
                   "description": wl.description},
        "roofline": rl,
        "ms_per_step_passes": r["ms_per_step_passes"],
        "ms_per_step_p10": r["ms_per_step_p10"],
        "ms_per_step_p50": r["ms_per_step_p50"],
        "ms_per_step_p90": r["ms_per_step_p90"],
        "step_roofline_frac": r["step_roofline"]["frac"],
        "node_updates_per_s": n / (r["ms_per_step"] * 1e-3),
        "active_edges_per_s": e_act / (r["ms_per_step"] * 1e-3),
        "warm_cache_ms_per_step": r["warm_ms"],
        "rotation_buffers": r["k"],
        "nbr_build_ms": r["nbr_ms"],
        "jobs_variants": list(plan.schedule()),
    }
    del r, plan
    out["hbm_copy"] = copy_bandwidth(dev)
    cfgs = {}
    for name in [c for c in a.configs.split(",") if c]:
        if name == wl.name:
            rc = {"same_as_headline": True}
        else:
            q = measure_forward(C, WL.WORKLOADS[name], dev, K, W, f64=f64, warm_cache=False)
            rc = {"ms_per_step": q["ms_per_step"], "ms_per_step_passes": q["ms_per_step_passes"],
                  "ms_per_step_p10": q["ms_per_step_p10"],
                  "ms_per_step_p90": q["ms_per_step_p90"], "edges_per_s": q["e"] / (q["ms_per_step"] * 1e-3),
                  "active_edges_per_s": q["e_act"] / (q["ms_per_step"] * 1e-3),
                  "node_updates_per_s": q["n"] / (q["ms_per_step"] * 1e-3),
                  "n_edges": q["e"], "n_active_edges": q["e_act"], "conv_ms": q["conv_ms"],
                  "conv_ms_p10": q["conv_ms_p10"], "conv_ms_p90": q["conv_ms_p90"],
                  "roofline": {k_: q["roofline"][k_] for k_ in ("bound", "achieved", "peak", "unit", "frac",
                                                                "hbm_frac", "fp_frac", "bytes", "flops")},
                  "traffic": read_traffic(name, a.dtype)}
            if "frac_of_unpacked_fp32" in q["roofline"]:
                rc["roofline"]["frac_of_unpacked_fp32"] = q["roofline"]["frac_of_unpacked_fp32"]
            del q
        cfgs[name] = rc
    out["configs"] = cfgs
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def bench_backward(a, C, wl, dev):
    """K backward steps (x, w and position gradients) over rotated weight and gradient
    buffers; the roofline is taken over the whole step (every backward kernel)."""
    import ctypes

    import numpy as np
    import torch

    import workloads as WL

    pos, box, cell, rng = WL.positions(wl)
    pos_d = torch.from_numpy(pos).to(dev)
    t_nbr = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        row_ptr, col, shift = C.neighbors_build(pos_d, box, wl.cutoff)
        t_nbr.append(time.perf_counter() - t0)
    n, e = wl.n_atoms, int(col.shape[0])
    plan = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, n, plan.f_in, e, plan.w_per_edge)
    gate = WL.gate_values(wl, rng, e)
    active = np.ones(e, dtype=bool)
    if mask is not None:
        active &= mask != 0
    if gate is not None:
        active &= gate != 0
    e_act = int(active.sum())
    x_d = torch.from_numpy(x).to(dev)
    mask_d = torch.from_numpy(mask).to(dev) if mask is not None else None
    gate_d = torch.from_numpy(gate).to(dev) if gate is not None else None
    k = min(64, max(3, math.ceil(ROTATE_BYTES / max(w.nbytes, 1))))
    w0 = torch.from_numpy(w).to(dev)
    wbufs = [w0] + [w0.clone() for _ in range(k - 1)]
    g0 = torch.from_numpy(np.random.default_rng(1234).standard_normal((n, plan.f_out)).astype(np.float32)).to(dev)
    gouts = [g0] + [g0.clone() for _ in range(k - 1)]
    gws = [torch.empty_like(wbufs[0]) for _ in range(k)]
    gx = torch.empty((n, plan.f_in), dtype=torch.float32, device=dev)
    gp = torch.empty((n, 3), dtype=torch.float32, device=dev)
    ws = torch.empty(plan.backward_workspace_size(n, e), dtype=torch.uint8, device=dev)
    lib = C._lib.load()
    cella = None if cell is None else np.ascontiguousarray(np.asarray(cell, dtype=np.float32).reshape(-1))
    cellp = None if cella is None else cella.ctypes.data_as(C._lib.FP)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())

    def step(s):
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        C.check(lib.cgtp_conv_backward(plan.handle, P(pos_d), n, cellp, P(row_ptr), P(col), P(shift), e,
                                       P(x_d), P(wbufs[s % k]), P(mask_d), P(gate_d), P(gouts[s % k]), P(gx),
                                       P(gws[s % k]), P(gp), P(ws), ws.numel(), stream))

    K, W = a.steps, a.warmup
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    passes = timed_passes(step, W, K)
    ms_step = min(passes)
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
        "ms_per_step_passes": passes,
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

    plan, pos, cell, rp, col, sh, x, w, mask, gate = _oracle_inputs(wl)
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
