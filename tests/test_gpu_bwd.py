"""GPU parity of the backward (cgtp_conv_backward: x, w and position gradients) against
the fp64 oracle's conv_backward, through the C ABI.

Bars (fp32 arithmetic, as the forward): relative L2 <= 1e-5 for every gradient, max
|diff| <= 1e-4 for grad_x and grad_w; grad_pos, whose per-node values are sums of
+/- edge terms that largely cancel (their sum over all nodes is exactly zero), is held
to max |diff| <= 1e-4 * max |grad_pos| and its sum over nodes to 1e-4 * max |grad_pos|.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

C = pytest.importorskip("clebsch_gordan_tensor_node_amd")

pytestmark = pytest.mark.gpu

REL_L2 = 1e-5
MAX_ABS = 1e-4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def _t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _rel(got, ref):
    nref = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got - ref)


def _check(got, ref, what, whole=True):
    gx, gw, gp = (np.asarray(g, dtype=np.float64) for g in got)
    rx, rw, rp = ref
    for g in (gx, gw, gp):
        assert np.all(np.isfinite(g)), what
    ex, ew, ep = _rel(gx, rx), _rel(gw, rw), _rel(gp, rp)
    mx, mw = np.abs(gx - rx).max(initial=0), np.abs(gw - rw).max(initial=0)
    scale = max(np.abs(rp).max(initial=0), 1e-30)
    mp = np.abs(gp - rp).max(initial=0) / scale
    drift = np.abs(gp.sum(axis=0)).max(initial=0) / scale
    print(f"{what}: x rel {ex:.2e} max {mx:.2e} | w rel {ew:.2e} max {mw:.2e} | "
          f"pos rel {ep:.2e} max/scale {mp:.2e} sum/scale {drift:.2e}", flush=True)
    assert ex <= REL_L2 and mx <= MAX_ABS, (what, "x", ex, mx)
    assert ew <= REL_L2 and mw <= MAX_ABS, (what, "w", ew, mw)
    assert ep <= REL_L2 and mp <= 1e-4, (what, "pos", ep, mp)
    if whole:   # over all nodes the position gradient sums to zero
        assert drift <= 1e-4, (what, "pos sum", drift)


_CACHE = {}


def _workload(name):
    if name in _CACHE:
        return _CACHE[name]
    wl = WL.WORKLOADS[name]
    pos, box, cell, rng = WL.positions(wl)
    rp, col, sh = O.neighbors(pos, box, wl.cutoff)
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    gate = WL.gate_values(wl, rng, len(col))
    gout = np.random.default_rng(1234).standard_normal((wl.n_atoms, plan.f_out)).astype(np.float32)
    _CACHE[name] = (wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout)
    return _CACHE[name]


def _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout, mask=None, gate=None):
    gx, gw, gp = C.conv_backward(p, _t(pos, dev), cell, _t(rp, dev), _t(col, dev), _t(sh, dev), _t(x, dev),
                                 _t(w, dev), _t(gout, dev), None if mask is None else _t(mask, dev),
                                 None if gate is None else _t(gate, dev))
    torch.cuda.synchronize()
    return gx.cpu().numpy(), gw.cpu().numpy(), gp.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "c1_768", "c2_768", "si_mask", "si_gate"])
def test_backward_workloads(dev, name):
    wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout = _workload(name)
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    got = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout, mask, gate)
    ref = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout, mask, gate)
    _check(got, ref, name)


@pytest.mark.parametrize("name", ["c5_768", "c6_768"])
def test_backward_full_size_sampled(dev, name):
    """LunaTP Table 1 cases 5 and 6 (L = 4) at full size on the GPU.  The oracle takes the
    edges incident to 12 sampled nodes: the w-gradient of an edge depends on that edge
    alone, and a node's x- and position gradients on the edges it sends or receives, so
    on those edges and nodes the sub-graph's gradients are the full graph's."""
    wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout = _workload(name)
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    gx, gw, gp = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout)
    n = len(pos)
    nodes = np.random.default_rng(5).choice(n, 12, replace=False)
    recv = np.repeat(np.arange(n), np.diff(rp))
    keep = np.isin(recv, nodes) | np.isin(col, nodes)
    eids = np.flatnonzero(keep)
    rp_sub = np.concatenate([[0], np.cumsum(np.bincount(recv[eids], minlength=n))]).astype(np.int32)
    rx, rw, rpos = O.conv_backward(plan, pos, cell, rp_sub, col[eids], sh[eids], x, w[eids], gout)
    got = (gx[nodes], gw[eids], gp[nodes])
    _check(got, (rx[nodes], rw, rpos[nodes]), f"{name}[{len(nodes)} nodes, {len(eids)} edges]", whole=False)


def _small_system(n, box_len, cutoff, seed):
    rng = np.random.default_rng(seed)
    pos = (rng.random((n, 3)) * box_len).astype(np.float32)
    pos[pos >= np.float32(box_len)] = 0
    box = np.full(3, box_len, dtype=np.float32)
    cell = np.diag(box).astype(np.float32)
    rp, col, sh = O.neighbors(pos, box, cutoff)
    return rng, pos, cell, rp, col, sh


@pytest.mark.parametrize("l1", range(5))
@pytest.mark.parametrize("mul", [3, 70])
def test_backward_every_path(dev, l1, mul):
    """Every (l1, l2, l3) with l <= 4; 70 channels = two 64-lane chunks, the second ragged."""
    rng, pos, cell, rp, col, sh = _small_system(36, 6.0, 2.7, 300 + l1)
    for l2 in range(5):
        spec_in, spec_sh = f"{mul}x{l1}e", f"1x{l2}e"
        plan = O.build_plan(spec_in, spec_sh, 4, O.PATHS_ALL)
        x = rng.standard_normal((len(pos), plan.f_in)).astype(np.float32)
        w = rng.standard_normal((len(col), plan.w_per_edge)).astype(np.float32)
        gout = rng.standard_normal((len(pos), plan.f_out)).astype(np.float32)
        p = C.Plan(spec_in, spec_sh, 4, "all")
        got = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout)
        ref = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout)
        _check(got, ref, f"{spec_in} x {spec_sh}")


def test_backward_several_irreps_one_l(dev):
    # two input irreps of the same l (two x-gradient blocks of one wave shape) and paths
    # dropped by the parity rule
    rng, pos, cell, rp, col, sh = _small_system(30, 5.5, 2.6, 77)
    spec_in, spec_sh = "5x1o+7x1e+4x0e+3x2o", "1x0e+1x1o+1x2e+1x3o"
    plan = O.build_plan(spec_in, spec_sh, 3, O.PATHS_PARITY)
    x = rng.standard_normal((len(pos), plan.f_in)).astype(np.float32)
    w = rng.standard_normal((len(col), plan.w_per_edge)).astype(np.float32)
    gout = rng.standard_normal((len(pos), plan.f_out)).astype(np.float32)
    mask = (rng.random(len(col)) < 0.7).astype(np.uint8)
    p = C.Plan(spec_in, spec_sh, 3, "parity")
    got = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout, mask)
    _check(got, O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout, mask), "mixed irreps, masked")


def test_backward_l4_whole_irrep_waves(dev):
    """A plan reaching l = 4 on a graph large enough (senders times input irreps >= 4096)
    that the x-gradient runs one wave per (sender, input irrep), the l = 4 paths in their
    own launch; 70 channels at l = 4 make two chunks, the second ragged."""
    rng, pos, cell, rp, col, sh = _small_system(840, (840 / 0.05) ** (1 / 3), 3.2, 91)
    spec_in, spec_sh = "16x0e+8x1o+8x2e+4x3o+70x4e", "1x0e+1x1o+1x2e+1x3o+1x4e"
    plan = O.build_plan(spec_in, spec_sh, 4, O.PATHS_PARITY)
    assert len(pos) * len(plan.irreps_in) >= 4096
    x = rng.standard_normal((len(pos), plan.f_in)).astype(np.float32)
    w = rng.standard_normal((len(col), plan.w_per_edge)).astype(np.float32)
    gout = rng.standard_normal((len(pos), plan.f_out)).astype(np.float32)
    mask = (rng.random(len(col)) < 0.8).astype(np.uint8)
    p = C.Plan(spec_in, spec_sh, 4, "parity")
    got = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout, mask)
    _check(got, O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout, mask), "l = 4, whole-irrep waves")


def test_backward_deterministic_and_nan_safe(dev):
    wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout = _workload("si_mask")
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    w_nan = w.copy()
    w_nan[mask == 0] = np.nan
    a = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w_nan, gout, mask)
    b = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w_nan, gout, mask)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)             # bitwise run to run
        assert np.all(np.isfinite(u))           # NaN in inactive weights never read
    assert np.all(a[1][mask == 0] == 0.0)       # inactive edges: zero w-gradient rows


def test_backward_subsets_and_empty(dev):
    wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout = _workload("tiny")
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    full = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout)
    for need in [("x",), ("w",), ("pos",), ("x", "pos")]:
        got = C.conv_backward(p, _t(pos, dev), cell, _t(rp, dev), _t(col, dev), _t(sh, dev), _t(x, dev),
                              _t(w, dev), _t(gout, dev), need=need)
        for k, name in enumerate(("x", "w", "pos")):
            if name in need:
                assert np.array_equal(got[k].cpu().numpy(), full[k])
            else:
                assert got[k] is None
    # no active edge: every gradient is zero
    zero = np.zeros(len(col), dtype=np.uint8)
    gx, gw, gp = _gpu_bwd(dev, p, pos, cell, rp, col, sh, x, w, gout, zero)
    assert not gx.any() and not gw.any() and not gp.any()


def test_backward_refusals(dev):
    lib = C._lib.load()
    wl, plan, pos, cell, rp, col, sh, x, w, mask, gate, gout = _workload("tiny")
    n, e = len(pos), len(col)
    d = lambda a: ctypes.c_void_p(a.data_ptr())
    tens = [_t(a, dev) for a in (pos, rp, col, x, w, gout)]
    pos_d, rp_d, col_d, x_d, w_d, g_d = tens
    out = torch.empty(n * 3, dtype=torch.float32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for plan_args, code in [((wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, False, True), -1),
                            (("8x0e+8x5e", "1x0e+1x1o", 5, "all"), -3)]:
        p = C.Plan(*plan_args)
        ws = torch.empty(p.backward_workspace_size(n, e), dtype=torch.uint8, device=dev)
        rc = lib.cgtp_conv_backward(p.handle, d(pos_d), n, None, d(rp_d), d(col_d), None, e, d(x_d), d(w_d), None,
                                    None, d(g_d), None, None, d(out), d(ws), ws.numel(), s)
        assert rc == code, (plan_args, rc, lib.cgtp_last_error())
