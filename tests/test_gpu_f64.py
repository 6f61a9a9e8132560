"""GPU parity of the fp64 forward (plans made with fp64=True) against the fp64 oracle.

LunaTP measures its kernels in double precision (Figure 8, Table 11).  Here geometry,
harmonics, CG coefficients and accumulation are all fp64 on both sides, so the two
differ only by rounding order.  Bar: relative L2 <= 1e-12 and max |diff| <= 1e-10.
Each output sums about deg * nnz(C) <= 40 * 400 products whose magnitudes are O(10);
a worst-case accumulation bound is 16000 * 1.1e-16 * O(10) ~ 2e-11 absolute, and the
typical (random-sign) error is orders of magnitude smaller.  The fp32-drawn inputs are
exact in fp64, so both sides see the same numbers.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

C = pytest.importorskip("clebsch_gordan_tensor_node_amd")

pytestmark = pytest.mark.gpu

REL_L2 = 1e-12
MAX_ABS = 1e-10


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def _t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _compare(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), what
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mx = np.abs(diff).max() if diff.size else 0.0
    print(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)


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
    _CACHE[name] = (wl, plan, pos, box, cell, rp, col, sh, x, w, mask, gate)
    return _CACHE[name]


def _gpu_conv64(dev, spec, pos, cell, rp, col, sh, x, w, mask=None, gate=None, plan=None):
    p = plan or C.Plan(*spec, fp64=True)
    f64 = lambda a: _t(np.asarray(a, dtype=np.float64), dev)
    out = C.conv_forward(p, f64(pos), None if cell is None else np.asarray(cell, np.float64), _t(rp, dev),
                         _t(col, dev), _t(sh, dev), f64(x), f64(w), None if mask is None else _t(mask, dev),
                         gate=None if gate is None else f64(gate))
    torch.cuda.synchronize()
    assert out.dtype == torch.float64
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "c1_768", "c2_768", "si_mask", "si_gate"])
def test_conv_f64_workloads(dev, name):
    wl, plan, pos, box, cell, rp, col, sh, x, w, mask, gate = _workload(name)
    spec = (wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    got = _gpu_conv64(dev, spec, pos, cell, rp, col, sh, x, w, mask, gate)
    ref = O.conv_forward(plan, pos.astype(np.float64), cell, rp, col, sh, x.astype(np.float64),
                         w.astype(np.float64), mask, gate)
    _compare(got, ref, f"{name} fp64")


def _small_system(n, box_len, cutoff, seed):
    rng = np.random.default_rng(seed)
    pos = (rng.random((n, 3)) * box_len).astype(np.float32)
    pos[pos >= np.float32(box_len)] = 0
    box = np.full(3, box_len, dtype=np.float32)
    cell = np.diag(box).astype(np.float32)
    rp, col, sh = O.neighbors(pos, box, cutoff)
    return rng, pos, box, cell, rp, col, sh


@pytest.mark.parametrize("l1", range(5))
@pytest.mark.parametrize("mul", [2, 3, 130])
def test_conv_f64_every_variant(dev, l1, mul):
    """Every (l1, l2, l3) with l <= 4 in fp64: K = 2 (mul 2; mul 130 = one full channel
    block of 64 lanes * 2 and a ragged one) and K = 1 (mul 3)."""
    rng, pos, box, cell, rp, col, sh = _small_system(40, 6.0, 2.6, 200 + l1)
    for l2 in range(5):
        spec_in, spec_sh = f"{mul}x{l1}e", f"1x{l2}e"
        plan = O.build_plan(spec_in, spec_sh, 4, O.PATHS_ALL)
        x = rng.standard_normal((len(pos), plan.f_in))
        w = rng.standard_normal((len(col), plan.w_per_edge))
        got = _gpu_conv64(dev, (spec_in, spec_sh, 4, "all"), pos, cell, rp, col, sh, x, w)
        ref = O.conv_forward(plan, pos.astype(np.float64), cell, rp, col, sh, x, w)
        _compare(got, ref, f"{spec_in} x {spec_sh} fp64")


@pytest.mark.parametrize("name", ["c5_768", "c6_768"])
def test_conv_f64_large(dev, name):
    # LunaTP Table 1 cases 5 and 6 (L = 4) in fp64 at full size, over the whole output
    wl, plan, pos, box, cell, rp, col, sh, x, w, mask, gate = _workload(name)
    spec = (wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    got = _gpu_conv64(dev, spec, pos, cell, rp, col, sh, x, w)
    ref = O.conv_forward(plan, pos.astype(np.float64), cell, rp, col, sh, x.astype(np.float64),
                         w.astype(np.float64), None)
    _compare(got, ref, f"{name} fp64")


def test_conv_f64_deterministic(dev):
    wl, plan, pos, box, cell, rp, col, sh, x, w, mask, gate = _workload("si_mask")
    spec = (wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    p = C.Plan(*spec, fp64=True)
    a = _gpu_conv64(dev, spec, pos, cell, rp, col, sh, x, w, mask, plan=p)
    b = _gpu_conv64(dev, spec, pos, cell, rp, col, sh, x, w, mask, plan=p)
    assert np.array_equal(a, b)


def test_conv_precision_mismatch_rejected(dev):
    # an fp64 plan with the fp32 entry point and an fp32 plan with the fp64 one: errors
    lib = C._lib.load()
    wl, plan, pos, box, cell, rp, col, sh, x, w, mask, gate = _workload("tiny")
    spec = (wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    n, e = len(pos), len(col)
    p64, p32 = C.Plan(*spec, fp64=True), C.Plan(*spec)
    d = lambda a: ctypes.c_void_p(a.data_ptr())
    pos_d, rp_d, col_d = _t(pos, dev), _t(rp, dev), _t(col, dev)
    x_d, w_d = _t(x, dev), _t(w, dev)
    out = torch.empty((n, plan.f_out), dtype=torch.float32, device=dev)
    ws = torch.empty(p64.workspace_size(n, e), dtype=torch.uint8, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.cgtp_conv_forward(p64.handle, d(pos_d), n, None, d(rp_d), d(col_d), None, e, d(x_d), d(w_d), None,
                               d(out), d(ws), ws.numel(), s)
    assert rc == -1 and b"precision" in lib.cgtp_last_error()
    rc = lib.cgtp_conv_forward_f64(p32.handle, d(pos_d), n, None, d(rp_d), d(col_d), None, e, d(x_d), d(w_d),
                                   None, None, d(out), d(ws), ws.numel(), s, None, None)
    assert rc == -1 and b"precision" in lib.cgtp_last_error()
    with pytest.raises(TypeError):        # the binding checks the element type first
        C.conv_forward(p64, pos_d, cell, rp_d, col_d, _t(sh, dev), x_d, w_d)
