"""GPU test of cgtp_conv_forward_noalloc (the forward for callers that cannot allocate:
its scratch is the library's per-GPU device array) against cgtp_conv_forward_gated with
a caller workspace, through the C ABI: two calls in a row, the second on a smaller
graph (the array keeps the first call's contents), each equal to the workspace entry
point's output bit for bit (the same kernels) and within the parity bar of the oracle
comparison (relative L2 <= 1e-5, max |diff| <= 1e-4)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

C = pytest.importorskip("clebsch_gordan_tensor_node_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def _inputs(name, dev, gated=False):
    wl = WL.WORKLOADS[name]
    pos, box, cell, rng = WL.positions(wl)
    rp, col, sh = O.neighbors(pos, box, wl.cutoff)
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    x, w, mask = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    gate = None
    if gated:
        gate = np.where(np.random.default_rng(5).random(len(col)) < 0.3, 0.0, 0.5).astype(np.float32)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return wl, cell, [t(a) for a in (pos, rp, col, sh, x, w, mask, gate)]


def _noalloc(p, cell, tens, out):
    pos, rp, col, sh, x, w, mask, gate = tens
    lib = C._lib.load()
    cella = np.ascontiguousarray(np.asarray(cell, dtype=np.float32).reshape(-1))
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.cgtp_conv_forward_noalloc(p.handle, P(pos), pos.shape[0], cella.ctypes.data_as(C._lib.FP), P(rp),
                                         P(col), P(sh), col.shape[0], P(x), P(w), P(mask), P(gate), P(out),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _check(got, ref, what):
    g, r = got.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    mx = np.abs(g - r).max(initial=0.0)
    print(f"{what}: rel_l2={rel:.2e} max_abs={mx:.2e} bitwise={np.array_equal(g, r)}", flush=True)
    assert rel <= 1e-5 and mx <= 1e-4, (what, rel, mx)
    assert torch.equal(got, ref), what


def test_noalloc_matches_workspace_forward(dev):
    for name, gated in (("si_mask", False), ("c1_768", True), ("tiny", False)):
        wl, cell, tens = _inputs(name, dev, gated)
        pos, rp, col, sh, x, w, mask, gate = tens
        p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
        ref = C.conv_forward(p, pos, cell, rp, col, sh, x, w, mask, gate=gate)
        out = torch.full_like(ref, float("nan"))
        rc = _noalloc(p, cell, tens, out)
        assert rc == 0, C._lib.load().cgtp_last_error()
        torch.cuda.synchronize()
        _check(out, ref, f"{name} (gated={gated})")


def test_noalloc_refuses_oversized_and_fp64(dev):
    lib = C._lib.load()
    wl, cell, tens = _inputs("tiny", dev)
    pos, rp, col, sh, x, w, mask, gate = tens
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    need = ctypes.c_size_t()
    big_e = 3_000_000
    assert lib.cgtp_workspace_size(p.handle, pos.shape[0], big_e, 0, ctypes.byref(need)) == 0
    assert need.value > (64 << 20)
    out = torch.empty((pos.shape[0], p.f_out), dtype=torch.float32, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # refused on the host before any launch: the undersized buffers are never read
    rc = lib.cgtp_conv_forward_noalloc(p.handle, P(pos), pos.shape[0], None, P(rp), P(col), None, big_e, P(x), P(w),
                                       None, None, P(out), s)
    assert rc == -5, lib.cgtp_last_error()
    p64 = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, fp64=True)
    rc = lib.cgtp_conv_forward_noalloc(p64.handle, P(pos), pos.shape[0], None, P(rp), P(col), None, col.shape[0],
                                       P(x), P(w), None, None, P(out), s)
    assert rc == -1, lib.cgtp_last_error()
