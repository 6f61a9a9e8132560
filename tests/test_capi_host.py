"""CPU tests of libcgtp: the library loads, exports every symbol the header declares,
and its host-side plan (parser, paths, layouts, real CG, schedule, argument checks)
agrees with the oracle.  No device work is done here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C = pytest.importorskip("clebsch_gordan_tensor_node_amd")


def _header_functions():
    src = open(os.path.join(ROOT, "include", "cgtp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cgtp_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = C.load() if hasattr(C, "load") else C._lib.load()
    names = _header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C._lib.EXPORTED)
    assert C.version().startswith("cgtp")


@pytest.mark.parametrize("name", WL.ORDER)
def test_host_plan_matches_oracle(name):
    wl = WL.WORKLOADS[name]
    p = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, host_only=True)
    q = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    assert (p.f_in, p.f_out, p.w_per_edge, p.n_paths) == (q.f_in, q.f_out, q.w_per_edge, len(q.paths))
    assert p.irreps_out == O.format_irreps(q.irreps_out)
    rows = p.paths()
    for k, r in enumerate(q.paths):
        assert rows[k].tolist() == [r.l1, r.p1, r.l2, r.p2, r.l3, r.p3, r.mul, r.in_off, r.out_off, r.w_off]
        ref = O.real_cg(r.l1, r.l2, r.l3)
        got = p.cg(k)
        np.testing.assert_allclose(got, ref, rtol=0, atol=6e-8)
        assert np.array_equal(got != 0, np.abs(ref) > 1e-12)     # identical sparsity
    nj, nv = p.schedule()
    assert nj >= p.n_paths and 1 <= nv <= p.n_paths


def test_all_real_cg_tables_l6():
    # every triangle triple up to l = 6 through single-path plans
    for l1 in range(7):
        for l2 in range(7):
            p = C.Plan(f"4x{l1}e", f"1x{l2}e", 6, "all", host_only=True)
            for k, r in enumerate(p.paths()):
                ref = O.real_cg(int(r[0]), int(r[2]), int(r[4]))
                np.testing.assert_allclose(p.cg(k), ref, rtol=0, atol=6e-8)


@pytest.mark.parametrize("bad", ["", "8x", "x0e", "8x0", "8x0q", "8x0e+", "ax1o"])
def test_parse_errors(bad):
    with pytest.raises(C.CgtpError) as e:
        C.Plan(bad, "1x0e", 1, "all", host_only=True)
    assert e.value.code == -2


def test_unsupported_and_invalid():
    with pytest.raises(C.CgtpError) as e:
        C.Plan("4x7e", "1x0e", 7, "all", host_only=True)
    assert e.value.code == -3
    with pytest.raises(C.CgtpError) as e:
        C.Plan("4x1e", "2x1e", 2, "all", host_only=True)          # SH multiplicity 2
    assert e.value.code == -3
    with pytest.raises(C.CgtpError) as e:
        C.Plan("4x0e", "1x1e", 2, "parity", host_only=True)      # 0e x 1e -> 1e is not natural
    assert e.value.code == -3
    with pytest.raises(C.CgtpError) as e:
        C.Plan("4x1o", "1x0e", 2, 7, host_only=True)
    assert e.value.code == -1


def test_host_only_plan_refuses_device_calls():
    lib = C._lib.load()
    p = C.Plan("8x0e+8x1o", "1x0e+1x1o", 1, "all", host_only=True)
    rc = lib.cgtp_conv_forward(p.handle, None, 0, None, None, None, None, 0, None, None, None, None,
                               None, 0, None)
    assert rc == -1 and b"HOST_ONLY" in lib.cgtp_last_error()
    rc = lib.cgtp_conv_prepare(p.handle, None, None, 0, 0, None, None, None, None, 0, None)
    assert rc == -1


def test_workspace_size_monotone():
    p = C.Plan("128x0e+64x1o+32x2e+32x3o", "1x0e+1x1o+1x2e+1x3o", 3, "parity", host_only=True)
    a = p.workspace_size(100, 1000)
    b = p.workspace_size(200, 5000)
    assert 0 < a < b and a % 256 == 0
    lib = C._lib.load()
    sz = ctypes.c_size_t()
    box = np.full(3, 10.0, dtype=np.float32)
    assert lib.cgtp_neighbors_workspace_size(100, box.ctypes.data_as(C._lib.FP), 3.0, ctypes.byref(sz)) == 0
    assert sz.value > 0
    assert lib.cgtp_neighbors_workspace_size(100, box.ctypes.data_as(C._lib.FP), -1.0, ctypes.byref(sz)) == -1


@pytest.mark.parametrize("name", ["tiny", "c1_768", "c2_768", "si_mask"])
def test_fp64_plan_host(name):
    # an fp64 plan has the fp32 plan's layout; only its schedule (16-byte chunks of two
    # elements) and its workspace (fp64 harmonics) differ
    wl = WL.WORKLOADS[name]
    p32 = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, host_only=True)
    p64 = C.Plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule, host_only=True, fp64=True)
    assert (p64.f_in, p64.f_out, p64.w_per_edge, p64.n_paths) == (p32.f_in, p32.f_out, p32.w_per_edge, p32.n_paths)
    assert np.array_equal(p64.paths(), p32.paths())
    nj, nv = p64.schedule()
    assert nj >= p64.n_paths and nv >= 1
    assert p64.workspace_size(768, 20000) > p32.workspace_size(768, 20000)


def test_fp64_plan_limits():
    with pytest.raises(C.CgtpError) as e:        # fp64 kernels are built for l <= 4
        C.Plan("8x0e+8x5e", "1x0e+1x1o", 5, "all", host_only=True, fp64=True)
    assert e.value.code == -3
    with pytest.raises(C.CgtpError) as e:        # l = 5 in the harmonics only
        C.Plan("8x2o", "1x0e+1x5e", 3, "all", host_only=True, fp64=True)
    assert e.value.code == -3
    C.Plan("8x0e+8x4e", "1x0e+1x4e", 4, "all", host_only=True, fp64=True)
    lib = C._lib.load()
    h = ctypes.c_void_p()
    assert lib.cgtp_plan_create(b"8x0e", b"1x0e", 0, 0, 4, ctypes.byref(h)) == -1   # unknown flag
    p = C.Plan("8x0e+8x3o", "1x0e+1x3o", 3, "all", host_only=True, fp64=True)
    rc = lib.cgtp_conv_forward_f64(p.handle, None, 0, None, None, None, None, 0, None, None, None, None,
                                   None, None, 0, None, None, None)
    assert rc == -1 and b"HOST_ONLY" in lib.cgtp_last_error()
