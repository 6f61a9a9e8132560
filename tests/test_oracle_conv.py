"""Pins of the oracle's convolution.

Independent references: a pure-Python loop over the definition; textbook special
cases (a CSR sparse-matrix/vector product from scipy.sparse, the cross and dot
products of vectors); whole-convolution invariants: SO(3) equivariance (TransIP
Sec. 2.1, Eq. (1)), inversion, translation, relabelling, linearity, and BranchIP's
sparse-equals-dense statement (Method, proof intuition).
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle as O
import workloads as WL


def _random_system(n, box_len, cutoff, seed):
    rng = np.random.default_rng(seed)
    pos = (rng.random((n, 3)) * box_len).astype(np.float32)
    box = np.full(3, box_len, dtype=np.float32)
    row_ptr, col, shift = O.neighbors(pos, box, cutoff)
    cell = np.diag(box).astype(np.float32)
    return rng, pos, box, cell, row_ptr, col, shift


def _case(irr_in, irr_sh, lmax, rule, n=24, box_len=7.0, cutoff=3.2, seed=0, masked=False):
    plan = O.build_plan(irr_in, irr_sh, lmax, rule)
    rng, pos, box, cell, row_ptr, col, shift = _random_system(n, box_len, cutoff, seed)
    e = len(col)
    x = rng.standard_normal((n, plan.f_in))
    w = rng.standard_normal((e, plan.w_per_edge))
    mask = (rng.random(e) < 0.5).astype(np.uint8) if masked else None
    return plan, pos, box, cell, row_ptr, col, shift, x, w, mask


def _sh_spec(lmax, natural=True):
    return "+".join(f"1x{l}{('e' if l % 2 == 0 else 'o') if natural else 'e'}" for l in range(lmax + 1))


def _rot_x(plan, x, R):
    """Apply D_l(R) to every channel of every input irrep block."""
    out = np.array(x, dtype=np.float64, copy=True)
    off = 0
    for mul, l, _ in plan.irreps_in:
        n = 2 * l + 1
        D = O.wigner_d_real(l, R)
        blk = out[:, off:off + mul * n].reshape(-1, mul, n)
        out[:, off:off + mul * n] = (blk @ D.T).reshape(-1, mul * n)
        off += mul * n
    return out


def _rot_out(plan, y, R):
    out = np.array(y, copy=True)
    off = 0
    for mul, l, _ in plan.irreps_out:
        n = 2 * l + 1
        D = O.wigner_d_real(l, R)
        blk = out[:, off:off + mul * n].reshape(-1, mul, n)
        out[:, off:off + mul * n] = (blk @ D.T).reshape(-1, mul * n)
        off += mul * n
    return out


def _parity_scale(irreps, y):
    out = np.array(y, copy=True)
    off = 0
    for mul, l, p in irreps:
        n = mul * (2 * l + 1)
        out[:, off:off + n] *= p
        off += n
    return out


CASES = {
    "tiny": ("8x0e+8x1o", _sh_spec(1), 1, O.PATHS_ALL),
    "case1": ("8x0e+4x1e+4x2e", _sh_spec(2, natural=False), 2, O.PATHS_ALL),
    "case2": ("4x0e+4x1o+4x2e", _sh_spec(3), 3, O.PATHS_PARITY),
    "si": ("8x0e+4x1o+4x2e+4x3o", _sh_spec(3), 3, O.PATHS_PARITY),
    "highl": ("+".join(f"2x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(7)), _sh_spec(6), 6, O.PATHS_PARITY),
}


@pytest.mark.parametrize("masked", [False, True])
def test_vectorised_equals_python_loops_tiny(masked):
    wl = WL.WORKLOADS["tiny"]
    plan = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
    pos, box, cell, rng = WL.positions(wl)
    row_ptr, col, shift = O.neighbors(pos, box, wl.cutoff)
    x, w, _ = WL.draw_payload(wl, rng, wl.n_atoms, plan.f_in, len(col), plan.w_per_edge)
    mask = (np.arange(len(col)) % 3 != 0).astype(np.uint8) if masked else None
    a = O.conv_forward(plan, pos, cell, row_ptr, col, shift, x, w, mask)
    b = O.conv_forward_loops(plan, pos, cell, row_ptr, col, shift, x, w, mask)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_vectorised_equals_python_loops_high_l():
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(
        "2x0e+1x1o+1x2e+1x3o+1x4e", _sh_spec(4), 4, O.PATHS_PARITY, n=8, box_len=4.0, cutoff=1.9, masked=True)
    a = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask)
    b = O.conv_forward_loops(plan, pos, cell, rp, col, sh, x, w, mask)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def _csr(rp, col, vals, n):
    return sp.csr_matrix((vals, col, rp), shape=(n, n))


def test_scalar_path_is_spmv():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case("16x0e", "1x0e", 0, O.PATHS_ALL)
    out = O.conv_forward(plan, pos, cell, rp, col, sh, x, w)
    n = len(rp) - 1
    ref = np.stack([_csr(rp, col, w[:, u], n) @ x[:, u] for u in range(16)], 1)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_l1_times_scalar_sh_is_spmv():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case("6x2e", "1x0e", 2, O.PATHS_ALL)
    out = O.conv_forward(plan, pos, cell, rp, col, sh, x, w).reshape(-1, 6, 5)
    n = len(rp) - 1
    xb = x.reshape(n, 6, 5)
    for u in range(6):
        A = _csr(rp, col, w[:, u], n)
        np.testing.assert_allclose(out[:, u, :], A @ xb[:, u, :], atol=1e-12)


def test_scalar_times_sh_path():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case("5x0e", "1x3o", 3, O.PATHS_ALL)
    out = O.conv_forward(plan, pos, cell, rp, col, sh, x, w).reshape(-1, 5, 7)
    n = len(rp) - 1
    r = O.edge_vectors(pos, cell, rp, col, sh)
    Y = O.real_sh(3, r)
    recv = np.repeat(np.arange(n), np.diff(rp))
    ref = np.zeros((n, 5, 7))
    np.add.at(ref, recv, (w[:, :, None] * x[col][:, :, None]) * Y[:, None, :])
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_vector_couplings_are_dot_and_cross():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case("4x1o", "1x1o", 2, O.PATHS_ALL)
    assert [(p.l3, p.p3) for p in plan.paths] == [(0, 1), (1, 1), (2, 1)]
    out = O.conv_forward(plan, pos, cell, rp, col, sh, x, w)
    n = len(rp) - 1
    r = O.edge_vectors(pos, cell, rp, col, sh)
    rhat = r / np.linalg.norm(r, axis=1, keepdims=True)
    perm, inv = [1, 2, 0], [2, 0, 1]            # (x,y,z) <-> (y,z,x)
    xv = x.reshape(n, 4, 3)[:, :, inv][col]      # sender vectors in (x,y,z)
    yv = math.sqrt(3) * rhat                    # Y_1 in (x,y,z)
    recv = np.repeat(np.arange(n), np.diff(rp))
    p0, p1 = plan.paths[0], plan.paths[1]
    dot = -np.einsum("euk,ek->eu", xv, yv) / math.sqrt(3)
    ref0 = np.zeros((n, 4))
    np.add.at(ref0, recv, w[:, p0.w_off:p0.w_off + 4] * dot)
    np.testing.assert_allclose(out[:, p0.out_off:p0.out_off + 4], ref0, atol=1e-12)
    cross = np.cross(xv, yv[:, None, :]) / math.sqrt(2)
    ref1 = np.zeros((n, 4, 3))
    np.add.at(ref1, recv, w[:, p1.w_off:p1.w_off + 4, None] * cross)
    got1 = out[:, p1.out_off:p1.out_off + 12].reshape(n, 4, 3)[:, :, inv]
    np.testing.assert_allclose(got1, ref1, atol=1e-12)


@pytest.mark.parametrize("name", list(CASES))
def test_so3_equivariance(name):
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES[name], masked=(name == "si"))
    ref = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask)
    rng = np.random.default_rng(11)
    scale = np.abs(ref).max()
    for _ in range(10):
        R = O.random_rotation(rng)
        out = O.conv_forward(plan, pos.astype(np.float64) @ R.T, cell.astype(np.float64) @ R.T,
                             rp, col, sh, _rot_x(plan, x, R), w, mask)
        np.testing.assert_allclose(out, _rot_out(plan, ref, R), rtol=0, atol=1e-12 * scale)


@pytest.mark.parametrize("name", ["tiny", "case2", "si", "highl"])
def test_inversion(name):
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES[name])
    ref = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask)
    out = O.conv_forward(plan, -pos.astype(np.float64), cell, rp, col, -sh.astype(np.int64),
                         _parity_scale(plan.irreps_in, x), w, mask)
    np.testing.assert_allclose(out, _parity_scale(plan.irreps_out, ref), atol=1e-12 * np.abs(ref).max())


def test_translation_with_rewrap():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case(*CASES["si"])
    ref = O.conv_forward(plan, pos, cell, rp, col, sh, x, w)
    moved = np.mod(pos.astype(np.float64) + np.array([2.3, -5.1, 0.7]), box[0]).astype(np.float32)
    moved[moved >= box[0]] = 0
    rp2, col2, sh2 = O.neighbors(moved, box, 3.2)
    assert np.array_equal(rp2, rp) and np.array_equal(col2, col)
    out = O.conv_forward(plan, moved, cell, rp2, col2, sh2, x, w)
    np.testing.assert_allclose(out, ref, atol=1e-5 * np.abs(ref).max())


def test_relabelling():
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES["case2"], masked=True)
    n = len(rp) - 1
    ref = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask)
    q = np.random.default_rng(4).permutation(n)          # old atom a -> new label q[a]
    pos2 = np.empty_like(pos)
    pos2[q] = pos
    x2 = np.empty_like(x)
    x2[q] = x
    rp2, col2, sh2 = O.neighbors(pos2, box, 3.2)
    recv = np.repeat(np.arange(n), np.diff(rp))
    old = {(int(q[recv[e]]), int(q[col[e]])): e for e in range(len(col))}
    recv2 = np.repeat(np.arange(n), np.diff(rp2))
    idx = np.array([old[(int(recv2[e]), int(col2[e]))] for e in range(len(col2))])
    out = O.conv_forward(plan, pos2, cell, rp2, col2, sh2, x2, w[idx], mask[idx])
    np.testing.assert_allclose(out[q], ref, atol=1e-12 * np.abs(ref).max())


def test_linearity():
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case(*CASES["case2"])
    rng = np.random.default_rng(9)
    x2, w2 = rng.standard_normal(x.shape), rng.standard_normal(w.shape)
    f = lambda xx, ww: O.conv_forward(plan, pos, cell, rp, col, sh, xx, ww)
    np.testing.assert_allclose(f(2 * x - 3 * x2, w), 2 * f(x, w) - 3 * f(x2, w), atol=1e-11)
    np.testing.assert_allclose(f(x, 0.5 * w + w2), 0.5 * f(x, w) + f(x, w2), atol=1e-11)


def test_sparse_equals_dense_and_nan_never_read():
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES["si"], masked=True)
    sparse = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask)
    wd = w.copy()
    wd[mask == 0] = 0.0
    dense = O.conv_forward(plan, pos, cell, rp, col, sh, x, wd, None)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-13 * np.abs(dense).max())
    wn = w.copy()
    wn[mask == 0] = np.nan
    np.testing.assert_array_equal(O.conv_forward(plan, pos, cell, rp, col, sh, x, wn, mask), sparse)
    # all edges masked: exactly zero
    z = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, np.zeros_like(mask))
    assert np.all(z == 0.0)


def _gate(rng, e):
    """A continuation gate with a flat exact-zero region: half the edges exactly 0, the
    rest in (0, 1] (BranchIP, Method)."""
    g = rng.random(e)
    return np.where(rng.random(e) < 0.5, 0.0, 1.0 - g)


def test_gate_equals_dense_with_scaled_weights():
    # gating an edge's feature scales its message: the gated sparse evaluation equals the
    # ungated dense one with each weight row multiplied by the gate (zero rows included)
    plan, pos, box, cell, rp, col, sh, x, w, _ = _case(*CASES["si"])
    g = _gate(np.random.default_rng(3), len(col))
    gated = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, gate=g)
    dense = O.conv_forward(plan, pos, cell, rp, col, sh, x, w * g[:, None])
    np.testing.assert_allclose(gated, dense, rtol=0, atol=1e-13 * np.abs(dense).max())


def test_gate_special_cases_and_nan_never_read():
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES["case2"], masked=True)
    e = len(col)
    plain = O.conv_forward(plan, pos, cell, rp, col, sh, x, w)
    # a gate of ones is no gate; a 0/1 gate is the mask
    np.testing.assert_array_equal(O.conv_forward(plan, pos, cell, rp, col, sh, x, w, gate=np.ones(e)), plain)
    np.testing.assert_array_equal(
        O.conv_forward(plan, pos, cell, rp, col, sh, x, w, gate=mask.astype(np.float64)),
        O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask))
    # a constant gate scales the whole output
    np.testing.assert_allclose(O.conv_forward(plan, pos, cell, rp, col, sh, x, w, gate=np.full(e, 0.25)),
                               0.25 * plain, rtol=0, atol=1e-14 * np.abs(plain).max())
    # zero-gated edges are never read, also combined with a mask
    g = _gate(np.random.default_rng(5), e)
    ref = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask, g)
    wn = w.copy()
    wn[(g == 0) | (mask == 0)] = np.nan
    np.testing.assert_array_equal(O.conv_forward(plan, pos, cell, rp, col, sh, x, wn, mask, g), ref)


def test_gated_vectorised_equals_python_loops():
    plan, pos, box, cell, rp, col, sh, x, w, mask = _case(*CASES["tiny"], n=16, box_len=5.0, cutoff=2.6,
                                                          masked=True)
    g = _gate(np.random.default_rng(7), len(col))
    a = O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask, g)
    b = O.conv_forward_loops(plan, pos, cell, rp, col, sh, x, w, mask, g)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
