"""Pins of the oracle's path enumeration and Clebsch-Gordan coefficients.

Independent references: the output irreps printed in LunaTP Table 1; sympy's exact
CG (a library routine); orthogonality relations; closed forms of low-l couplings.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from conftest import read_golden


def _lmax_sh(spec):
    return max(l for _, l, _ in O.parse_irreps(spec))


@pytest.mark.parametrize("row", read_golden("lunatp_table1_irreps.txt"), ids=lambda r: "case" + r[0])
def test_table1_output_irreps(row):
    case, _lmax, hidden, edge, expected = row
    rule = O.PATHS_ALL if case == "1" else O.PATHS_PARITY
    plan = O.build_plan(hidden, edge, _lmax_sh(edge), rule)
    assert O.format_irreps(plan.irreps_out) == expected


def test_workload_plans():
    import workloads as WL
    expect = {  # paths, F_in, F_out, W, output irreps
        "tiny": (5, 32, 88, 40, "16x0e+8x1e+16x1o"),
        "c1_768": (15, 480, 3136, 960, "224x0e+384x1e+352x2e"),
        "c2_768": (17, 1152, 9088, 2176, "384x0e+640x1o+640x2e+512x3o"),
        "highl_768": (106, 3136, 52864, 6784,
                      "448x0e+768x1o+1024x2e+1152x3o+1216x4e+1152x5o+1024x6e"),
        "si_mask": (23, 704, 5472, 1312, "256x0e+352x1o+384x2e+320x3o"),
    }
    for name, (npaths, fi, fo, w, irr) in expect.items():
        wl = WL.WORKLOADS[name]
        p = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
        assert (len(p.paths), p.f_in, p.f_out, p.w_per_edge, O.format_irreps(p.irreps_out)) == \
            (npaths, fi, fo, w, irr), name


def test_layout_offsets_tile_the_output():
    p = O.build_plan("8x0e+8x1o", "1x0e+1x1o", 1, O.PATHS_ALL)
    cover = np.zeros(p.f_out, dtype=int)
    wcover = np.zeros(p.w_per_edge, dtype=int)
    for q in p.paths:
        cover[q.out_off:q.out_off + q.mul * (2 * q.l3 + 1)] += 1
        wcover[q.w_off:q.w_off + q.mul] += 1
    assert (cover == 1).all() and (wcover == 1).all()


@pytest.mark.parametrize("bad", ["", "8x", "x0e", "8x0", "8x0q", "8x0e+", "ax1o", "8y0e"])
def test_parse_errors(bad):
    with pytest.raises(ValueError):
        O.parse_irreps(bad)


def test_cg_matches_sympy_exact():
    from sympy import S
    from sympy.physics.wigner import clebsch_gordan
    rng = np.random.default_rng(0)
    checked = 0
    for l1, l2 in itertools.product(range(7), repeat=2):
        for l3 in range(abs(l1 - l2), min(l1 + l2, 6) + 1):
            full = max(l1, l2, l3) <= 3
            for m1 in range(-l1, l1 + 1):
                for m2 in range(-l2, l2 + 1):
                    m3 = m1 + m2
                    if abs(m3) > l3 or (not full and rng.random() > 0.05):
                        continue
                    ref = float(clebsch_gordan(S(l1), S(l2), S(l3), S(m1), S(m2), S(m3)).evalf(30))
                    assert abs(O.cg_complex(l1, m1, l2, m2, l3, m3) - ref) <= 1e-15, (l1, m1, l2, m2, l3, m3)
                    checked += 1
    assert checked > 800


def test_cg_orthogonality_both_ways():
    for l1, l2 in [(1, 1), (2, 1), (2, 3), (3, 3), (4, 2), (6, 5)]:
        rows = []
        for J in range(abs(l1 - l2), l1 + l2 + 1):
            for M in range(-J, J + 1):
                rows.append([O.cg_complex(l1, m1, l2, m2, J, M)
                             for m1 in range(-l1, l1 + 1) for m2 in range(-l2, l2 + 1)])
        T = np.array(rows)                        # square: (2l1+1)(2l2+1)
        assert T.shape[0] == T.shape[1]
        np.testing.assert_allclose(T @ T.T, np.eye(T.shape[0]), atol=1e-14)
        np.testing.assert_allclose(T.T @ T, np.eye(T.shape[0]), atol=1e-14)


def test_cg_known_values():
    for l1 in range(7):
        for l2 in range(7):
            assert O.cg_complex(l1, l1, l2, l2, l1 + l2, l1 + l2) == pytest.approx(1.0, abs=1e-15)
    for m in (-1, 0, 1):
        assert O.cg_complex(1, m, 1, -m, 0, 0) == pytest.approx((-1) ** (1 - m) / math.sqrt(3), abs=1e-15)
    # swap symmetry <l2 m2 l1 m1|L M> = (-1)^(l1+l2-L) <l1 m1 l2 m2|L M>
    for l1, l2, L in [(1, 2, 2), (2, 3, 4), (3, 3, 3), (1, 1, 1)]:
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= L:
                    a = O.cg_complex(l1, m1, l2, m2, L, m1 + m2)
                    b = O.cg_complex(l2, m2, l1, m1, L, m1 + m2)
                    assert b == pytest.approx((-1) ** (l1 + l2 - L) * a, abs=1e-15)


def test_real_cg_residual_exactly_zero_and_orthonormal():
    for l1, l2 in itertools.product(range(7), repeat=2):
        for l3 in range(abs(l1 - l2), min(l1 + l2, 6) + 1):
            assert O.real_cg_residual(l1, l2, l3) <= 1e-15
            C = O.real_cg(l1, l2, l3)
            G = np.einsum("abk,abq->kq", C, C)
            np.testing.assert_allclose(G, np.eye(2 * l3 + 1), atol=2e-15)


def test_real_cg_low_l_closed_forms():
    s2, s3 = math.sqrt(2), math.sqrt(3)
    # identity couplings (0, l -> l) and (l, 0 -> l)
    for l in range(7):
        np.testing.assert_allclose(O.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-15)
        np.testing.assert_allclose(O.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-15)
    # (1,1 -> 0) = -delta/sqrt(3): minus the dot product
    np.testing.assert_allclose(O.real_cg(1, 1, 0)[:, :, 0], -np.eye(3) / s3, atol=1e-15)
    # (1,1 -> 1) = +cross product / sqrt(2) in the (y, z, x) component order
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal(3), rng.standard_normal(3)
    perm = [1, 2, 0]          # (x,y,z) -> (y,z,x)
    out = np.einsum("ijk,i,j->k", O.real_cg(1, 1, 1), a[perm], b[perm])
    np.testing.assert_allclose(out, np.cross(a, b)[perm] / s2, atol=1e-15)
    C = O.real_cg(1, 1, 2)          # indexes [m1+1, m2+1, m3+2]
    assert C[1, 1, 2] == pytest.approx(math.sqrt(6) / 3, abs=1e-15)
    assert C[0, 0, 2] == pytest.approx(-math.sqrt(6) / 6, abs=1e-15)
    assert C[2, 2, 2] == pytest.approx(-math.sqrt(6) / 6, abs=1e-15)
    assert C[2, 2, 4] == pytest.approx(math.sqrt(2) / 2, abs=1e-15)
    assert C[0, 0, 4] == pytest.approx(-math.sqrt(2) / 2, abs=1e-15)


def test_real_cg_nonzero_counts():
    expect = {(1, 1, 1): 6, (2, 2, 2): 25, (6, 6, 6): 217}
    for k, v in expect.items():
        assert O.cg_nnz(*k) == v
    import workloads as WL
    totals = []
    for name in WL.ORDER:
        wl = WL.WORKLOADS[name]
        p = O.build_plan(wl.irreps_in, wl.irreps_sh, wl.l_out_max, wl.rule)
        totals.append(sum(O.cg_nnz(q.l1, q.l2, q.l3) for q in p.paths))
    assert totals == [16, 137, 215, 6460, 353]


def test_real_cg_intertwines_rotations():
    rng = np.random.default_rng(7)
    for _ in range(3):
        R = O.random_rotation(rng)
        for l1, l2, l3 in [(1, 1, 1), (1, 2, 3), (2, 2, 2), (3, 2, 1), (3, 3, 6), (6, 5, 4)]:
            D1, D2, D3 = (O.wigner_d_real(l, R) for l in (l1, l2, l3))
            C = O.real_cg(l1, l2, l3)
            # coupling (D1 x, D2 y) gives D3 times the coupling of (x, y)
            lhs = np.einsum("abc,ai,bj->ijc", C, D1, D2)
            rhs = np.einsum("ck,ijk->ijc", D3, C)
            np.testing.assert_allclose(lhs, rhs, atol=1e-11)
