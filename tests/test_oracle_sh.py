"""Pins of the oracle's real spherical harmonics and fitted Wigner-D.

Independent references: hand-derived closed forms for l <= 2, Unsoeld's theorem,
orthonormality by a product quadrature exact to the needed degree, and the rotation
matrix itself as the l = 1 representation.
"""
import math

import numpy as np
import pytest

import oracle as O


def _unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_closed_forms_l_le_2():
    rng = np.random.default_rng(0)
    v = _unit(rng, 50)
    x, y, z = v.T
    s3, s5, s15 = math.sqrt(3), math.sqrt(5), math.sqrt(15)
    np.testing.assert_allclose(O.real_sh(0, v)[:, 0], 1.0, atol=1e-15)
    np.testing.assert_allclose(O.real_sh(1, v), s3 * np.stack([y, z, x], 1), atol=1e-14)
    y2 = np.stack([s15 * x * y, s15 * y * z, s5 / 2 * (3 * z * z - 1), s15 * x * z, s15 / 2 * (x * x - y * y)], 1)
    np.testing.assert_allclose(O.real_sh(2, v), y2, atol=1e-13)
    # only the direction matters
    np.testing.assert_allclose(O.real_sh(2, 3.7 * v), y2, atol=1e-13)


def test_zero_vector_convention():
    z = np.zeros((1, 3))
    assert O.real_sh(0, z)[0, 0] == 1.0
    for l in range(1, 7):
        assert np.all(O.real_sh(l, z) == 0.0)


@pytest.mark.parametrize("l", range(7))
def test_unsold(l):
    v = _unit(np.random.default_rng(l), 200)
    np.testing.assert_allclose((O.real_sh(l, v) ** 2).sum(1), 2 * l + 1, rtol=1e-12)


def test_quadrature_orthonormality():
    lmax = 6
    # Gauss-Legendre in cos(theta) (exact to degree 2n-1) x uniform phi (exact to 2n-1)
    nt, nphi = 16, 32
    ct, wt = np.polynomial.legendre.leggauss(nt)
    phi = 2 * np.pi * np.arange(nphi) / nphi
    st = np.sqrt(1 - ct * ct)
    pts = np.stack([np.outer(st, np.cos(phi)), np.outer(st, np.sin(phi)),
                    np.outer(ct, np.ones(nphi))], -1).reshape(-1, 3)
    wq = np.outer(wt, np.full(nphi, 2 * np.pi / nphi)).reshape(-1) / (4 * np.pi)
    Y = np.concatenate([O.real_sh(l, pts) for l in range(lmax + 1)], 1)
    G = (Y * wq[:, None]).T @ Y
    np.testing.assert_allclose(G, np.eye(G.shape[0]), atol=1e-12)


def test_wigner_d_properties():
    rng = np.random.default_rng(3)
    R1, R2 = O.random_rotation(rng), O.random_rotation(rng)
    perm = [1, 2, 0]
    np.testing.assert_allclose(O.wigner_d_real(1, R1), R1[np.ix_(perm, perm)], atol=1e-12)
    for l in range(7):
        D1, D2 = O.wigner_d_real(l, R1), O.wigner_d_real(l, R2)
        np.testing.assert_allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-11)
        np.testing.assert_allclose(O.wigner_d_real(l, R1 @ R2), D1 @ D2, atol=1e-11)
        np.testing.assert_allclose(O.wigner_d_real(l, np.eye(3)), np.eye(2 * l + 1), atol=1e-11)
        v = _unit(rng, 20)
        np.testing.assert_allclose(O.real_sh(l, v @ R1.T), O.real_sh(l, v) @ D1.T, atol=1e-11)
        # parity: Y_l(-r) = (-1)^l Y_l(r)
        np.testing.assert_allclose(O.real_sh(l, -v), (-1) ** l * O.real_sh(l, v), atol=1e-12)


def test_random_rotation_is_rotation():
    rng = np.random.default_rng(5)
    for _ in range(10):
        R = O.random_rotation(rng)
        np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-14)
        assert np.linalg.det(R) == pytest.approx(1.0, abs=1e-13)
