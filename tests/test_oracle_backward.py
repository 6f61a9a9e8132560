"""Pins of the oracle's gradients (conv_backward, real_sh_grad) against things other
than themselves: finite differences of the (separately pinned) forward, the l = 1
closed form of the harmonics' gradient, tangency and homogeneity of that gradient, and
translation invariance of the forces."""
import math

import numpy as np
import pytest

import oracle as O


def _system(seed, n=24, box_len=5.5, cutoff=2.9, spec_in="3x0e+2x1o+2x2e+2x3o",
            spec_sh="1x0e+1x1o+1x2e+1x3o", lmax=3, rule=O.PATHS_PARITY):
    rng = np.random.default_rng(seed)
    pos = rng.random((n, 3)) * box_len
    box = np.full(3, box_len)
    cell = np.diag(box)
    rp, col, sh = O.neighbors(pos.astype(np.float32), box.astype(np.float32), cutoff)
    plan = O.build_plan(spec_in, spec_sh, lmax, rule)
    x = rng.standard_normal((n, plan.f_in))
    w = rng.standard_normal((len(col), plan.w_per_edge))
    gout = rng.standard_normal((n, plan.f_out))
    return rng, plan, pos, cell, rp, col, sh, x, w, gout


def _loss(plan, pos, cell, rp, col, sh, x, w, gout, mask=None, gate=None):
    return float((O.conv_forward(plan, pos, cell, rp, col, sh, x, w, mask, gate) * gout).sum())


# ---------------------------------------------------------------------------------
# real_sh_grad
# ---------------------------------------------------------------------------------

def test_sh_grad_l1_closed_form():
    # Y_1 = sqrt(3) (y, z, x) / |r|  =>  dY_1/dr = sqrt(3) (I - rhat rhat^T) / |r| rows (y, z, x)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((50, 3)) * 2.0
    r = np.linalg.norm(v, axis=1)
    rh = v / r[:, None]
    proj = (np.eye(3)[None] - rh[:, :, None] * rh[:, None, :]) / r[:, None, None]
    ref = math.sqrt(3.0) * proj[:, [1, 2, 0], :]
    np.testing.assert_allclose(O.real_sh_grad(1, v), ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("l", range(0, 7))
def test_sh_grad_finite_difference(l):
    rng = np.random.default_rng(10 + l)
    v = rng.standard_normal((40, 3)) * 1.7
    got = O.real_sh_grad(l, v)
    h = 1e-6
    fd = np.zeros_like(got)
    for k in range(3):
        d = np.zeros(3)
        d[k] = h
        fd[:, :, k] = (O.real_sh(l, v + d) - O.real_sh(l, v - d)) / (2 * h)
    scale = max(1.0, np.abs(got).max())
    assert np.abs(got - fd).max() <= 2e-7 * scale


@pytest.mark.parametrize("l", range(1, 7))
def test_sh_grad_tangent_and_homogeneous(l):
    # Y depends on the direction only: the gradient is orthogonal to r and scales as 1/|r|
    rng = np.random.default_rng(30 + l)
    v = rng.standard_normal((30, 3))
    gr = O.real_sh_grad(l, v)
    assert np.abs(np.einsum("ebk,ek->eb", gr, v)).max() <= 1e-12 * np.abs(gr).max()
    np.testing.assert_allclose(O.real_sh_grad(l, 3.0 * v), gr / 3.0, rtol=1e-12, atol=1e-14)


def test_sh_grad_refuses_pole():
    with pytest.raises(ValueError):
        O.real_sh_grad(2, np.array([[0.0, 0.0, 1.0]]))


# ---------------------------------------------------------------------------------
# conv_backward
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_grad_w_and_x_exact_directional(seed):
    # L is linear in w and in x: L(w + d) - L(w) = <grad_w, d> exactly (up to rounding)
    rng, plan, pos, cell, rp, col, sh, x, w, gout = _system(seed)
    gx, gw, _ = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout)
    L0 = _loss(plan, pos, cell, rp, col, sh, x, w, gout)
    dw = rng.standard_normal(w.shape)
    lw = _loss(plan, pos, cell, rp, col, sh, x, w + dw, gout) - L0
    assert abs(lw - (gw * dw).sum()) <= 1e-10 * max(1.0, abs(lw))
    dx = rng.standard_normal(x.shape)
    lx = _loss(plan, pos, cell, rp, col, sh, x + dx, w, gout) - L0
    assert abs(lx - (gx * dx).sum()) <= 1e-10 * max(1.0, abs(lx))
    # and entry by entry on a few coordinates (catches a misplaced block)
    for (a, b) in [(0, 0), (3, plan.w_per_edge - 1), (len(col) // 2, plan.w_per_edge // 2)]:
        d = np.zeros_like(w)
        d[a, b] = 1.0
        assert abs(_loss(plan, pos, cell, rp, col, sh, x, w + d, gout) - L0 - gw[a, b]) <= 1e-10 * max(1, abs(gw[a, b]))
    for (a, b) in [(1, 0), (5, plan.f_in - 1), (7, plan.f_in // 2)]:
        d = np.zeros_like(x)
        d[a, b] = 1.0
        assert abs(_loss(plan, pos, cell, rp, col, sh, x + d, w, gout) - L0 - gx[a, b]) <= 1e-10 * max(1, abs(gx[a, b]))


@pytest.mark.parametrize("seed", [0, 1])
def test_grad_pos_finite_difference(seed):
    rng, plan, pos, cell, rp, col, sh, x, w, gout = _system(seed)
    _, _, gp = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout)
    h = 1e-5
    for a in [0, 5, 11, 17]:
        for k in range(3):
            d = np.zeros_like(pos)
            d[a, k] = h
            fd = (_loss(plan, pos + d, cell, rp, col, sh, x, w, gout)
                  - _loss(plan, pos - d, cell, rp, col, sh, x, w, gout)) / (2 * h)
            assert abs(fd - gp[a, k]) <= 1e-6 * max(1.0, abs(gp[a, k])), (a, k, fd, gp[a, k])


def test_forces_translation_invariant():
    rng, plan, pos, cell, rp, col, sh, x, w, gout = _system(3)
    _, _, gp = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout)
    assert np.abs(gp.sum(axis=0)).max() <= 1e-11 * np.abs(gp).max()


def test_backward_masked_and_gated():
    rng, plan, pos, cell, rp, col, sh, x, w, gout = _system(4)
    e = len(col)
    mask = (rng.random(e) < 0.6).astype(np.uint8)
    gate = np.where(rng.random(e) < 0.3, 0.0, rng.random(e))
    inactive = (mask == 0) | (gate == 0.0)
    w_nan = w.copy()
    w_nan[inactive] = np.nan
    gx, gw, gp = O.conv_backward(plan, pos, cell, rp, col, sh, x, w_nan, gout, mask, gate)
    assert np.all(np.isfinite(gx)) and np.all(np.isfinite(gp)) and np.all(np.isfinite(gw))
    assert np.all(gw[inactive] == 0.0)
    # directional checks with mask and gate
    L0 = _loss(plan, pos, cell, rp, col, sh, x, w, gout, mask, gate)
    dw = rng.standard_normal(w.shape)
    lw = _loss(plan, pos, cell, rp, col, sh, x, w + dw, gout, mask, gate) - L0
    assert abs(lw - (gw * dw).sum()) <= 1e-10 * max(1.0, abs(lw))
    dx = rng.standard_normal(x.shape)
    lx = _loss(plan, pos, cell, rp, col, sh, x + dx, w, gout, mask, gate) - L0
    assert abs(lx - (gx * dx).sum()) <= 1e-10 * max(1.0, abs(lx))
    h = 1e-5
    for a in [2, 9]:
        for k in range(3):
            d = np.zeros_like(pos)
            d[a, k] = h
            fd = (_loss(plan, pos + d, cell, rp, col, sh, x, w, gout, mask, gate)
                  - _loss(plan, pos - d, cell, rp, col, sh, x, w, gout, mask, gate)) / (2 * h)
            assert abs(fd - gp[a, k]) <= 1e-6 * max(1.0, abs(gp[a, k]))


def test_backward_all_paths_rule_and_empty():
    rng, plan, pos, cell, rp, col, sh, x, w, gout = _system(5, spec_in="2x0e+2x1e+2x2e", spec_sh="1x0e+1x1e+1x2e",
                                                            lmax=2, rule=O.PATHS_ALL)
    gx, gw, gp = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout)
    L0 = _loss(plan, pos, cell, rp, col, sh, x, w, gout)
    dx = rng.standard_normal(x.shape)
    lx = _loss(plan, pos, cell, rp, col, sh, x + dx, w, gout) - L0
    assert abs(lx - (gx * dx).sum()) <= 1e-10 * max(1.0, abs(lx))
    zero = np.zeros(len(col), dtype=np.uint8)
    gx0, gw0, gp0 = O.conv_backward(plan, pos, cell, rp, col, sh, x, w, gout, zero)
    assert not gx0.any() and not gw0.any() and not gp0.any()
