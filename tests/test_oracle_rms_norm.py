"""Pins for the RMSNorm-backward oracle: each checks it against something other than itself.

CPU only.  The subject page (trueno-gpu 0.4.17, src/kernels/backward/rms_norm.rs, module
documentation) predicts that the backward matches finite differences within 1e-5; here the fp64
oracle is held to finite differences of the fp64 forward far tighter, plus the scale invariance of
RMSNorm and a closed form.
"""

import numpy as np
import pytest

from oracle.rms_norm_oracle import rms_norm_backward, rms_norm_backward_bound, rms_norm_forward


def _inputs(rows, H, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(rows, H))
    gamma = rng.normal(1.0, 0.3, size=H)
    u = rng.normal(0.0, 1.0, size=(rows, H))  # upstream gradient: L = sum(y * u)
    return x, gamma, u


@pytest.mark.parametrize("rows,H,eps,seed", [(3, 5, 1e-6, 0), (2, 17, 1e-2, 1), (4, 64, 1e-5, 2), (1, 1, 0.5, 3)])
def test_rms_norm_backward_matches_central_differences(rows, H, eps, seed):
    x, gamma, u = _inputs(rows, H, seed)
    _, rms = rms_norm_forward(x, gamma, eps)
    dx, dgamma = rms_norm_backward(x, gamma, rms, u)

    def loss(xx, gg):
        y, _ = rms_norm_forward(xx, gg, eps)
        return float(np.sum(y * u))

    h = 1e-6
    fdx = np.zeros_like(x)
    for i in range(rows):
        for j in range(H):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fdx[i, j] = (loss(xp, gamma) - loss(xm, gamma)) / (2 * h)
    fdg = np.zeros_like(gamma)
    for j in range(H):
        gp, gm = gamma.copy(), gamma.copy()
        gp[j] += h
        gm[j] -= h
        fdg[j] = (loss(x, gp) - loss(x, gm)) / (2 * h)
    assert np.allclose(dx, fdx, rtol=1e-6, atol=1e-7)
    assert np.allclose(dgamma, fdg, rtol=1e-6, atol=1e-7)


def test_rms_norm_backward_scale_invariance_without_eps():
    """With eps = 0, y(c x) = y(x) for c > 0, so the derivative along x vanishes: sum_i x_i dx_i = 0."""
    x, gamma, u = _inputs(6, 40, 7)
    _, rms = rms_norm_forward(x, gamma, 0.0)
    dx, _ = rms_norm_backward(x, gamma, rms, u)
    along = np.sum(x * dx, axis=1)
    assert np.all(np.abs(along) <= 1e-12 * np.sum(np.abs(x * dx), axis=1))


def test_rms_norm_backward_equals_printed_formula_at_unit_gamma():
    """With gamma = 1 the page's printed dx formula and the exact derivative coincide."""
    x, _, u = _inputs(4, 20, 13)
    ones = np.ones(20)
    _, rms = rms_norm_forward(x, ones, 1e-5)
    dx, _ = rms_norm_backward(x, ones, rms, u)
    r = rms[:, None]
    printed = ones / r * (u - x / (r * r) * np.mean(x * u * ones, axis=1, keepdims=True))
    assert np.allclose(dx, printed, rtol=1e-14, atol=1e-15)


def test_rms_norm_backward_constant_row_closed_form():
    """x = a * 1, gamma = 1, eps = 0: rms = |a| and dx = (dy - mean(dy)) / |a| (the mean is projected out)."""
    H = 12
    rng = np.random.default_rng(9)
    for a in (0.5, -3.0):
        x = np.full((1, H), a)
        dy = rng.normal(size=(1, H))
        _, rms = rms_norm_forward(x, np.ones(H), 0.0)
        assert rms[0] == abs(a)
        dx, dgamma = rms_norm_backward(x, np.ones(H), rms, dy)
        assert np.allclose(dx, (dy - dy.mean()) / abs(a), rtol=1e-14, atol=1e-15)
        assert np.allclose(dgamma, dy[0] * np.sign(a), rtol=1e-14, atol=1e-15)


def test_rms_norm_backward_bound_dominates_terms():
    x, gamma, u = _inputs(5, 33, 11)
    _, rms = rms_norm_forward(x, gamma, 1e-5)
    dx, dgamma = rms_norm_backward(x, gamma, rms, u)
    sx, sg = rms_norm_backward_bound(x, gamma, rms, u)
    assert np.all(np.abs(dx) <= sx * (1 + 1e-12))
    assert np.all(np.abs(dgamma) <= sg * (1 + 1e-12))
