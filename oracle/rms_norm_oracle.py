"""Plain CPU oracle (numpy, fp64) for the RMSNorm backward.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` legs of ``bench.py`` use
it; the HIP library never does, and the two share no code.

Subject page: trueno-gpu 0.4.17, ``src/kernels/backward/rms_norm.rs``, the
module documentation's "Mathematical Specification".  Per row of x (hidden
size H):

    forward:  rms = sqrt(mean_j(x_j^2) + eps),   y_i = x_i / rms * gamma_i
    dgamma_i = sum over rows of dy_i * x_i / rms

and the page predicts that the backward matches finite differences of that
forward.  Readings taken (the page is at odds with itself on the first):

* dx.  The page prints dx_i = gamma_i / rms * (dy_i - x_i / rms^2 * m) with
  m = mean_j(x_j dy_j gamma_j), which scales the correction term by gamma_i as
  well and matches finite differences only when gamma = 1.  The exact
  derivative of the stated forward is

      dx_i = (gamma_i dy_i - x_i / rms^2 * m) / rms,

  which is what the page's finite-difference prediction requires; it is what
  is computed here (and it equals the printed formula when gamma = 1).
* rms is the forward pass's value, which already contains eps; it is used as
  stored.  (The page's listing adds eps to its square a second time; the
  specification's formulas do not.)
"""

from __future__ import annotations

import numpy as np


def rms_norm_forward(x: np.ndarray, gamma: np.ndarray, eps: float):
    """(y, rms) in fp64 for x [rows][H], gamma [H]."""
    xd = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    rms = np.sqrt(np.mean(xd * xd, axis=1) + eps)
    return xd / rms[:, None] * g[None, :], rms


def rms_norm_backward(x: np.ndarray, gamma: np.ndarray, rms: np.ndarray, dy: np.ndarray):
    """(dx [rows][H], dgamma [H]) in fp64: the exact derivative of the forward, with the stored rms."""
    xd = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    r = np.asarray(rms, dtype=np.float64)[:, None]
    dyd = np.asarray(dy, dtype=np.float64)
    mean_term = np.mean(xd * dyd * g[None, :], axis=1, keepdims=True)
    dx = (g[None, :] * dyd - xd / (r * r) * mean_term) / r
    dgamma = np.sum(dyd * xd / r, axis=0)
    return dx, dgamma


def rms_norm_backward_bound(x: np.ndarray, gamma: np.ndarray, rms: np.ndarray, dy: np.ndarray):
    """Magnitude scales the acceptance bound is stated against: for dx the sum of the absolute values of
    the terms that form it, for dgamma the sum over rows of |dy x / rms|."""
    xd = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    r = np.asarray(rms, dtype=np.float64)[:, None]
    dyd = np.asarray(dy, dtype=np.float64)
    mean_abs = np.mean(np.abs(xd * dyd * g[None, :]), axis=1, keepdims=True)
    sx = (np.abs(g[None, :] * dyd) + np.abs(xd) / (r * r) * mean_abs) / r
    sg = np.sum(np.abs(dyd * xd / r), axis=0)
    return sx, sg
