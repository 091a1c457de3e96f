"""GPU parity of the RMSNorm backward nf4_rms_norm_backward against the CPU oracle.

Inputs: x ~ N(0, 1), gamma ~ U[0.5, 1.5), dy ~ N(0, 1); rms is the forward
pass's sqrt(mean(x^2) + eps) from the oracle's fp64 forward, rounded to fp32
and handed to both sides.  The HIP path works in fp32 with fixed summation
orders, so each output is accepted against the fp64 oracle at

  dx:     (H/64 + 32) * 2^-24 * sx   (per-thread partial sums of at most
                                       H/256 terms, a 6-level butterfly, a
                                       4-wave sum, a handful of rounded
                                       products and the division)
  dgamma: (ceil(rows / 256) + 72) * 2^-24 * sg   (a run of rows per
                                       workgroup, at most 512 workgroup
                                       partials added in 16 runs of 32 and
                                       the 16 runs, three rounded products)

where sx, sg are the sums of the absolute values of the terms that form each
output (oracle.rms_norm_backward_bound).
"""

import math

import numpy as np
import pytest

import synth
from oracle import rms_norm_oracle as ro

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def make_case(rows, H, seed, eps=1e-5):
    x, gamma, dy = synth.rms_norm_inputs(rows, H, seed)
    _, rms = ro.rms_norm_forward(x, gamma, eps)
    return x, gamma, rms.astype(np.float32), dy


def check(lib, rows, H, seed, eps=1e-5, what=""):
    x, gamma, rms, dy = make_case(rows, H, seed, eps)
    dx, dg = lib.rms_norm_backward(dev(x), dev(gamma), dev(rms), dev(dy))
    dx, dg = host(dx), host(dg)
    ref_dx, ref_dg = ro.rms_norm_backward(x, gamma, rms, dy)
    sx, sg = ro.rms_norm_backward_bound(x, gamma, rms, dy)
    lim_x = (H / 64 + 32) * 2.0 ** -24 * sx + 1e-30
    lim_g = (math.ceil(rows / 256) + 72) * 2.0 ** -24 * sg + 1e-30
    ex = np.abs(dx.astype(np.float64) - ref_dx)
    eg = np.abs(dg.astype(np.float64) - ref_dg)
    if (ex > lim_x).any():
        i = np.unravel_index(np.argmax(ex / lim_x), ex.shape)
        raise AssertionError(f"{what}: dx {int((ex > lim_x).sum())} out of bound; worst at {i}: "
                             f"gpu={dx[i]!r} ref={ref_dx[i]!r} lim={lim_x[i]!r}")
    if (eg > lim_g).any():
        i = int(np.argmax(eg / lim_g))
        raise AssertionError(f"{what}: dgamma {int((eg > lim_g).sum())} out of bound; worst at {i}: "
                             f"gpu={dg[i]!r} ref={ref_dg[i]!r} lim={lim_g[i]!r}")
    assert np.all(np.isfinite(dx)) and np.all(np.isfinite(dg))
    return dx, dg


@pytest.mark.parametrize("rows,H", [(1, 4), (3, 32), (7, 100), (5, 252), (1000, 1536), (1025, 3584),
                                    (300, 8192), (4096, 260), (2050, 7168), (65536, 64)])
def test_rms_norm_backward_shapes(lib, rows, H):
    """One to eight float4 chunks per thread (H up to 8192); rows below, at and far above the 512
    workgroups of the grid (1 to 128 rows each); H not a multiple of 1024 (threads past the row idle)."""
    check(lib, rows, H, seed=rows * 7 + H, what=f"rms {rows}x{H}")


@pytest.mark.parametrize("rows,H,eps", [(64, 32, 1e-6), (128, 16, 1e-5)])
def test_rms_norm_backward_page_sizes(lib, rows, H, eps):
    """The subject page's own kernel sizes (rows, hidden, eps)."""
    check(lib, rows, H, seed=rows + H, eps=eps, what=f"rms page {rows}x{H}")


@pytest.mark.parametrize("rows,H", [(8192, 3584), (8192, 1536)])
def test_rms_norm_backward_full_step_shapes(lib, rows, H):
    """The decoder's hidden size and the attention-projection width over 8192 tokens, in the launch
    configuration the benchmark times; every output checked."""
    check(lib, rows, H, seed=H, what=f"rms full {rows}x{H}")


def test_rms_norm_backward_unit_gamma_matches_printed_formula(lib):
    """At gamma = 1 the page's printed dx formula and the exact derivative coincide."""
    rows, H = 96, 512
    x, _, rms, dy = make_case(rows, H, seed=3)
    gamma = np.ones(H, dtype=np.float32)
    dx, _ = lib.rms_norm_backward(dev(x), dev(gamma), dev(rms), dev(dy))
    dx = host(dx).astype(np.float64)
    xd, dyd, r = x.astype(np.float64), dy.astype(np.float64), rms.astype(np.float64)[:, None]
    m = np.mean(xd * dyd, axis=1, keepdims=True)
    printed = 1.0 / r * (dyd - xd / (r * r) * m)
    sx, _ = ro.rms_norm_backward_bound(x, gamma, rms, dy)
    assert np.all(np.abs(dx - printed) <= (H / 64 + 32) * 2.0 ** -24 * sx)


def test_rms_norm_backward_deterministic(lib):
    x, gamma, rms, dy = make_case(3000, 2048, seed=5)
    args = (dev(x), dev(gamma), dev(rms), dev(dy))
    a = [host(t) for t in lib.rms_norm_backward(*args)]
    b = [host(t) for t in lib.rms_norm_backward(*args)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_rms_norm_backward_zero_dy(lib):
    x, gamma, rms, _ = make_case(40, 96, seed=6)
    dy = np.zeros_like(x)
    dx, dg = lib.rms_norm_backward(dev(x), dev(gamma), dev(rms), dev(dy))
    assert np.all(host(dx) == 0.0) and np.all(host(dg) == 0.0)


def test_rms_norm_backward_empty_and_rejected(lib):
    gamma = dev(np.ones(64, dtype=np.float32))
    # rows == 0: dgamma is an empty sum
    dg = dev(np.full(64, 5.0, dtype=np.float32))
    e = dev(np.zeros((0, 64), dtype=np.float32))
    lib.rms_norm_backward(e, gamma, dev(np.zeros(0, dtype=np.float32)), e, dx=e, dgamma=dg)
    assert np.all(host(dg) == 0.0)
    # H % 4 != 0 and H > 8192 are rejected before any launch
    for H in (6, 8196):
        x = dev(np.ones((2, H), dtype=np.float32))
        with pytest.raises(lib.Nf4Error):
            lib.rms_norm_backward(x, dev(np.ones(H, dtype=np.float32)), dev(np.ones(2, dtype=np.float32)), x)
