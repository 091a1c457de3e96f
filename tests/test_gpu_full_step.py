"""GPU parity on the full-step workload at its real size: layer 0 of the 28-layer sweep.

The full step is 28 layers x 7 projections of a 7B-class decoder (hidden 3584,
KV dim 512, intermediate 18944) at M = 8192 tokens; every projection of layer
0 is checked here on EVERY element, in the launch plan nf4_grad_a picks for it
(the one the benchmark times), against the fp64 oracle at the bound
|gpu - ref| <= 2e-3 * S + 1e-6 and against the fp16-operand diagnostic.  The
grouped launch of the same layer is checked bitwise against separate launches
and against the oracle on sampled rows.

Inputs: weights N(0, 0.02) quantised by the oracle's pack on the CPU (seed
100 + projection index), grad_out N(0, 1e-2) (seed 200 + projection index).
"""

import functools

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

M_FULL = 8192
PROJ = [p for (p, _, _) in synth.FULL_STEP_PROJECTIONS]
SHAPE = {p: (n, k) for (p, n, k) in synth.FULL_STEP_PROJECTIONS}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@functools.lru_cache(maxsize=len(PROJ))
def layer0_weights(proj):
    N, K = SHAPE[proj]
    w = synth.weights_normal(N, K, seed=100 + PROJ.index(proj))
    return oracle.pack(w, N, K)


def layer0_grad_out(proj):
    N, _ = SHAPE[proj]
    return synth.grad_out_normal(M_FULL, N, seed=200 + PROJ.index(proj), std=1e-2)


def check_rows(gpu, g, w, rows, what):
    """Bound and fp16-operand diagnostic on `rows` (gpu holds exactly those rows)."""
    N = w.shape[0]
    ref, S = oracle.grad_a_from_weights(g, w, rows=rows)
    err = np.abs(gpu.astype(np.float64) - ref)
    lim = 2e-3 * S + 1e-6
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound; worst at {i}")
    assert np.all(np.isfinite(gpu)), what
    del ref, S, err, lim, bad
    ref16, S16 = oracle.grad_a_fp16_operands_from_weights(g, w, rows=rows)
    tol = (N / 8 + 64) * 2.0 ** -24 * S16 + 1e-30
    bad = np.abs(gpu.astype(np.float64) - ref16) > tol
    assert not bad.any(), f"{what}: fp16-operand diagnostic failed on {int(bad.sum())} elements"


@pytest.mark.parametrize("proj", PROJ)
def test_grad_a_full_step_layer0_every_element(lib, proj):
    N, K = SHAPE[proj]
    s, b = layer0_weights(proj)
    g = layer0_grad_out(proj)
    gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    torch.cuda.empty_cache()
    w = oracle.dequant(s, b, N, K)
    step = 4096
    for r0 in range(0, M_FULL, step):
        rows = np.arange(r0, min(M_FULL, r0 + step))
        check_rows(gpu[rows], g, w, rows, f"layer 0 {proj} rows {r0}..")


def test_grad_a_grouped_full_step_layer0(lib):
    """Layer 0's seven projections in one grouped call at M = 8192: bitwise equal to a separate launch of the
    same tiles (the fragment-fed wide kernel, one N-chunk) for each projection, and within the bound and
    the diagnostic on 16 sampled rows of each."""
    devs = []
    for p in PROJ:
        s, b = layer0_weights(p)
        devs.append((dev(layer0_grad_out(p)), dev(s), dev(b)))
    outs = lib.grad_a_grouped(devs)
    grouped = [host(o) for o in outs]
    del outs
    for p, d, gr in zip(PROJ, devs, grouped):
        sep = host(lib.grad_a_forced(*d, "wide16", rb=1, splits=1))
        assert np.array_equal(gr.view(np.uint32), sep.view(np.uint32)), p
    del devs
    torch.cuda.empty_cache()
    rng = np.random.default_rng(300)
    rows = np.unique(np.concatenate([[0, 511, 512, M_FULL - 1], rng.integers(0, M_FULL, size=12)]))
    for p, gr in zip(PROJ, grouped):
        N, K = SHAPE[p]
        s, b = layer0_weights(p)
        check_rows(gr[rows], layer0_grad_out(p), oracle.dequant(s, b, N, K), rows, f"grouped layer 0 {p}")
