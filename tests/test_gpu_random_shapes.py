"""Seeded random shapes across every planner regime (M from 1 to ~1200, N ragged, K any multiple of 64):
nf4_grad_a (default plan) and nf4_forward against the oracle, element by element, with the bound and the
fp16-operand diagnostic; the plan taken is printed on failure.  NF4_SHAPE_SEED (an integer) draws the
same number of shapes from other seeds, for wider sweeps run by hand; the default seeds are the committed
cases."""

import os

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 300)), int(rng.integers(300, 1200))]))
        N = int(rng.integers(1, 3000))
        K = 64 * int(rng.integers(1, 40))
        out.append((M, N, K))
    return out


_SEED = int(os.environ.get("NF4_SHAPE_SEED", "0"))
SHAPES = _shapes(36, seed=2024 + 1000 * _SEED)


def _tile_shapes(count, seed):
    """N a multiple of 64 and M > 16, so that the planner's tile kernels (512 x 128, 256 x 128, 128 x 128, split
    or not, fp16-fragment-fed or fp32-fed) are what the default plans pick; every fourth shape at M >= 4000."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        if i % 4 == 3:
            M, N = int(rng.integers(4000, 6200)), 64 * int(rng.integers(24, 49))
        else:
            M, N = int(rng.integers(17, 2600)), 64 * int(rng.integers(1, 49))
        out.append((M, N, 64 * int(rng.integers(1, 41))))
    return out


TILE_SHAPES = _tile_shapes(20, seed=2025 + 1000 * _SEED)


def _check(gpu, ref, S, ref16, S16, red, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    lim = 2e-3 * S + 1e-6
    assert np.all(err <= lim), f"{what}: {int((err > lim).sum())} out of bound"
    tol = (red / 8 + 64) * 2.0 ** -24 * S16 + 1e-30
    assert np.all(np.abs(gpu.astype(np.float64) - ref16) <= tol), f"{what}: fp16-operand diagnostic"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_grad_a_random_shape(lib, M, N, K):
    seed = M * 7919 + N * 31 + K
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    gpu = lib.grad_a(dev(g), dev(s), dev(b)).cpu().numpy()
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    ref16, S16 = oracle.grad_a_fp16_operands(g, s, b, M, N, K)
    _check(gpu, ref, S, ref16, S16, N, f"grad_a {M}x{N}x{K} plan {lib.grad_a_plan(M, N, K)}")


@pytest.mark.parametrize("M,N,K", [(M, 8 * (-(-N // 8)), K) for (M, N, K) in SHAPES[:18]])
def test_forward_random_shape(lib, M, N, K):
    seed = M * 104729 + N * 17 + K
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    a = synth.grad_out_normal(M, K, seed + 2)
    gpu = lib.forward(dev(a), dev(s), dev(b)).cpu().numpy()
    ref, S = oracle.forward(a, s, b, M, N, K)
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float64)
    a16 = a.astype(np.float16).astype(np.float64)
    _check(gpu, ref, S, a16 @ w16.T, np.abs(a16) @ np.abs(w16).T, K, f"forward {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_grad_a_random_tile_shape(lib, M, N, K):
    seed = M * 6151 + N * 37 + K
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    gpu = lib.grad_a(dev(g), dev(s), dev(b)).cpu().numpy()
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    ref16, S16 = oracle.grad_a_fp16_operands(g, s, b, M, N, K)
    _check(gpu, ref, S, ref16, S16, N, f"grad_a {M}x{N}x{K} plan {lib.grad_a_plan(M, N, K)}")


@pytest.mark.parametrize("M,N,K", TILE_SHAPES[:10])
def test_forward_random_tile_shape(lib, M, N, K):
    seed = M * 7927 + N * 13 + K
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    a = synth.grad_out_normal(M, K, seed + 2)
    gpu = lib.forward(dev(a), dev(s), dev(b)).cpu().numpy()
    ref, S = oracle.forward(a, s, b, M, N, K)
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float64)
    a16 = a.astype(np.float16).astype(np.float64)
    _check(gpu, ref, S, a16 @ w16.T, np.abs(a16) @ np.abs(w16).T, K, f"forward {M}x{N}x{K}")

