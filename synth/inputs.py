"""Seeded random inputs (numpy PCG64).  No method arithmetic lives here.

Conventions
-----------
* ``grad_out`` is fp32 ``[M][N]`` row-major.
* ``weights`` are fp32 ``[N][K]`` row-major: the stored orientation of the
  frozen weight (out-features by in-features, the ``nn.Linear`` layout),
  i.e. the transpose of the logical ``B[K][N]`` of the forward product.
* ``code bytes`` are ``uint8 [N][K/2]``: two 4-bit codes per byte.  Drawing
  every byte uniformly in 0..255 draws every 4-bit code uniformly in 0..15,
  independently, whatever the nibble order.
* ``scales`` are fp32 ``[N][K/64]``.

"N(0, s)" in a workload description means a normal law with standard
deviation ``s``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Shape:
    """One input-gradient GEMM: grad_A[M x K] = grad_out[M x N] . W[N x K]."""

    name: str
    M: int
    N: int
    K: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> int:
        # grad_out fp32 + packed codes + fp32 scales + grad_A fp32
        return 4 * self.M * self.N + self.K * self.N // 2 + self.K * self.N // 16 + 4 * self.M * self.K


# The five workloads.  Seeds: the tiny case is seed 0; the others use the
# seeds listed per shape.
CONFIGS = {
    "tiny": [Shape("tiny", 64, 256, 256)],
    "attn_proj": [Shape("attn_proj", 2048, 1536, 1536)],
    "mlp_pair": [Shape("mlp_up_gate", 4096, 8960, 1536), Shape("mlp_down", 4096, 1536, 8960)],
}

# Skinny (decode-like) sweep: two weight shapes, three token counts.
SKINNY_SHAPES = [
    Shape(f"skinny_m{m}_{tag}", m, n, k)
    for (tag, k, n) in (("k3584_n18944", 3584, 18944), ("k18944_n3584", 18944, 3584))
    for m in (1, 8, 16)
]
CONFIGS["skinny"] = SKINNY_SHAPES

# Full training-step sweep: 28 layers x 7 projections of a 7B-class decoder
# (hidden 3584, KV dim 512, intermediate 18944), 8192 tokens.  For each
# projection N is its out-features and K its in-features.
FULL_STEP_LAYERS = 28
FULL_STEP_PROJECTIONS = [
    # name, N (out-features), K (in-features)
    ("q", 3584, 3584),
    ("k", 512, 3584),
    ("v", 512, 3584),
    ("o", 3584, 3584),
    ("gate", 18944, 3584),
    ("up", 18944, 3584),
    ("down", 3584, 18944),
]
CONFIGS["full_step"] = [Shape(f"full_step_{p}", 8192, n, k) for (p, n, k) in FULL_STEP_PROJECTIONS]


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def random_code_bytes(N: int, K: int, seed: int) -> np.ndarray:
    """uint8 [N][K/2], every byte uniform in 0..255 (so every code uniform in 0..15)."""
    return _rng(seed).integers(0, 256, size=(N, K // 2), dtype=np.uint8)


def random_scales_uniform(N: int, K: int, seed: int, lo: float = 0.01, hi: float = 0.1) -> np.ndarray:
    """fp32 [N][K/64], uniform in [lo, hi)."""
    return _rng(seed).uniform(lo, hi, size=(N, K // 64)).astype(np.float32)


def weights_normal(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """fp32 [N][K] weights ~ N(0, std)."""
    return _rng(seed).normal(0.0, std, size=(N, K)).astype(np.float32)


def grad_out_normal(M: int, N: int, seed: int, std: float = 1.0) -> np.ndarray:
    """fp32 [M][N] upstream gradient ~ N(0, std)."""
    return _rng(seed).normal(0.0, std, size=(M, N)).astype(np.float32)


def rms_norm_inputs(rows: int, H: int, seed: int):
    """RMSNorm backward inputs: x [rows][H] ~ N(0, 1), gamma [H] ~ U[0.5, 1.5), dy [rows][H] ~ N(0, 1), fp32.

    Draw order x, gamma, dy from one stream.  (The per-row rms is the forward pass's, computed by whoever
    consumes these.)
    """
    rng = _rng(seed)
    x = rng.normal(0.0, 1.0, size=(rows, H)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=(H,)).astype(np.float32)
    dy = rng.normal(0.0, 1.0, size=(rows, H)).astype(np.float32)
    return x, gamma, dy


# RMSNorm backward workloads: the decoder's hidden size over the full step's 8192 tokens, the
# attention-projection width, and the subject page's own (rows, hidden) test sizes.
RMS_NORM_SHAPES = [(8192, 3584), (8192, 1536), (64, 32), (128, 16)]


def tiny_inputs(seed: int = 0):
    """The tiny workload: random codes, scales U[0.01, 0.1), grad_out N(0, 1).

    Draw order is codes, then scales, then grad_out, all from one stream.
    """
    s = CONFIGS["tiny"][0]
    rng = _rng(seed)
    codes = rng.integers(0, 256, size=(s.N, s.K // 2), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.1, size=(s.N, s.K // 64)).astype(np.float32)
    g = rng.normal(0.0, 1.0, size=(s.M, s.N)).astype(np.float32)
    return g, scales, codes
