"""Plain CPU oracle (numpy, fp64) for the NF4-dequant-fused input-gradient GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant with the HIP library; its codebook is its own literal copy.

What is computed (subject page: aprender-gpu 0.32.0,
``src/kernels/backward/nf4_tensor_core.rs``, the doc comment of
``Nf4TensorCoreGemmBackwardAKernel`` and its four phases):

    grad_A[M x K] = grad_out[M x N] . dequant(B_nf4[K x N])^T

The packed weight is stored per out-feature ``n``: its K codes are
contiguous, two per byte, low nibble first, and there is one fp32 scale per
(n, 64-wide block of k) (Phase 2, "NF4 addressing": block index k/64, scale
at n*(K/64) + k/64, byte at n*(K/64)*32 + (k/64)*32 + (k%64)/2, nibble
shift 4*(k%2)).  So the stored array is W = B^T, N x K row-major.

Each element is decoded as one fp32 multiply, scale times the codebook value
(Phase 2, "NF4 LUT lookup + dequant").  Because the product of two fp32
numbers has at most 48 significant bits it is exact in fp64, and one cast to
fp32 then rounds it once: the oracle's dequant is bit-identical to the
single fp32 multiply.

grad_A is the definition itself: an fp64 matmul of grad_out and the fp32
dequantised weights.  The forward product of the same layer (the page's header
comment: C = A @ B over the shared dimension K) is likewise the definition,
C = A . W^T in fp64.  The companion ``S[m][k] = sum_n |g[m][n] * w[n][k]|``
is the scale the acceptance bound is stated against.

Readings taken where the page is silent (each listed in the design notes):

* codebook values: the QLoRA NormalFloat-4 table (Dettmers et al., 2023,
  "QLoRA: Efficient Finetuning of Quantized LLMs", arXiv:2305.14314), code 7
  is 0.0 and code 15 is 1.0; the page only imports it;
* scale semantics: the block's absolute maximum, stored as is;
* quantiser: nearest level to w/absmax, ties to the lower code; an all-zero
  block gets scale 0 and code 7;
* fp32 -> fp16 conversions round to nearest even.

Every function here is pinned by a CPU test against something other than
itself (closed forms, brute force, exact rational arithmetic, the quantile
construction of the codebook).
"""

from __future__ import annotations

import math

import numpy as np

NF4_BLOCK = 64

# The 16 NormalFloat-4 levels as exact fp32 values (hex).  Code 7 is 0.0,
# code 0 is -1.0 and code 15 is 1.0.
_NF4_HEX = (
    "-0x1.000000p+0",
    "-0x1.647362p-1",
    "-0x1.0cd660p-1",
    "-0x1.946540p-2",
    "-0x1.23449ap-2",
    "-0x1.7a6a7ep-3",
    "-0x1.74f0e2p-4",
    "0x0p+0",
    "0x1.45f5fep-4",
    "0x1.4995c6p-3",
    "0x1.f809bap-3",
    "0x1.5a0674p-2",
    "0x1.c34970p-2",
    "0x1.200f56p-1",
    "0x1.722766p-1",
    "0x1.000000p+0",
)
NF4_LEVELS = np.array([float.fromhex(h) for h in _NF4_HEX], dtype=np.float32)


def num_k_blocks(K: int) -> int:
    """Number of 64-wide scale blocks along K (the page's ``num_k_blocks``)."""
    return K // NF4_BLOCK


def codebook_from_quantiles() -> np.ndarray:
    """The NF4 levels rebuilt from their definition (fp64), for pinning.

    QLoRA builds the 4-bit NormalFloat levels from standard-normal quantiles:
    with offset d = 1 - (1/32 + 1/30)/2, take 8 positive quantiles at evenly
    spaced probabilities from d down to 1/2 (excluding 1/2), 7 negative ones
    the same way, add an exact zero, sort, and divide by the largest.
    """
    from statistics import NormalDist

    nd = NormalDist()
    d = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    pos = [nd.inv_cdf(p) for p in np.linspace(d, 0.5, 9)[:-1]]
    neg = [-nd.inv_cdf(p) for p in np.linspace(d, 0.5, 8)[:-1]]
    vals = np.array(sorted(pos + neg + [0.0]), dtype=np.float64)
    return vals / vals.max()


def unpack_codes(code_bytes: np.ndarray, N: int, K: int) -> np.ndarray:
    """uint8 [N][K/2] packed bytes -> uint8 [N][K] codes; even k is the low nibble."""
    b = np.asarray(code_bytes, dtype=np.uint8).reshape(N, K // 2)
    out = np.empty((N, K), dtype=np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [N][K] codes (0..15) -> uint8 [N][K/2] bytes, even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def dequant(scales: np.ndarray, code_bytes: np.ndarray, N: int, K: int) -> np.ndarray:
    """fp32 [N][K] weights: w[n][k] = fl32(scale[n][k/64] * level[code(n, k)])."""
    codes = unpack_codes(code_bytes, N, K)
    s = np.asarray(scales, dtype=np.float32).reshape(N, K // NF4_BLOCK).astype(np.float64)
    q = NF4_LEVELS.astype(np.float64)[codes]
    return (np.repeat(s, NF4_BLOCK, axis=1) * q).astype(np.float32)


def dequant_columns(scales: np.ndarray, code_bytes: np.ndarray, N: int, K: int, cols: np.ndarray) -> np.ndarray:
    """fp32 [N][len(cols)]: the columns k in `cols` of dequant(), from the same definition -- code(n, k) is
    the low nibble of byte k/2 of row n for even k, the high nibble for odd k; w = fl32(scale[n][k/64] *
    level[code]) -- without unpacking the other columns (for weights too large to dequantise whole)."""
    c = np.asarray(cols, dtype=np.int64)
    b = np.asarray(code_bytes, dtype=np.uint8).reshape(N, K // 2)[:, c // 2]
    codes = np.where((c % 2) == 0, b & 0x0F, b >> 4)
    s = np.asarray(scales, dtype=np.float32).reshape(N, K // NF4_BLOCK)[:, c // NF4_BLOCK].astype(np.float64)
    return (s * NF4_LEVELS.astype(np.float64)[codes]).astype(np.float32)


def grad_a(grad_out: np.ndarray, scales: np.ndarray, code_bytes: np.ndarray, M: int, N: int, K: int,
           rows: np.ndarray | None = None, with_bound: bool = True, cols: np.ndarray | None = None):
    """fp64 grad_A and its bound scale S for the given (or all) rows and columns.

    ref[m][k] = sum_n g[m][n] * w[n][k];  S[m][k] = sum_n |g[m][n] * w[n][k]|.
    """
    if cols is None:
        w = dequant(scales, code_bytes, N, K)
    else:
        w = dequant_columns(scales, code_bytes, N, K, cols)
    g = np.asarray(grad_out, dtype=np.float32).reshape(M, N)
    return grad_a_from_weights(g, w, rows=rows, with_bound=with_bound)


def grad_a_from_weights(grad_out: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None,
                        with_bound: bool = True):
    """grad_a() with the fp32 weights already dequantised (w = dequant(...), [N][K'] for any column set).

    ref[m][k] = sum_n g[m][n] * w[n][k] in fp64;  S[m][k] = sum_n |g[m][n] * w[n][k]|.
    """
    wd = np.asarray(w, dtype=np.float32).astype(np.float64)
    g = np.asarray(grad_out, dtype=np.float32)
    if g.ndim != 2 or g.shape[1] != wd.shape[0]:
        raise ValueError(f"grad_out must be [M][N] with N = {wd.shape[0]}, got shape {g.shape}")
    if rows is not None:
        g = g[np.asarray(rows)]
    g = g.astype(np.float64)
    ref = g @ wd
    if not with_bound:
        return ref
    return ref, np.abs(g) @ np.abs(wd)


def forward(a: np.ndarray, scales: np.ndarray, code_bytes: np.ndarray, M: int, N: int, K: int,
            rows: np.ndarray | None = None, with_bound: bool = True):
    """fp64 forward product of the same frozen layer and its bound scale S.

    The subject page's header comment states the forward this backward kernel
    is the analog of: C = A @ B with the shared dimension K, B_nf4 being
    K x N.  With the stored W = B^T (N x K):

        C[m][n] = sum_k a[m][k] * w[n][k];  S[m][n] = sum_k |a[m][k] * w[n][k]|.
    """
    w = dequant(scales, code_bytes, N, K).astype(np.float64)
    x = np.asarray(a, dtype=np.float32).reshape(M, K)
    if rows is not None:
        x = x[np.asarray(rows)]
    x = x.astype(np.float64)
    ref = x @ w.T
    if not with_bound:
        return ref
    return ref, np.abs(x) @ np.abs(w).T


def grad_a_fp16_operands(grad_out: np.ndarray, scales: np.ndarray, code_bytes: np.ndarray,
                         M: int, N: int, K: int, rows: np.ndarray | None = None):
    """Diagnostic: sum_n fp16(g) * fp16(w) in fp64 (both operands rounded to fp16, RNE).

    This is what an fp16-operand product computes before accumulation error;
    it is not a gate, it exposes wrong operand rounding that the loose bound
    would hide.
    """
    g = np.asarray(grad_out, dtype=np.float32).reshape(M, N)
    return grad_a_fp16_operands_from_weights(g, dequant(scales, code_bytes, N, K), rows=rows)


def grad_a_fp16_operands_from_weights(grad_out: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None):
    """grad_a_fp16_operands() with the fp32 weights already dequantised (w = dequant(...), [N][K]).

    Returns (sum_n fp16(g) * fp16(w), sum_n |fp16(g) * fp16(w)|), fp64, fp16() round-to-nearest-even.
    """
    w16 = np.asarray(w, dtype=np.float32).astype(np.float16).astype(np.float64)
    g = np.asarray(grad_out, dtype=np.float32)
    if g.ndim != 2 or g.shape[1] != w16.shape[0]:
        raise ValueError(f"grad_out must be [M][N] with N = {w16.shape[0]}, got shape {g.shape}")
    if rows is not None:
        g = g[np.asarray(rows)]
    g16 = g.astype(np.float16).astype(np.float64)
    return g16 @ w16, np.abs(g16) @ np.abs(w16)


def grad_a_bruteforce(grad_out: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Correctly rounded sum_n g*w for tiny shapes (pure Python, math.fsum).

    Each product of two fp32 values is exact in fp64 and fsum rounds the
    exact sum once, so this is the exact result rounded to fp64.
    """
    g = np.asarray(grad_out, dtype=np.float64)
    wd = np.asarray(w, dtype=np.float64)
    M, N = g.shape
    K = wd.shape[1]
    out = np.empty((M, K), dtype=np.float64)
    for m in range(M):
        for k in range(K):
            out[m, k] = math.fsum(float(g[m, n]) * float(wd[n, k]) for n in range(N))
    return out


def _midpoints() -> np.ndarray:
    """Midpoints between consecutive levels, exact in fp64 (at most 25 significant bits)."""
    q = NF4_LEVELS.astype(np.float64)
    return (q[:-1] + q[1:]) * 0.5


def pack(w: np.ndarray, N: int, K: int, chunk_rows: int = 1024):
    """Quantise fp32 [N][K] weights to NF4: (scales fp32 [N][K/64], code bytes uint8 [N][K/2]).

    Per (n, 64-block): scale = absmax of the block; code = nearest level to
    w/absmax with ties to the lower code, decided exactly as
    code = #{i : w > absmax * mid_i} in fp64 (each product has at most 49
    significant bits, so it and the comparison are exact).  An all-zero block
    gets scale 0 and code 7 (level 0.0).
    """
    w = np.asarray(w, dtype=np.float32).reshape(N, K)
    nb = K // NF4_BLOCK
    scales = np.empty((N, nb), dtype=np.float32)
    codes = np.empty((N, K), dtype=np.uint8)
    mids = _midpoints()
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        blk = w[r0:r1].reshape(r1 - r0, nb, NF4_BLOCK)
        absmax = np.max(np.abs(blk), axis=2)
        scales[r0:r1] = absmax
        a = absmax.astype(np.float64)[..., None]
        x = blk.astype(np.float64)
        c = np.zeros(blk.shape, dtype=np.uint8)
        for m in mids:
            c += (x > a * m)
        c[np.broadcast_to(absmax[..., None] == 0, c.shape)] = 7
        codes[r0:r1] = c.reshape(r1 - r0, K)
    return scales, pack_codes(codes)
