"""Pins for the CPU oracle: each test checks it against something other than itself.

All of these run on the CPU (no GPU marker).  A plausible mistake in the
oracle -- a dropped term, a wrong sign, a swapped nibble, a transposed
operand, a wrong scale index -- fails at least one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- codebook

def test_codebook_matches_quantile_construction():
    """The literal table equals the QLoRA quantile construction to fp32 precision."""
    built = oracle.codebook_from_quantiles()
    diff = np.max(np.abs(oracle.NF4_LEVELS.astype(np.float64) - built))
    assert diff <= 5e-7, diff


def test_codebook_fixed_points_and_order():
    q = oracle.NF4_LEVELS
    assert q.dtype == np.float32 and q.shape == (16,)
    assert q[0] == -1.0 and q[7] == 0.0 and q[15] == 1.0
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    assert np.sum(q < 0) == 7 and np.sum(q > 0) == 8


def test_num_k_blocks_page_value():
    with open(os.path.join(GOLDEN, "page_shapes.json")) as f:
        gold = json.load(f)
    for K, nb in gold["num_k_blocks"]:
        assert oracle.num_k_blocks(K) == nb


# ----------------------------------------------------------- layout / unpack

def _layout_example():
    with open(os.path.join(GOLDEN, "nibble_layout_example.json")) as f:
        gold = json.load(f)
    N, K = gold["N"], gold["K"]
    flat = np.full(N * K // 2, gold["bytes_default"], dtype=np.uint8)
    for idx, val in gold["bytes_set"].items():
        flat[int(idx)] = val
    return gold, N, K, flat.reshape(N, K // 2)


def test_unpack_matches_hand_worked_addressing():
    gold, N, K, b = _layout_example()
    codes = oracle.unpack_codes(b, N, K)
    for key, want in gold["expected_codes_at"].items():
        n, k = key.split("_")
        assert codes[int(n[1:]), int(k[1:])] == want, key


def test_pack_codes_inverts_unpack():
    b = synth.random_code_bytes(5, 192, seed=3)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(b, 5, 192)), b)


def test_dequant_nibble_order_probe():
    """Even-k nibble 15 and odd-k nibble 7 dequantise to s, 0, s, 0, ..."""
    N, K = 3, 128
    b = np.full((N, K // 2), 0x7F, dtype=np.uint8)
    s = np.array([[0.5, 2.0], [4.0, 0.25], [1.0, 8.0]], dtype=np.float32)
    w = oracle.dequant(s, b, N, K)
    for n in range(N):
        for k in range(K):
            want = s[n, k // 64] if k % 2 == 0 else 0.0
            assert w[n, k] == want


def test_dequant_scale_index_probe():
    """Distinct power-of-two scales per (n, block) with all codes 15 reveal the scale map."""
    N, K = 4, 256
    s = np.array([[2.0 ** (n * 4 + kb - 8) for kb in range(4)] for n in range(N)], dtype=np.float32)
    b = np.full((N, K // 2), 0xFF, dtype=np.uint8)
    w = oracle.dequant(s, b, N, K)
    for n in range(N):
        for k in range(K):
            assert w[n, k] == 2.0 ** (n * 4 + k // 64 - 8)


def test_dequant_columns_probes_and_agreement():
    """Column-sampled dequant: the nibble-order and scale-index probes on odd and even sampled columns, and
    bitwise agreement with the full dequant's columns (and grad_a's) on random inputs."""
    N, K = 4, 256
    s = np.array([[2.0 ** (n * 4 + kb - 8) for kb in range(4)] for n in range(N)], dtype=np.float32)
    b = np.full((N, K // 2), 0x7F, dtype=np.uint8)  # even k -> code 15, odd k -> code 7
    cols = np.array([0, 1, 63, 64, 130, 255])
    w = oracle.dequant_columns(s, b, N, K, cols)
    for n in range(N):
        for j, k in enumerate(cols):
            assert w[n, j] == (2.0 ** (n * 4 + k // 64 - 8) if k % 2 == 0 else 0.0)
    N, K = 29, 448
    b = synth.random_code_bytes(N, K, seed=21)
    s = synth.random_scales_uniform(N, K, seed=22)
    cols = np.random.default_rng(23).choice(K, size=40, replace=False)
    assert np.array_equal(oracle.dequant_columns(s, b, N, K, cols).view(np.uint32),
                          oracle.dequant(s, b, N, K)[:, cols].view(np.uint32))
    g = synth.grad_out_normal(5, N, seed=24)
    ref, S = oracle.grad_a(g, s, b, 5, N, K)
    ref_c, S_c = oracle.grad_a(g, s, b, 5, N, K, cols=cols)
    assert np.array_equal(ref_c, ref[:, cols]) and np.array_equal(S_c, S[:, cols])


def test_dequant_is_one_fp32_multiply():
    """Bit-identical to an IEEE fp32 multiply done in float32 arithmetic."""
    N, K = 37, 320
    b = synth.random_code_bytes(N, K, seed=11)
    s = synth.random_scales_uniform(N, K, seed=12, lo=1e-3, hi=3.0)
    w = oracle.dequant(s, b, N, K)
    codes = np.empty((N, K), dtype=np.int64)
    for n in range(N):                      # independent unpack: Python integer ops per byte
        for i in range(K // 2):
            v = int(b[n, i])
            codes[n, 2 * i] = v % 16
            codes[n, 2 * i + 1] = v // 16
    q32 = oracle.NF4_LEVELS[codes]
    s32 = np.repeat(s, 64, axis=1)
    with np.errstate(all="raise"):
        direct = np.multiply(s32, q32, dtype=np.float32)
    assert np.array_equal(w.view(np.uint32), direct.view(np.uint32))


# ----------------------------------------------------------------- grad_A

@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 64, 0), (3, 5, 64, 1), (4, 17, 128, 2), (2, 33, 192, 3)])
def test_grad_a_matches_fsum_bruteforce(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 100)
    g = synth.grad_out_normal(M, N, seed + 200)
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    w = oracle.dequant(s, b, N, K)
    exact = oracle.grad_a_bruteforce(g, w)
    assert np.all(np.abs(ref - exact) <= 1e-12 * S + 1e-300)
    # S itself: brute-force sum of absolute products
    S_bf = oracle.grad_a_bruteforce(np.abs(g), np.abs(w))
    assert np.allclose(S, S_bf, rtol=1e-13, atol=0)


def test_grad_a_single_weight_probe():
    """One nonzero weight at (n0, k0) moves column n0 of grad_out into column k0 of grad_A."""
    M, N, K = 3, 5, 128
    n0, k0 = 3, 70
    b = np.full((N, K // 2), 0x77, dtype=np.uint8)         # all codes 7 -> 0.0
    byte = b[n0, k0 // 2]
    b[n0, k0 // 2] = (byte & 0xF0) | 15 if k0 % 2 == 0 else (byte & 0x0F) | (15 << 4)
    s = np.full((N, K // 64), 0.75, dtype=np.float32)
    g = synth.grad_out_normal(M, N, seed=5)
    ref, _ = oracle.grad_a(g, s, b, M, N, K)
    want = np.zeros((M, K))
    want[:, k0] = g[:, n0].astype(np.float64) * 0.75
    assert np.array_equal(ref, want)


def test_grad_a_one_hot_rows_reproduce_dequant_rows():
    M, N, K = 6, 9, 192
    b = synth.random_code_bytes(N, K, seed=21)
    s = synth.random_scales_uniform(N, K, seed=22)
    g = np.zeros((M, N), dtype=np.float32)
    picks = [0, 8, 3, 3, 5, 1]
    for m, n in enumerate(picks):
        g[m, n] = 1.0
    ref, _ = oracle.grad_a(g, s, b, M, N, K)
    w = oracle.dequant(s, b, N, K)
    for m, n in enumerate(picks):
        assert np.array_equal(ref[m], w[n].astype(np.float64))


def test_grad_a_adjoint_identity():
    """<grad_A, A> = <grad_out, A . W^T> with (A . W^T)[m][n] = sum_k A[m][k] W[n][k]."""
    M, N, K = 7, 48, 256
    b = synth.random_code_bytes(N, K, seed=31)
    s = synth.random_scales_uniform(N, K, seed=32)
    g = synth.grad_out_normal(M, N, seed=33)
    A = synth.grad_out_normal(M, K, seed=34)
    ref, _ = oracle.grad_a(g, s, b, M, N, K)
    w = oracle.dequant(s, b, N, K).astype(np.float64)
    fwd = np.einsum("mk,nk->mn", A.astype(np.float64), w)
    lhs = np.sum(ref * A)
    rhs = np.sum(g.astype(np.float64) * fwd)
    assert abs(lhs - rhs) <= 1e-11 * (np.sum(np.abs(ref * A)) + 1.0)


def test_grad_a_special_cases():
    M, N, K = 5, 40, 128
    g = synth.grad_out_normal(M, N, seed=41)
    # all codes 7 -> level 0 -> grad_A identically zero
    b7 = np.full((N, K // 2), 0x77, dtype=np.uint8)
    s = synth.random_scales_uniform(N, K, seed=42)
    ref, _ = oracle.grad_a(g, s, b7, M, N, K)
    assert np.all(ref == 0.0)
    # unit scales, all codes 15 -> every column is the row sum of grad_out
    bF = np.full((N, K // 2), 0xFF, dtype=np.uint8)
    ones = np.ones((N, K // 64), dtype=np.float32)
    ref, _ = oracle.grad_a(g, ones, bF, M, N, K)
    rs = np.sum(g.astype(np.float64), axis=1)
    assert np.allclose(ref, np.repeat(rs[:, None], K, axis=1), rtol=1e-14, atol=1e-14)
    # unit scales, random codes -> sum over levels of level * (grad_out @ one-hot(code == level))
    b = synth.random_code_bytes(N, K, seed=43)
    ref, _ = oracle.grad_a(g, ones, b, M, N, K)
    lo = (b & 0x0F).astype(np.int64)
    hi = (b >> 4).astype(np.int64)
    alt = np.zeros((M, K))
    for v in range(16):
        onehot = np.zeros((N, K))
        onehot[:, 0::2] = lo == v
        onehot[:, 1::2] = hi == v
        alt += float(oracle.NF4_LEVELS[v]) * (g.astype(np.float64) @ onehot)
    assert np.allclose(ref, alt, rtol=1e-12, atol=1e-12)
    # N = 0: the empty sum, zeros of shape M x K, in both the definition and the fp16-operand reference
    g0 = np.zeros((M, 0), dtype=np.float32)
    s0 = np.zeros((0, K // 64), dtype=np.float32)
    b0 = np.zeros((0, K // 2), dtype=np.uint8)
    for fn in (oracle.grad_a, oracle.grad_a_fp16_operands):
        ref, S = fn(g0, s0, b0, M, 0, K)
        assert ref.shape == (M, K) and np.all(ref == 0.0) and np.all(S == 0.0)


# ----------------------------------------------------------------- forward C = A . W^T

@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 64, 0), (3, 5, 64, 1), (4, 17, 128, 2), (2, 9, 192, 3)])
def test_forward_matches_fsum_bruteforce(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed + 50)
    s = synth.random_scales_uniform(N, K, seed + 150)
    a = synth.grad_out_normal(M, K, seed + 250)
    ref, S = oracle.forward(a, s, b, M, N, K)
    w = oracle.dequant(s, b, N, K).astype(np.float64)
    ad = a.astype(np.float64)
    for m in range(M):
        for n in range(N):
            exact = math.fsum(float(ad[m, k]) * float(w[n, k]) for k in range(K))
            bound = math.fsum(abs(float(ad[m, k]) * float(w[n, k])) for k in range(K))
            assert abs(ref[m, n] - exact) <= 1e-12 * bound + 1e-300
            assert abs(S[m, n] - bound) <= 1e-13 * bound


def test_forward_one_hot_rows_pick_weight_columns():
    """A row of A that is e_k0 gives the dequantised column k0 of W (every out-feature's weight at k0)."""
    M, N, K = 5, 11, 192
    b = synth.random_code_bytes(N, K, seed=61)
    s = synth.random_scales_uniform(N, K, seed=62)
    a = np.zeros((M, K), dtype=np.float32)
    picks = [0, 63, 64, 191, 100]
    for m, k in enumerate(picks):
        a[m, k] = 1.0
    ref, _ = oracle.forward(a, s, b, M, N, K)
    w = oracle.dequant(s, b, N, K)
    for m, k in enumerate(picks):
        assert np.array_equal(ref[m], w[:, k].astype(np.float64))


def test_forward_is_the_adjoint_of_grad_a():
    """<forward(A), X> = <A, grad_a(X)>: the two oracles contract the same weights over different
    dimensions, so a transposed operand or a swapped dimension in either breaks this."""
    M, N, K = 6, 40, 256
    b = synth.random_code_bytes(N, K, seed=71)
    s = synth.random_scales_uniform(N, K, seed=72)
    a = synth.grad_out_normal(M, K, seed=73)
    x = synth.grad_out_normal(M, N, seed=74)
    c, _ = oracle.forward(a, s, b, M, N, K)
    ga, _ = oracle.grad_a(x, s, b, M, N, K)
    lhs = np.sum(c * x.astype(np.float64))
    rhs = np.sum(a.astype(np.float64) * ga)
    assert abs(lhs - rhs) <= 1e-11 * (np.sum(np.abs(c * x)) + 1.0)


def test_forward_special_cases():
    M, N, K = 4, 24, 128
    a = synth.grad_out_normal(M, K, seed=81)
    # all codes 7 -> zero output
    b7 = np.full((N, K // 2), 0x77, dtype=np.uint8)
    s = synth.random_scales_uniform(N, K, seed=82)
    ref, _ = oracle.forward(a, s, b7, M, N, K)
    assert np.all(ref == 0.0)
    # unit scales and all codes 15 -> every output column is the row sum of A
    bF = np.full((N, K // 2), 0xFF, dtype=np.uint8)
    ref, _ = oracle.forward(a, np.ones((N, K // 64), dtype=np.float32), bF, M, N, K)
    rs = np.sum(a.astype(np.float64), axis=1)
    assert np.allclose(ref, np.repeat(rs[:, None], N, axis=1), rtol=1e-14, atol=1e-14)
    # one nonzero weight at (n0, k0) with scale 0.5: column n0 of C is 0.5 * column k0 of A
    n0, k0 = 7, 45
    b = np.full((N, K // 2), 0x77, dtype=np.uint8)
    b[n0, k0 // 2] = (0x7 | (15 << 4)) if k0 % 2 else (0x70 | 15)
    ref, _ = oracle.forward(a, np.full((N, K // 64), 0.5, dtype=np.float32), b, M, N, K)
    want = np.zeros((M, N))
    want[:, n0] = 0.5 * a[:, k0].astype(np.float64)
    assert np.array_equal(ref, want)


def test_fp16_operand_reference_rounds_to_nearest_even():
    """The diagnostic reference converts with RNE (ties to even), not toward zero."""
    one = np.float32(1.0)
    tie_down = np.float32(1.0 + 2.0 ** -11)        # halfway between 1 and 1+2^-10 -> 1 (even)
    tie_up = np.float32(1.0 + 3 * 2.0 ** -11)      # halfway between 1+2^-10 and 1+2^-9 -> 1+2^-9
    above = np.float32(1.0 + 2.0 ** -11 + 2.0 ** -20)
    g = np.array([[1.0]], dtype=np.float32)
    for val, want in [(tie_down, 1.0), (tie_up, 1.0 + 2.0 ** -9), (above, 1.0 + 2.0 ** -10), (one, 1.0)]:
        # build a 1x64 weight row with scale=val and code 15 at k=0
        b = np.full((1, 32), 0x77, dtype=np.uint8)
        b[0, 0] = 0x7F
        s = np.array([[val]], dtype=np.float32)
        ref16, _ = oracle.grad_a_fp16_operands(g, s, b, 1, 1, 64)
        assert ref16[0, 0] == want


# grad_out values (fp32) and their fp16 round-to-nearest-even images, worked out
# by hand from the binary16 format (11 significant bits, normals down to 2^-14,
# subnormals in steps of 2^-24, largest finite 65504): ties go to the even
# significand, values below 2^-25 in magnitude round to zero.
FP16_RNE_CASES = [
    (1.0 + 2.0 ** -11, 1.0),                               # tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),               # tie -> even (1 + 2^-9)
    (-(1.0 + 2.0 ** -11), -1.0),
    (1.0 + 2.0 ** -11 + 2.0 ** -22, 1.0 + 2.0 ** -10),     # just above the tie -> up
    (0.1, 1638.0 / 16384.0),                               # fp32 0.1 = 1638.4000... * 2^-14 -> 1638 * 2^-14
    (2.0 ** -14 + 2.0 ** -25, 2.0 ** -14),                 # smallest normal: tie -> even
    (2.0 ** -15 + 2.0 ** -25, 2.0 ** -15),                 # subnormal: 512.5 steps -> 512
    (2.0 ** -15 + 3 * 2.0 ** -25, 514 * 2.0 ** -24),       # subnormal: 513.5 steps -> 514
    (1.25 * 2.0 ** -24, 2.0 ** -24),                       # subnormal: 1.25 steps -> 1
    (3 * 2.0 ** -25, 2 * 2.0 ** -24),                      # 1.5 steps -> 2 (even)
    (2.0 ** -25, 0.0),                                     # 0.5 steps -> 0 (even)
    (2.0 ** -26, 0.0),                                     # rounds to zero
    (65504.0, 65504.0),                                    # largest finite
    (65519.0, 65504.0),                                    # below the overflow midpoint 65520
    (-65504.0, -65504.0),
    (3.0, 3.0),
]


def test_fp16_operand_reference_rounds_grad_out_to_nearest_even():
    """The diagnostic reference rounds grad_out to fp16 (RNE), checked against hand-worked values.

    The weight is a single exact 1.0 (scale 1, code 15), so grad_A[m][0] is the
    fp16 image of grad_out[m][0] itself and the bound scale is its magnitude.
    Leaving grad_out in fp32, or rounding it any other way, fails here.
    """
    vals = np.array([v for v, _ in FP16_RNE_CASES], dtype=np.float32).reshape(-1, 1)
    want = np.array([w for _, w in FP16_RNE_CASES], dtype=np.float64)
    M = vals.shape[0]
    b = np.full((1, 32), 0x77, dtype=np.uint8)
    b[0, 0] = 0x7F                                         # code 15 (level 1.0) at k = 0, zeros elsewhere
    s = np.ones((1, 1), dtype=np.float32)
    ref16, S16 = oracle.grad_a_fp16_operands(vals, s, b, M, 1, 64)
    assert np.array_equal(ref16[:, 0], want)
    assert np.array_equal(S16[:, 0], np.abs(want))
    assert np.all(ref16[:, 1:] == 0.0)
    # the same values as one row against a column of unit weights: the sum of their fp16 images
    # (every partial sum is exact in fp64)
    b2 = np.full((M, 32), 0x77, dtype=np.uint8)
    b2[:, 0] = 0x7F
    ref16, _ = oracle.grad_a_fp16_operands(vals.reshape(1, M), np.ones((M, 1), dtype=np.float32), b2, 1, M, 64)
    assert ref16[0, 0] == math.fsum(want)


# ---------------------------------------------------------------------- pack

def _pack_bruteforce(w_block):
    """Exact rational argmin over the 16 levels, ties to the lower code."""
    absmax = max(abs(Fraction(float(x))) for x in w_block)
    if absmax == 0:
        return 0.0, [7] * len(w_block)
    levels = [Fraction(float(q)) for q in oracle.NF4_LEVELS]
    codes = []
    for x in w_block:
        r = Fraction(float(x)) / absmax
        dists = [abs(r - q) for q in levels]
        best = min(dists)
        codes.append(dists.index(best))          # first index = lower code on ties
    return float(absmax), codes


def test_pack_matches_exact_rational_argmin():
    N, K = 3, 128
    w = synth.weights_normal(N, K, seed=51)
    scales, b = oracle.pack(w, N, K)
    codes = oracle.unpack_codes(b, N, K)
    for n in range(N):
        for kb in range(K // 64):
            blk = w[n, kb * 64:(kb + 1) * 64]
            a, c = _pack_bruteforce(blk)
            assert scales[n, kb] == a
            assert list(codes[n, kb * 64:(kb + 1) * 64]) == c


def test_pack_exact_ties_go_to_lower_code():
    # absmax 1.0; q6/2 and q8/2 are exact midpoints against level 0.0 and are fp32-representable
    q = oracle.NF4_LEVELS
    row = np.zeros(64, dtype=np.float32)
    row[0] = 1.0
    row[1] = q[6] / 2          # tie between codes 6 and 7 -> 6
    row[2] = q[8] / 2          # tie between codes 7 and 8 -> 7
    row[3] = -1.0              # tie-free endpoint -> 0
    row[4] = np.nextafter(np.float32(q[8] / 2), np.float32(1))  # just above -> 8
    _, b = oracle.pack(row[None, :], 1, 64)
    c = oracle.unpack_codes(b, 1, 64)[0]
    assert list(c[:5]) == [15, 6, 7, 0, 8]
    for i, x in enumerate(row[:5]):
        assert _pack_bruteforce(row)[1][i] == c[i]


def test_pack_special_blocks_and_round_trip():
    N, K = 4, 256
    w = synth.weights_normal(N, K, seed=61)
    w[1, 64:128] = 0.0                            # an all-zero block
    w[2, 0:64] = -0.0
    scales, b = oracle.pack(w, N, K)
    codes = oracle.unpack_codes(b, N, K)
    assert scales[1, 1] == 0.0 and np.all(codes[1, 64:128] == 7)
    assert scales[2, 0] == 0.0 and np.all(codes[2, 0:64] == 7)
    back = oracle.dequant(scales, b, N, K)
    for n in range(N):
        for kb in range(K // 64):
            blk = w[n, kb * 64:(kb + 1) * 64]
            a = scales[n, kb]
            # the max half-gap between neighbouring levels is below 0.152
            assert np.all(np.abs(back[n, kb * 64:(kb + 1) * 64].astype(np.float64) - blk)
                          <= 0.152 * float(a) * (1 + 1e-6))
            if a > 0:
                i = int(np.argmax(np.abs(blk)))
                assert abs(float(back[n, kb * 64 + i])) == float(a)   # the absmax element is exact
                assert codes[n, kb * 64 + i] in (0, 15)
