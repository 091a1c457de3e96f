"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bars:
* nf4_dequant and nf4_pack: bit-exact.
* nf4_grad_a: |gpu - ref| <= 2e-3 * S + 1e-6 element by element, with ref the
  fp64 definition and S = sum_n |g * w|.  A tighter diagnostic compares with
  the fp16-operand reference (sum_n fp16(g) * fp16(w) in fp64): the only
  difference left there is fp32 accumulation, bounded by
  (N/8 + 64) * 2^-24 * S16, which fp16 rounding in the wrong direction
  (e.g. toward zero) would break at the small sizes used.
Every input is seeded and synthetic; no expected value comes from the GPU.
"""

import functools

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within_bound(gpu, ref, S, what=""):
    err = np.abs(gpu.astype(np.float64) - ref)
    lim = 2e-3 * S + 1e-6
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} S={S[i]!r}")
    assert np.all(np.isfinite(gpu))


def assert_fp16_diag(gpu, g, s, b, M, N, K, rows=None, what=""):
    ref16, S16 = oracle.grad_a_fp16_operands(g, s, b, M, N, K, rows=rows)
    tol = (N / 8 + 64) * 2.0 ** -24 * S16 + 1e-30
    err = np.abs(gpu.astype(np.float64) - ref16)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError(f"{what}: fp16-operand diagnostic failed at {i}: gpu={gpu[i]!r} "
                             f"ref16={ref16[i]!r} tol={tol[i]!r}")


@functools.lru_cache(maxsize=8)
def packed_weights(N, K, seed):
    """Oracle-quantised N(0, 0.02) weights (CPU): the inputs both sides use."""
    w = synth.weights_normal(N, K, seed)
    s, b = oracle.pack(w, N, K)
    return s, b


def random_inputs(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    return g, s, b


def check_grad_a(nb, g, s, b, M, N, K, kernel=None, rb=2, splits=1, what="", diag=True):
    gd, sd, bd = dev(g), dev(s), dev(b)
    if kernel is None:
        out = nb.grad_a(gd, sd, bd)
    else:
        out = nb.grad_a_forced(gd, sd, bd, kernel, rb=rb, splits=splits)
    gpu = host(out)
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    assert_within_bound(gpu, ref, S, what)
    if diag:
        assert_fp16_diag(gpu, g, s, b, M, N, K, what=what)
    return gpu


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("N,K", [(1, 64), (3, 128), (17, 320), (256, 256), (1536, 1536), (18944, 3584)])
def test_dequant_bit_exact(lib, N, K):
    b = synth.random_code_bytes(N, K, seed=N + K)
    s = synth.random_scales_uniform(N, K, seed=N + K + 1)
    w = host(lib.dequant(dev(s), dev(b)))
    assert np.array_equal(w.view(np.uint32), oracle.dequant(s, b, N, K).view(np.uint32))


def test_dequant_bit_exact_wide_scale_range(lib):
    """Scales from 1e-40 (fp32 subnormal) to 1e30: products round exactly like the oracle, subnormals kept."""
    N, K = 64, 512
    rng = np.random.default_rng(7)
    s = (10.0 ** rng.uniform(-40, 30, size=(N, K // 64))).astype(np.float32)
    s *= np.where(rng.random(s.shape) < 0.5, -1, 1).astype(np.float32)
    b = synth.random_code_bytes(N, K, seed=8)
    w = host(lib.dequant(dev(s), dev(b)))
    assert np.array_equal(w.view(np.uint32), oracle.dequant(s, b, N, K).view(np.uint32))


# --------------------------------------------------------------------- pack

@pytest.mark.parametrize("N,K", [(1, 64), (5, 192), (64, 1024), (1536, 1536), (3584, 3584)])
def test_pack_bit_exact(lib, N, K):
    w = synth.weights_normal(N, K, seed=N * 7 + K)
    if N >= 5:
        w[0, :64] = 0.0
        w[1, :64] = -0.0
        w[2, :64] = 0.0
        w[2, 5] = 3.5
        q = oracle.NF4_LEVELS
        w[3, :64] = 0.0
        w[3, 0] = 1.0
        w[3, 1] = q[6] / 2          # exact tie -> lower code
        w[3, 2] = q[8] / 2
        w[4, 64 % K:64 % K + 64] = np.float32(2.0 ** -130)   # subnormal block
    s, b = lib.pack(dev(w))
    s_ref, b_ref = oracle.pack(w, N, K)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(b), b_ref)


def test_pack_weights_on_and_beside_the_thresholds(lib):
    """Blocks whose weights sit on the fp32 values nearest to each decision threshold absmax * mid_i and on
    their fp32 neighbours above and below, for absmax over the whole fp32 range (subnormal to 2^100) and both
    signs of the absmax element: the codes must match the oracle's exact fp64 decision bit for bit."""
    rng = np.random.default_rng(31)
    q = oracle.NF4_LEVELS.astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2
    N, K = 256, 128
    w = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        for kb in range(K // 64):
            a = np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-140, 100)))
            t = (np.float64(a) * mids).astype(np.float32)  # nearest fp32 (ties to even)
            vals = np.concatenate([t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))])
            blk = rng.choice(vals, size=63)
            lead = a if rng.random() < 0.5 else -a
            w[n, 64 * kb:64 * kb + 64] = np.concatenate([[lead], blk]).astype(np.float32)
    assert np.all(np.abs(w).reshape(N, -1, 64).max(axis=2) == np.abs(w[:, ::64]))
    s, b = lib.pack(dev(w))
    s_ref, b_ref = oracle.pack(w, N, K)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(b), b_ref)


# ------------------------------------------------------------------- grad_A

SMALL = [
    # (M, N, K)
    (1, 1, 64), (2, 17, 64), (8, 64, 128), (15, 100, 192), (16, 128, 256), (17, 64, 64),
    (33, 200, 320), (100, 64, 512), (130, 257, 256), (257, 128, 192), (64, 1, 128),
]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_grad_a_small_default_plan(lib, M, N, K):
    g, s, b = random_inputs(M, N, K, seed=M * 1000 + N + K)
    check_grad_a(lib, g, s, b, M, N, K, what=f"default {M}x{N}x{K}")


@pytest.mark.parametrize("kernel,rb,splits", [("tile", 1, 1), ("tile", 2, 1), ("tile", 1, 3), ("tile", 2, 2),
                                              ("skinny", 0, 1), ("skinny", 0, 3),
                                              ("stream", 0, 1), ("stream", 0, 3), ("stream", 0, 7)])
@pytest.mark.parametrize("M,N,K", [(1, 300, 320), (5, 200, 192), (16, 1000, 512), (3, 129, 64), (12, 64, 1088)])
def test_grad_a_every_variant_small(lib, kernel, rb, splits, M, N, K):
    g, s, b = random_inputs(M, N, K, seed=M + N * 3 + K * 5 + splits)
    check_grad_a(lib, g, s, b, M, N, K, kernel=kernel, rb=max(rb, 1), splits=splits,
                 what=f"{kernel} rb{rb} s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("kernel,rb,splits", [("tile", 1, 1), ("tile", 2, 1), ("tile", 2, 4), ("tile", 1, 2)])
@pytest.mark.parametrize("M,N,K", [(200, 384, 768), (300, 100, 320), (513, 640, 256)])
def test_grad_a_tile_variants_ragged(lib, kernel, rb, splits, M, N, K):
    g, s, b = random_inputs(M, N, K, seed=M + N + K + rb * 11 + splits)
    check_grad_a(lib, g, s, b, M, N, K, kernel=kernel, rb=rb, splits=splits,
                 what=f"{kernel} rb{rb} s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("rb,splits", [(1, 1), (1, 2), (1, 3)])
@pytest.mark.parametrize("M,N,K", [(17, 64, 64), (200, 384, 768), (513, 640, 320), (600, 1024, 448),
                                   (1030, 256, 1088)])
def test_grad_a_wide_variants_ragged(lib, rb, splits, M, N, K):
    """Wide tile kernel (N % 64 == 0), fp32 grad_out converted in the loop: 512x128 tiles, ragged M and K
    tails, N splits."""
    g, s, b = random_inputs(M, N, K, seed=M + 7 * N + K + rb * 13 + splits)
    check_grad_a(lib, g, s, b, M, N, K, kernel="wide", rb=rb, splits=splits,
                 what=f"wide rb{rb} s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("M,N,K", [(17, 64, 64), (200, 384, 768), (513, 640, 320), (600, 1024, 448),
                                   (1030, 256, 1088), (31, 128, 128)])
def test_grad_a_wide16_variants_ragged(lib, splits, M, N, K):
    """Wide kernel fed by the fp16 A-fragment pass: ragged M (fragment rows padded to 16, tile rows past
    the padded M), ragged K, N splits sharing the workspace with the fragments."""
    g, s, b = random_inputs(M, N, K, seed=M + 5 * N + K + 17 * splits)
    check_grad_a(lib, g, s, b, M, N, K, kernel="wide16", rb=1, splits=splits,
                 what=f"wide16 s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("rb,splits", [(1, 1), (3, 1), (1, 3), (3, 2)])
@pytest.mark.parametrize("M,N,K", [(17, 64, 64), (255, 384, 768), (257, 640, 320), (600, 1024, 448),
                                   (1030, 256, 1088), (31, 128, 128)])
def test_grad_a_mid_variants_ragged(lib, rb, splits, M, N, K):
    """Mid-size 256 x 128 tiles (four waves, two workgroups per CU) on the fp16 A fragments: ragged M around
    the 256-row tile, ragged K, N splits, both fragment prefetch depths; within the bound and bitwise equal to
    the 512 x 128 kernel (same operands, same reduction order)."""
    g, s, b = random_inputs(M, N, K, seed=M + 3 * N + K + 11 * rb + 19 * splits)
    got = check_grad_a(lib, g, s, b, M, N, K, kernel="mid", rb=rb, splits=splits,
                       what=f"mid rb{rb} s{splits} {M}x{N}x{K}")
    ref = host(lib.grad_a_forced(dev(g), dev(s), dev(b), "wide16", rb=1, splits=splits))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_grad_a_mid_rejects_unsupported_depth(lib):
    g, s, b = random_inputs(64, 128, 128, seed=3)
    with pytest.raises(lib.Nf4Error):
        lib.grad_a_forced(dev(g), dev(s), dev(b), "mid", rb=2)
    with pytest.raises(lib.Nf4Error):
        lib.grad_a_forced(dev(g), dev(s), dev(b), "small", rb=3)


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("M,N,K", [(17, 64, 64), (127, 384, 768), (129, 640, 320), (600, 1024, 448),
                                   (1030, 256, 1088), (31, 128, 128), (1100, 1024, 1088)])
def test_grad_a_small_tiles_ragged(lib, splits, M, N, K):
    """Small 128 x 128 tiles (four waves of 32 rows, three workgroups per CU) on the fp16 A fragments: ragged M
    around the 128-row tile, ragged K, N splits; within the bound and bitwise equal to the 512 x 128 kernel
    (same operands, same reduction order)."""
    g, s, b = random_inputs(M, N, K, seed=M + 5 * N + K + 23 * splits)
    got = check_grad_a(lib, g, s, b, M, N, K, kernel="small", rb=1, splits=splits,
                       what=f"small s{splits} {M}x{N}x{K}")
    ref = host(lib.grad_a_forced(dev(g), dev(s), dev(b), "wide16", rb=1, splits=splits))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_grad_a_small_tiles_chosen_for_short_reductions(lib):
    """The plan of a short reduction that the larger tiles would split (1100 x 1024 x 1088) is the unsplit
    small-tile kernel, and the default call gives its result."""
    M, N, K = 1100, 1024, 1088
    assert lib.grad_a_plan(M, N, K)["kernel"] == "small"
    g, s, b = random_inputs(M, N, K, seed=41)
    got = check_grad_a(lib, g, s, b, M, N, K, what=f"default {M}x{N}x{K}")
    ref = host(lib.grad_a_forced(dev(g), dev(s), dev(b), "small", rb=1, splits=1))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_grad_a_wide16_matches_wide_bitwise(lib):
    """Both grad_out paths give the same fp16 operands in the same reduction order, so the results are
    bitwise equal."""
    M, N, K = 700, 2048, 384
    g, s, b = random_inputs(M, N, K, seed=37)
    gd, sd, bd = dev(g), dev(s), dev(b)
    for splits in (1, 2):
        r1 = host(lib.grad_a_forced(gd, sd, bd, "wide", rb=1, splits=splits))
        r2 = host(lib.grad_a_forced(gd, sd, bd, "wide16", rb=1, splits=splits))
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
    with pytest.raises(lib.Nf4Error):
        lib.grad_a_forced(dev(g[:, :2000]), sd[:2000], bd[:2000], "wide16", rb=1)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("M,N,K", [(17, 64, 64), (200, 384, 768), (513, 640, 320), (1030, 256, 1088)])
def test_grad_a_unfused_matches_fused_bitwise(lib, splits, M, N, K):
    """The unfused comparison path (weights dequantised to fp16 by a separate pass, then a GEMM that copies
    them instead of decoding) multiplies the same fp16 operands in the same order as the fused kernel:
    bitwise equal results, and within the oracle's bound."""
    g, s, b = random_inputs(M, N, K, seed=3 * M + N + 5 * K + splits)
    gd, sd, bd = dev(g), dev(s), dev(b)
    fused = host(lib.grad_a_forced(gd, sd, bd, "wide16", rb=1, splits=splits))
    unfused = host(lib.grad_a_forced(gd, sd, bd, "unfused", rb=1, splits=splits))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    assert_within_bound(unfused, ref, S, f"unfused s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("M", [17, 600, 1100])
def test_grad_a_grouped_matches_separate_calls(lib, M):
    """A layer-like group: problems with different N and K (one the wide kernel does not take, N % 64 != 0),
    each checked against the oracle and bitwise against its separate launch."""
    shapes = [(256, 384), (64, 384), (640, 1088), (100, 192), (1024, 128)]  # (N, K)
    data = [random_inputs(M, N, K, seed=7 * M + N + K) for (N, K) in shapes]
    devs = [(dev(g), dev(s), dev(b)) for g, s, b in data]
    outs = lib.grad_a_grouped(devs)
    for (N, K), (g, s, b), d, o in zip(shapes, data, devs, outs):
        gpu = host(o)
        if N % 64 == 0:
            sep = host(lib.grad_a_forced(*d, "wide16", rb=1, splits=1))
        else:
            sep = host(lib.grad_a(*d))
        assert np.array_equal(gpu.view(np.uint32), sep.view(np.uint32)), (M, N, K)
        ref, S = oracle.grad_a(g, s, b, M, N, K)
        assert_within_bound(gpu, ref, S, f"grouped {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 8, 16])
def test_grad_a_grouped_skinny_matches_separate_calls(lib, M):
    """M <= 16: the streaming problems run as one grid, each bitwise equal to its own nf4_grad_a call (split
    and unsplit plans, N tails inside a k-step, K % 128 == 64); N % 4 != 0 and N == 0 problems run on their
    own; every output within the bound.  Run twice: the second pass reuses the arrival counters."""
    shapes = [(3000, 512), (700, 1344), (4100, 384), (102, 256), (2048, 640), (0, 128), (96, 64), (9000, 128)]
    data = [random_inputs(M, N, K, seed=11 * M + N + K) for (N, K) in shapes]
    devs = [(dev(g), dev(s), dev(b)) for g, s, b in data]
    seps = [host(lib.grad_a(*d)) for d in devs]
    for rnd in range(2):
        outs = [torch.full((M, K), float("nan"), device="cuda") for (N, K) in shapes]
        lib.grad_a_grouped(devs, outs=outs)
        for (N, K), (g, s, b), o, sep in zip(shapes, data, outs, seps):
            gpu = host(o)
            assert np.array_equal(gpu.view(np.uint32), sep.view(np.uint32)), (rnd, M, N, K)
            if rnd == 0:
                ref, S = oracle.grad_a(g, s, b, M, N, K)
                assert_within_bound(gpu, ref, S, f"grouped skinny {M}x{N}x{K}")


def test_grad_a_grouped_skinny_layer_shapes(lib):
    """A 7B-class layer's seven projections at M = 16 in one grouped call: bitwise equal to separate calls."""
    M = 16
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584), (18944, 3584), (3584, 18944)]
    devs = []
    for i, (N, K) in enumerate(shapes):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(500 + i)
        g = torch.empty((M, N), device="cuda").normal_(0.0, 1.0, generator=gen)
        sc = torch.empty((N, K // 64), device="cuda").uniform_(0.01, 0.1, generator=gen)
        cd = torch.randint(0, 256, (N, K // 2), device="cuda", dtype=torch.uint8, generator=gen)
        devs.append((g, sc, cd))
    seps = [host(lib.grad_a(*d)) for d in devs]
    outs = lib.grad_a_grouped(devs)
    for (N, K), o, sep in zip(shapes, outs, seps):
        assert np.array_equal(host(o).view(np.uint32), sep.view(np.uint32)), (N, K)


def test_grad_a_grouped_edges(lib):
    g, s, b = random_inputs(40, 128, 256, seed=5)
    d = (dev(g), dev(s), dev(b))
    assert lib.grad_a_grouped([]) == []
    # a single problem and a skinny M take the separate plans
    one = lib.grad_a_grouped([d])
    assert np.array_equal(host(one[0]).view(np.uint32), host(lib.grad_a_forced(*d, "wide16", rb=1, splits=1)).view(np.uint32))
    gs, ss, bs = random_inputs(8, 128, 256, seed=6)
    sk = lib.grad_a_grouped([(dev(gs), dev(ss), dev(bs))])
    ref, S = oracle.grad_a(gs, ss, bs, 8, 128, 256)
    assert_within_bound(host(sk[0]), ref, S, "grouped skinny")
    with pytest.raises(ValueError):
        lib.grad_a_grouped([d] * 9)


def test_grad_a_wide_deterministic_and_rejects_ragged_n(lib):
    M, N, K = 700, 4096, 384
    g, s, b = random_inputs(M, N, K, seed=31)
    gd, sd, bd = dev(g), dev(s), dev(b)
    for rb, splits in [(1, 1), (1, 3)]:
        r1 = host(lib.grad_a_forced(gd, sd, bd, "wide", rb=rb, splits=splits))
        r2 = host(lib.grad_a_forced(gd, sd, bd, "wide", rb=rb, splits=splits))
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
    with pytest.raises(lib.Nf4Error):
        lib.grad_a_forced(dev(g[:, :4000]), sd[:4000], bd[:4000], "wide", rb=1)


@pytest.mark.parametrize("splits", [1, 2, 5])
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (2, 33, 192), (7, 257, 320), (16, 2048, 640), (9, 5000, 128),
                                   (16, 31, 64)])
def test_grad_a_stream_ragged(lib, splits, M, N, K):
    """Streaming kernel (M <= 16): N tails inside a k-step, chunk ends, K tails inside a strip."""
    g, s, b = random_inputs(M, N, K, seed=13 * M + N + 3 * K + splits)
    check_grad_a(lib, g, s, b, M, N, K, kernel="stream", splits=splits, what=f"stream s{splits} {M}x{N}x{K}")


def test_grad_a_stream_deterministic(lib):
    M, N, K = 16, 3000, 512
    g, s, b = random_inputs(M, N, K, seed=77)
    gd, sd, bd = dev(g), dev(s), dev(b)
    for splits in (1, 4):
        r1 = host(lib.grad_a_forced(gd, sd, bd, "stream", rb=0, splits=splits))
        r2 = host(lib.grad_a_forced(gd, sd, bd, "stream", rb=0, splits=splits))
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


def _cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("M,N,K,splits", [(16, 3000, 512, 4), (3, 4100, 384, 7), (8, 2048, 640, 64),
                                          (1, 3584, 18944, 3), (16, 18944, 3584, 18)])
def test_grad_a_stream_split_sum_is_chunk_partials_in_order(lib, M, N, K, splits):
    """The streaming kernel's split reduction, done by each strip's last workgroup to finish, equals bit for
    bit the unsplit kernel run on each N-chunk alone (the same k-steps per wave, hence the same partial),
    summed on the host in fp32 in chunk order."""
    g, s, b = random_inputs(M, N, K, seed=7 * M + N + K + splits)
    chunk = _cdiv(_cdiv(N, splits), 32) * 32
    full = host(lib.grad_a_forced(dev(g), dev(s), dev(b), "stream", rb=0, splits=splits))
    acc = None
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        part = host(lib.grad_a_forced(dev(g[:, n0:n1]), dev(s[n0:n1]), dev(b[n0:n1]), "stream", rb=0, splits=1))
        acc = part.copy() if acc is None else (acc + part).astype(np.float32)
    assert _cdiv(N, chunk) > 1
    assert np.array_equal(full.view(np.uint32), acc.view(np.uint32))


def test_grad_a_stream_split_counters_across_calls(lib):
    """Split calls of different strip and split counts back to back on one stream (they share the
    workspace's arrival counters): every output written in full (outputs start as NaN), each within the
    bound, and the second pass bitwise equal to the first."""
    shapes = [(16, 3000, 512, 4), (8, 5000, 1024, 6), (1, 700, 128, 3), (16, 3000, 512, 11), (4, 9000, 256, 64)]
    data = [random_inputs(M, N, K, seed=300 + i) for i, (M, N, K, _) in enumerate(shapes)]
    devs = [(dev(g), dev(s), dev(b)) for g, s, b in data]
    firsts = []
    for rnd in range(2):
        outs = []
        for (M, N, K, sp), d in zip(shapes, devs):
            o = torch.full((M, K), float("nan"), device="cuda")
            outs.append(lib.grad_a_forced(*d, "stream", rb=0, splits=sp, out=o))
        res = [host(o) for o in outs]
        for i, ((M, N, K, sp), (g, s, b)) in enumerate(zip(shapes, data)):
            if rnd == 0:
                ref, S = oracle.grad_a(g, s, b, M, N, K)
                assert_within_bound(res[i], ref, S, f"shape {i}")
                firsts.append(res[i])
            else:
                assert np.array_equal(res[i].view(np.uint32), firsts[i].view(np.uint32)), f"shape {i}"


PAGE_SHAPES = [(128, 1536, 1536), (64, 256, 128), (16, 64, 64), (512, 1536, 1536), (512, 256, 1536),
               (512, 4608, 1536), (512, 1536, 4608)]


@pytest.mark.parametrize("M,N,K", PAGE_SHAPES)
def test_grad_a_page_test_shapes(lib, M, N, K):
    """The (m, n, k) triples of the subject page's own tests, packed N(0, 0.02) weights."""
    s, b = packed_weights(N, K, seed=N + K)
    g = synth.grad_out_normal(M, N, seed=M + 5, std=1e-2)
    check_grad_a(lib, g, s, b, M, N, K, what=f"page {M}x{N}x{K}")


def test_grad_a_tiny_config(lib):
    g, s, b = synth.inputs.tiny_inputs(seed=0)
    check_grad_a(lib, g, s, b, 64, 256, 256, what="tiny")


def test_grad_a_attention_projection_config(lib):
    M, N, K = 2048, 1536, 1536
    s, b = packed_weights(N, K, seed=0)
    g = synth.grad_out_normal(M, N, seed=0 + 100, std=1e-2)
    check_grad_a(lib, g, s, b, M, N, K, what="attn_proj")


@pytest.mark.parametrize("which,seed", [(0, 0), (1, 1)])
def test_grad_a_mlp_pair_config(lib, which, seed):
    shp = synth.CONFIGS["mlp_pair"][which]
    M, N, K = shp.M, shp.N, shp.K
    s, b = packed_weights(N, K, seed=seed)
    g = synth.grad_out_normal(M, N, seed=seed + 100, std=1e-2)
    check_grad_a(lib, g, s, b, M, N, K, what=shp.name)


@pytest.mark.parametrize("shp", synth.SKINNY_SHAPES, ids=lambda s: s.name)
def test_grad_a_skinny_config(lib, shp):
    M, N, K = shp.M, shp.N, shp.K
    seed = 0 if K == 3584 else 1
    s, b = packed_weights(N, K, seed=seed)
    g = synth.grad_out_normal(M, N, seed=10 + M, std=1.0)
    check_grad_a(lib, g, s, b, M, N, K, what=shp.name)


# ------------------------------------------------- maximum sizes: operands of 2 GiB and more

def test_grad_a_skinny_with_codes_of_2_gib(lib):
    """M <= 16 with a 2 GiB code array (N * K / 2 = 2^31 bytes, past the streaming kernel's 32-bit byte
    offsets): the planner falls back to the skinny kernel, whose offsets are 64-bit.  All 16 rows on 48
    sampled columns (column-sampled oracle)."""
    M, N, K = 16, 65536, 65536
    plan = lib.grad_a_plan(M, N, K)
    assert plan["kernel"] == "skinny"
    rng = np.random.default_rng(77)
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = synth.random_scales_uniform(N, K, seed=78)
    g = synth.grad_out_normal(M, N, seed=79)
    gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    cols = np.unique(np.concatenate([[0, 1, K - 2, K - 1], rng.integers(0, K, size=44)]))
    ref, S = oracle.grad_a(g, s, b, M, N, K, cols=cols)
    assert_within_bound(gpu[:, cols], ref, S, "skinny 2 GiB codes")
    assert np.all(np.isfinite(gpu))


def test_grad_a_large_m_with_grad_out_of_2_gib(lib):
    """M > 16 with a 2 GiB grad_out (M * N * 4 = 2^31 bytes, past the wide kernels' 32-bit offsets): the
    tile kernel's general path.  grad_out is drawn on the device (seeded torch generator); 12 sampled
    rows are copied back for the oracle."""
    M, N, K = 8192, 65536, 256
    plan = lib.grad_a_plan(M, N, K)
    assert plan["kernel"] == "tile"
    b = synth.random_code_bytes(N, K, seed=81)
    s = synth.random_scales_uniform(N, K, seed=82)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(83)
    gd = torch.empty((M, N), device="cuda").normal_(0.0, 1e-2, generator=gen)
    gpu = lib.grad_a(gd, dev(s), dev(b))
    rows = np.array([0, 1, 4095, 4096, 6000, M - 2, M - 1, 17, 512, 1023, 3000, 7777])
    g_rows = host(gd[torch.from_numpy(rows).cuda()])
    gpu_rows = host(gpu)[rows]
    del gd, gpu
    ref, S = oracle.grad_a(g_rows, s, b, len(rows), N, K)
    assert_within_bound(gpu_rows, ref, S, "tile 2 GiB grad_out")


def test_forward_rejects_codes_of_2_gib(lib):
    """The forward kernels take codes below 2 GiB only: NF4_ERR_SHAPE before any launch."""
    N, K = 65536, 65536
    b = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.ones((N, K // 64), dtype=torch.float32, device="cuda")
    a = torch.ones((1, K), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.Nf4Error):
        lib.forward(a, s, b)


# ------------------------------------------------- metamorphic / exact checks

def test_grad_a_deterministic(lib):
    M, N, K = 300, 4000, 512
    g, s, b = random_inputs(M, N, K, seed=9)
    gd, sd, bd = dev(g), dev(s), dev(b)
    for kernel, rb, splits in [("tile", 2, 3), ("tile", 1, 1)]:
        r1 = host(lib.grad_a_forced(gd, sd, bd, kernel, rb=rb, splits=splits))
        r2 = host(lib.grad_a_forced(gd, sd, bd, kernel, rb=rb, splits=splits))
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
    g1 = g[:7]
    r1 = host(lib.grad_a(dev(g1), sd, bd))
    r2 = host(lib.grad_a(dev(g1), sd, bd))
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


@pytest.mark.parametrize("M", [5, 200])
def test_grad_a_power_of_two_scaling_is_exact(lib, M):
    N, K = 640, 512
    g, s, b = random_inputs(M, N, K, seed=17)
    g = np.sign(g) * np.clip(np.abs(g), 2.0 ** -12, 1000.0)  # fp16 images stay normal
    g = g.astype(np.float32)
    base = host(lib.grad_a(dev(g), dev(s), dev(b)))
    twice_g = host(lib.grad_a(dev(g * 2), dev(s), dev(b)))
    half_s = host(lib.grad_a(dev(g), dev(s * np.float32(0.5)), dev(b)))
    assert np.array_equal(twice_g, base * 2)
    assert np.array_equal(half_s, base * 0.5)


@pytest.mark.parametrize("M", [6, 40])
def test_grad_a_one_hot_rows_give_fp16_dequant_rows(lib, M):
    N, K = 96, 320
    b = synth.random_code_bytes(N, K, seed=21)
    s = synth.random_scales_uniform(N, K, seed=22)
    g = np.zeros((M, N), dtype=np.float32)
    picks = np.random.default_rng(23).integers(0, N, size=M)
    g[np.arange(M), picks] = 1.0
    gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float32)
    assert np.array_equal(gpu, w16[picks])


def test_grad_a_operand_rounding_of_grad_out(lib):
    """A single weight 1.0 at (n0, k0): column k0 of grad_A is fp16(grad_out[:, n0]) exactly."""
    M, N, K = 70, 64, 256
    n0, k0 = 37, 201
    b = np.full((N, K // 2), 0x77, dtype=np.uint8)
    b[n0, k0 // 2] = 0xF7 if k0 % 2 else 0x7F
    s = np.ones((N, K // 64), dtype=np.float32)
    g = synth.grad_out_normal(M, N, seed=29)
    gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    want = np.zeros((M, K), dtype=np.float32)
    want[:, k0] = g[:, n0].astype(np.float16).astype(np.float32)
    assert np.array_equal(gpu, want)


# fp32 values whose fp16 images probe round-to-nearest-even, the subnormal range and the top of the range
_FP16_EDGE_VALUES = np.array([
    0.0, -0.0, 1e-8, 2.9802322e-08, 3.0e-8, 5.9604645e-08, 8.9406967e-08, 1e-6, -3.3e-6, 6.0975552e-05,
    6.1035156e-05, 1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -10), 2.0 ** -14 * 1.5,
    1024.5, 2049.0, 65504.0, -65504.0, 65519.0, -65519.0, 0.1, -0.3333333], dtype=np.float32)

_PLANS = [(None, 1, 1), ("tile", 1, 1), ("tile", 2, 2), ("wide", 1, 1), ("wide", 2, 1), ("wide16", 1, 2),
          ("mid", 1, 2), ("skinny", 0, 2), ("stream", 0, 2)]


@pytest.mark.parametrize("kernel,rb,splits", _PLANS, ids=lambda v: str(v))
def test_grad_a_fp16_edge_values_of_grad_out_every_kernel(lib, kernel, rb, splits):
    """A single weight 1.0 at (n0, k0) and grad_out column n0 holding RNE ties, fp16 subnormals, values that
    round to zero and to +-65504: column k0 of grad_A is fp16(grad_out[:, n0]) exactly and every other
    column is zero, in every kernel (the conversion is RNE and keeps subnormals)."""
    M = 16 if kernel in ("skinny", "stream") else 48
    N, K = 128, 256
    n0, k0 = 77, 130
    b = np.full((N, K // 2), 0x77, dtype=np.uint8)
    b[n0, k0 // 2] = 0xF7 if k0 % 2 else 0x7F
    s = np.ones((N, K // 64), dtype=np.float32)
    g = synth.grad_out_normal(M, N, seed=55)
    g[:, n0] = np.resize(_FP16_EDGE_VALUES, M)
    if kernel is None:
        gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    else:
        gpu = host(lib.grad_a_forced(dev(g), dev(s), dev(b), kernel, rb=rb, splits=splits))
    want = np.zeros((M, K), dtype=np.float32)
    want[:, k0] = g[:, n0].astype(np.float16).astype(np.float32)
    assert np.all(np.isfinite(gpu))
    assert np.array_equal(gpu, want)


@pytest.mark.parametrize("kernel,rb,splits", _PLANS, ids=lambda v: str(v))
def test_grad_a_one_hot_rows_fp16_subnormal_and_large_weights(lib, kernel, rb, splits):
    """Scales from 1e-7 to 65000 make the dequantised weights span fp16 subnormals (and values that round
    to zero) up to near the fp16 maximum: one-hot grad_out rows give fp16(fl32(scale * level)) rows
    exactly in every kernel."""
    M = 16 if kernel in ("skinny", "stream") else 40
    N, K = 128, 384
    b = synth.random_code_bytes(N, K, seed=56)
    scale_set = np.array([1e-7, 3e-6, 5e-5, 6.1e-5, 1.0, 3e4, 65000.0], dtype=np.float32)
    s = scale_set[np.random.default_rng(57).integers(0, len(scale_set), size=(N, K // 64))]
    g = np.zeros((M, N), dtype=np.float32)
    picks = np.random.default_rng(58).integers(0, N, size=M)
    g[np.arange(M), picks] = 1.0
    if kernel is None:
        gpu = host(lib.grad_a(dev(g), dev(s), dev(b)))
    else:
        gpu = host(lib.grad_a_forced(dev(g), dev(s), dev(b), kernel, rb=rb, splits=splits))
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float32)
    assert np.all(np.isfinite(gpu))
    assert np.array_equal(gpu, w16[picks])


def test_grad_a_joint_permutation_of_n(lib):
    """Permuting the reduction index n jointly in W (rows of codes and scales) and in grad_out (columns)
    leaves grad_A unchanged up to rounding order: both results within the oracle's bound."""
    M, N, K = 300, 1024, 384
    g, s, b = random_inputs(M, N, K, seed=61)
    perm = np.random.default_rng(62).permutation(N)
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    base = host(lib.grad_a(dev(g), dev(s), dev(b)))
    permuted = host(lib.grad_a(dev(np.ascontiguousarray(g[:, perm])), dev(s[perm]), dev(b[perm])))
    assert_within_bound(base, ref, S, "unpermuted")
    assert_within_bound(permuted, ref, S, "n permuted jointly")


def test_grad_a_adjoint_identity(lib):
    M, N, K = 48, 700, 384
    g, s, b = random_inputs(M, N, K, seed=31)
    A = synth.grad_out_normal(M, K, seed=34)
    gpu = host(lib.grad_a(dev(g), dev(s), dev(b))).astype(np.float64)
    w = oracle.dequant(s, b, N, K).astype(np.float64)
    _, S = oracle.grad_a(g, s, b, M, N, K)
    lhs = np.sum(gpu * A)
    rhs = np.sum(g.astype(np.float64) * (A.astype(np.float64) @ w.T))
    assert abs(lhs - rhs) <= np.sum(np.abs(A) * (2e-3 * S + 1e-6))


def test_grad_a_on_side_stream(lib):
    M, N, K = 64, 256, 256
    g, s, b = random_inputs(M, N, K, seed=41)
    st = torch.cuda.Stream()
    gd, sd, bd = dev(g), dev(s), dev(b)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        out = lib.grad_a(gd, sd, bd)
    st.synchronize()
    ref, S = oracle.grad_a(g, s, b, M, N, K)
    assert_within_bound(out.cpu().numpy(), ref, S, "side stream")


def test_grad_a_split_workspace_per_stream(lib):
    """Split plans on two streams at once, each stream's workspace growing from the smaller shape to the
    larger, then the same after the cached workspaces are released."""
    shapes = [(16, 3000, 512, 3), (8, 5000, 1024, 6)]  # (M, N, K, splits)
    data = [random_inputs(M, N, K, seed=90 + i) for i, (M, N, K, _) in enumerate(shapes)]
    refs = [oracle.grad_a(g, s, b, M, N, K) for (g, s, b), (M, N, K, _) in zip(data, shapes)]
    devs = [(dev(g), dev(s), dev(b)) for g, s, b in data]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(2):
        torch.cuda.synchronize()
        outs = []
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs.append([lib.grad_a_forced(*devs[j], "stream", rb=0, splits=shapes[j][3]) for j in (i, 1 - i)])
        for st in streams:
            st.synchronize()
        for i in range(2):
            for k, j in enumerate((i, 1 - i)):
                ref, S = refs[j]
                assert_within_bound(outs[i][k].cpu().numpy(), ref, S, f"stream {i} shape {j} round {rnd}")
        lib.release_workspaces()


# --------------------------------------------------------------- edge cases

def test_grad_a_empty_and_degenerate(lib):
    K = 128
    # N == 0: empty sum -> zeros (overwrites whatever was there)
    out = torch.full((5, K), 7.0, device="cuda")
    g = torch.empty((5, 0), device="cuda")
    s = torch.empty((0, K // 64), device="cuda")
    b = torch.empty((0, K // 2), dtype=torch.uint8, device="cuda")
    lib.grad_a(g, s, b, out=out)
    assert torch.count_nonzero(out).item() == 0
    # M == 0: nothing happens
    out0 = lib.grad_a(torch.empty((0, 64), device="cuda"), torch.ones((64, 2), device="cuda"),
                      torch.zeros((64, 64), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert tuple(out0.shape) == (0, 128)


def test_grad_a_rejects_bad_arguments_on_device(lib):
    M, N, K = 8, 64, 128
    g = torch.zeros((M, N + 1), device="cuda")
    s = torch.ones((N, K // 64), device="cuda")
    b = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    out = torch.zeros((M, K), device="cuda")
    hs = torch.cuda.current_stream().cuda_stream
    # misaligned grad_out (offset by one float)
    st = lib.grad_a_raw(g.data_ptr() + 4, s.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, hs)
    assert st == lib.NF4_ERR_ALIGN
    st = lib.grad_a_raw(g.data_ptr(), s.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K + 1, hs)
    assert st == lib.NF4_ERR_SHAPE
    with pytest.raises(lib.Nf4Error):
        lib.grad_a_forced(torch.zeros((17, N), device="cuda"), s, b, "skinny")   # skinny needs M <= 16


# ------------------------------------------- line streaming (M <= 16, 256-column strips, hybrid decode)

@pytest.mark.parametrize("vr", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("splits", [1, 3, 9])
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (2, 36, 192), (7, 260, 320), (16, 2048, 640), (9, 5000, 128),
                                   (16, 28, 64), (16, 300, 1088)])
def test_grad_a_lines_ragged(lib, vr, splits, M, N, K):
    """Line-streaming kernel, every split of its rows between register (byte-plane) decode and 16-bit table
    reads, and one row through the shared codebook (variant 5): ragged M, N inside a 16-row k-step, K % 256
    != 0 (the last strip part-empty), N-chunk partials summed in the kernel (the last workgroup's threads
    sharing an output when there are few)."""
    g, s, b = random_inputs(M, N, K, seed=M + 5 * N + 3 * K + 7 * splits + vr)
    check_grad_a(lib, g, s, b, M, N, K, kernel="lines", rb=vr, splits=splits,
                 what=f"lines vr{vr} s{splits} {M}x{N}x{K}")


def test_grad_a_lines_decode_paths_agree_bitwise(lib):
    """The register decode (byte-plane v_perm lookups) and the LDS decode produce the same fp16 weights, so
    every split of the rows between them gives bitwise the same result; one-hot rows give fp16(dequant)
    rows exactly on both paths; repeated calls with other split counts leave the arrival counters at zero."""
    M, N, K = 16, 3000, 768
    g, s, b = random_inputs(M, N, K, seed=91)
    gd, sd, bd = dev(g), dev(s), dev(b)
    base = host(lib.grad_a_forced(gd, sd, bd, "lines", rb=0, splits=4))
    for vr in (1, 2, 3, 4, 5):
        for splits in (4, 1, 7):
            r = host(lib.grad_a_forced(gd, sd, bd, "lines", rb=vr, splits=splits))
            if splits == 4:
                assert np.array_equal(r.view(np.uint32), base.view(np.uint32)), vr
            else:
                ref, S = oracle.grad_a(g, s, b, M, N, K)
                assert_within_bound(r, ref, S, f"lines vr{vr} s{splits}")
    # one-hot rows: grad_A row m = fp16(W[n_m][:]) exactly
    picks = [0, 1, 17, 255, 256, 1023, 2999, 5, 6, 7, 8, 9, 10, 11, 12, 13]
    oh = np.zeros((M, N), dtype=np.float32)
    for m, n in enumerate(picks):
        oh[m, n] = 1.0
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float32)
    for vr in (0, 2, 4, 5):
        r = host(lib.grad_a_forced(dev(oh), sd, bd, "lines", rb=vr, splits=3))
        for m, n in enumerate(picks):
            assert np.array_equal(r[m].view(np.uint32), w16[n].view(np.uint32)), (vr, m, n)
