"""GPU parity of the forward product nf4_forward against the CPU oracle.

c[m][n] = sum_k fp16(a[m][k]) * fp16(w[n][k]) accumulated in fp32; accepted
when |gpu - ref| <= 2e-3 * S + 1e-6 element by element (ref the fp64
definition, S = sum_k |a * w|), the same bound as grad_A.  The diagnostic
against the fp16-operand product sum_k fp16(a) * fp16(w) (fp64) leaves only
fp32 accumulation, bounded by (K/8 + 64) * 2^-24 * S16.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def fwd_inputs(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    a = synth.grad_out_normal(M, K, seed + 2)
    return a, s, b


def check_forward(nb, a, s, b, M, N, K, splits=0, rows=None, what="", kernel="auto"):
    out = nb.forward(dev(a), dev(s), dev(b), splits=splits, kernel=kernel)
    gpu = host(out)
    if rows is not None:
        gpu = gpu[rows]
    ref, S = oracle.forward(a, s, b, M, N, K, rows=rows)
    err = np.abs(gpu.astype(np.float64) - ref)
    lim = 2e-3 * S + 1e-6
    if (err > lim).any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {int((err > lim).sum())} out of bound; worst at {i}: gpu={gpu[i]!r} "
                             f"ref={ref[i]!r} S={S[i]!r}")
    assert np.all(np.isfinite(gpu))
    # fp16-operand diagnostic
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float64)
    a16 = (a if rows is None else a[rows]).astype(np.float16).astype(np.float64)
    ref16, S16 = a16 @ w16.T, np.abs(a16) @ np.abs(w16).T
    tol = (K / 8 + 64) * 2.0 ** -24 * S16 + 1e-30
    err16 = np.abs(gpu.astype(np.float64) - ref16)
    if (err16 > tol).any():
        i = np.unravel_index(np.argmax(err16 / np.maximum(tol, 1e-300)), err16.shape)
        raise AssertionError(f"{what}: fp16-operand diagnostic failed at {i}: gpu={gpu[i]!r} ref16={ref16[i]!r}")
    return gpu


@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (5, 24, 128), (17, 136, 192), (512, 128, 64), (513, 256, 640),
                                   (700, 1000, 448), (1030, 264, 1088), (64, 256, 256)])
def test_forward_ragged_shapes(lib, M, N, K):
    """Ragged M (fragment rows padded to 16, tile rows past M), N not a multiple of the 128-column tile,
    single-stage and many-stage reductions, the default split choice."""
    a, s, b = fwd_inputs(M, N, K, seed=M + 3 * N + 7 * K)
    check_forward(lib, a, s, b, M, N, K, what=f"forward {M}x{N}x{K}")


@pytest.mark.parametrize("splits", [1, 2, 5])
@pytest.mark.parametrize("M,N,K", [(300, 256, 1024), (64, 128, 3584), (40, 48, 320)])
def test_forward_split_k(lib, splits, M, N, K):
    a, s, b = fwd_inputs(M, N, K, seed=11 * M + N + K + splits)
    check_forward(lib, a, s, b, M, N, K, splits=splits, what=f"forward s{splits} {M}x{N}x{K}")


@pytest.mark.parametrize("kernel", ["mid", "small"])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("M,N,K", [(17, 136, 192), (129, 256, 640), (300, 256, 1024), (700, 1000, 448),
                                   (1030, 264, 1088)])
def test_forward_mid_and_small_tiles(lib, kernel, splits, M, N, K):
    """256 x 128 and 128 x 128 tiles (four waves, each lane doing two lanes' decode and table work of the
    eight-wave kernel): ragged M around both tile heights, N past the last 128-column tile, K splits; within
    the bound, the fp16-operand diagnostic, and bitwise equal to the 512 x 128 tiles with the same split."""
    a, s, b = fwd_inputs(M, N, K, seed=5 * M + N + 3 * K + splits)
    got = check_forward(lib, a, s, b, M, N, K, splits=splits, kernel=kernel,
                        what=f"forward {kernel} s{splits} {M}x{N}x{K}")
    ref = host(lib.forward(dev(a), dev(s), dev(b), splits=splits, kernel="tile"))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_forward_attention_projection_config(lib):
    """The attention-projection layer (K = N = 1536) at M = 2048, oracle-packed N(0, 0.02) weights,
    activations N(0, 1), every output checked."""
    M, N, K = 2048, 1536, 1536
    w = synth.weights_normal(N, K, 0)
    s, b = oracle.pack(w, N, K)
    a = synth.grad_out_normal(M, K, seed=5)
    check_forward(lib, a, s, b, M, N, K, what="forward attn proj")


@pytest.mark.parametrize("N,K", [(3584, 3584), (18944, 3584), (3584, 18944)])
def test_forward_full_step_shapes_sampled_rows(lib, N, K):
    """Full-step layer shapes at M = 8192 in the launch configuration the planner picks; 16 sampled
    rows checked against the oracle (row-wise exact definition)."""
    M = 8192
    b = synth.random_code_bytes(N, K, seed=N + K)
    s = synth.random_scales_uniform(N, K, seed=N + K + 1)
    a = synth.grad_out_normal(M, K, seed=N + K + 2, std=1e-2)
    rows = np.random.default_rng(N + K).choice(M, size=16, replace=False)
    rows.sort()
    check_forward(lib, a, s, b, M, N, K, rows=rows, what=f"forward 8192x{N}x{K}")


def test_forward_deterministic(lib):
    M, N, K = 600, 512, 1536
    a, s, b = fwd_inputs(M, N, K, seed=91)
    ad, sd, bd = dev(a), dev(s), dev(b)
    for splits in (0, 1, 3):
        r1 = host(lib.forward(ad, sd, bd, splits=splits))
        r2 = host(lib.forward(ad, sd, bd, splits=splits))
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


@pytest.mark.parametrize("M,N,K,splits", [(16, 2048, 1536, 4), (3, 520, 1344, 5), (1, 18944, 3584, 3),
                                          (16, 3584, 18944, 17), (8, 256, 8192, 64)])
def test_forward_stream_split_sum_is_chunk_partials_in_order(lib, M, N, K, splits):
    """The streaming forward's chunk sum, done by each strip's last workgroup to finish, equals bit for bit
    the unsplit kernel run on each K-chunk alone, summed on the host in fp32 in chunk order."""
    a, s, b = fwd_inputs(M, N, K, seed=5 * M + N + K + splits)
    chunk = -(-(-(-K // splits)) // 128) * 128
    full = host(lib.forward(dev(a), dev(s), dev(b), splits=splits, kernel="stream"))
    acc = None
    for k0 in range(0, K, chunk):
        k1 = min(K, k0 + chunk)
        part = host(lib.forward(dev(a[:, k0:k1]), dev(s[:, k0 // 64:k1 // 64]), dev(b[:, k0 // 2:k1 // 2]),
                                splits=1, kernel="stream"))
        acc = part.copy() if acc is None else (acc + part).astype(np.float32)
    assert -(-K // chunk) > 1
    assert np.array_equal(full.view(np.uint32), acc.view(np.uint32))


def test_forward_stream_split_counters_across_calls(lib):
    """Split streaming calls of different strip and chunk counts back to back on one stream, interleaved with
    backward split calls (all share the workspace's arrival counters): every output written in full (outputs
    start as NaN), within the bound, and the second pass bitwise equal to the first."""
    shapes = [(16, 2048, 1536, 4), (1, 520, 1344, 5), (8, 256, 8192, 64), (16, 4096, 512, 3)]
    data = [fwd_inputs(M, N, K, seed=400 + i) for i, (M, N, K, _) in enumerate(shapes)]
    devs = [(dev(a), dev(s), dev(b)) for a, s, b in data]
    gb = dev(synth.grad_out_normal(16, 2048, seed=450))
    firsts = []
    for rnd in range(2):
        outs = []
        for (M, N, K, sp), d in zip(shapes, devs):
            o = torch.full((M, N), float("nan"), device="cuda")
            outs.append(lib.forward(*d, out=o, splits=sp, kernel="stream"))
            lib.grad_a_forced(gb, devs[0][1], devs[0][2], "stream", rb=0, splits=5)
        res = [host(o) for o in outs]
        for i, ((M, N, K, sp), (a, s, b)) in enumerate(zip(shapes, data)):
            if rnd == 0:
                ref, S = oracle.forward(a, s, b, M, N, K)
                assert np.all(np.abs(res[i].astype(np.float64) - ref) <= 2e-3 * S + 1e-6), f"shape {i}"
                firsts.append(res[i])
            else:
                assert np.array_equal(res[i].view(np.uint32), firsts[i].view(np.uint32)), f"shape {i}"


def test_forward_one_hot_rows_give_fp16_weight_columns(lib):
    M, N, K = 9, 136, 320
    b = synth.random_code_bytes(N, K, seed=93)
    s = synth.random_scales_uniform(N, K, seed=94)
    a = np.zeros((M, K), dtype=np.float32)
    picks = np.random.default_rng(95).integers(0, K, size=M)
    a[np.arange(M), picks] = 1.0
    gpu = host(lib.forward(dev(a), dev(s), dev(b)))
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float32)
    assert np.array_equal(gpu, w16[:, picks].T)


@pytest.mark.parametrize("kernel", ["tile", "mid", "small", "stream"])
def test_forward_fp16_edge_values(lib, kernel):
    """Activations at RNE ties, fp16 subnormals, values rounding to zero and +-65504 against a single unit
    weight give fp16(a) exactly; one-hot activations against weights whose scales run from 1e-7 to 65000
    (fp16 subnormal to near-maximum weights) give fp16(fl32(scale * level)) exactly; both kernels."""
    M, N, K = 16, 128, 384
    edge = np.array([0.0, -0.0, 1e-8, 2.9802322e-08, 3.0e-8, 5.9604645e-08, 1e-6, 6.0975552e-05,
                     1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, -65504.0, 65519.0, 2049.0, 0.1,
                     -0.3333333], dtype=np.float32)
    n0, k0 = 45, 201
    b = np.full((N, K // 2), 0x77, dtype=np.uint8)
    b[n0, k0 // 2] = 0xF7 if k0 % 2 else 0x7F
    s = np.ones((N, K // 64), dtype=np.float32)
    a = synth.grad_out_normal(M, K, seed=66)
    a[:, k0] = edge
    gpu = host(lib.forward(dev(a), dev(s), dev(b), splits=1, kernel=kernel))
    want = np.zeros((M, N), dtype=np.float32)
    want[:, n0] = edge.astype(np.float16).astype(np.float32)
    assert np.array_equal(gpu, want)
    b = synth.random_code_bytes(N, K, seed=67)
    scale_set = np.array([1e-7, 3e-6, 5e-5, 6.1e-5, 1.0, 3e4, 65000.0], dtype=np.float32)
    s = scale_set[np.random.default_rng(68).integers(0, len(scale_set), size=(N, K // 64))]
    a = np.zeros((M, K), dtype=np.float32)
    picks = np.random.default_rng(69).integers(0, K, size=M)
    a[np.arange(M), picks] = 1.0
    gpu = host(lib.forward(dev(a), dev(s), dev(b), splits=2, kernel=kernel))
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float32)
    assert np.all(np.isfinite(gpu))
    assert np.array_equal(gpu, w16[:, picks].T)


def test_forward_power_of_two_scaling_is_exact(lib):
    M, N, K = 40, 256, 512
    a, s, b = fwd_inputs(M, N, K, seed=97)
    a = (np.sign(a) * np.clip(np.abs(a), 2.0 ** -12, 1000.0)).astype(np.float32)  # fp16 images stay normal
    base = host(lib.forward(dev(a), dev(s), dev(b)))
    assert np.array_equal(host(lib.forward(dev(a * 2), dev(s), dev(b))), base * 2)
    assert np.array_equal(host(lib.forward(dev(a), dev(s * np.float32(0.5)), dev(b))), base * 0.5)


def test_forward_and_grad_a_are_adjoint_on_the_gpu(lib):
    """<forward(A), X> = <A, grad_a(X)> up to the two products' bounds."""
    M, N, K = 48, 704, 384
    b = synth.random_code_bytes(N, K, seed=98)
    s = synth.random_scales_uniform(N, K, seed=99)
    a = synth.grad_out_normal(M, K, seed=100)
    x = synth.grad_out_normal(M, N, seed=101)
    c = host(lib.forward(dev(a), dev(s), dev(b))).astype(np.float64)
    ga = host(lib.grad_a(dev(x), dev(s), dev(b))).astype(np.float64)
    _, Sf = oracle.forward(a, s, b, M, N, K)
    _, Sg = oracle.grad_a(x, s, b, M, N, K)
    lhs = np.sum(c * x)
    rhs = np.sum(a.astype(np.float64) * ga)
    lim = np.sum(np.abs(x) * (2e-3 * Sf + 1e-6)) + np.sum(np.abs(a) * (2e-3 * Sg + 1e-6))
    assert abs(lhs - rhs) <= lim


def test_forward_empty_and_rejected_shapes(lib):
    s = dev(np.ones((8, 1), dtype=np.float32))
    b = dev(np.full((8, 32), 0xFF, dtype=np.uint8))
    # K == 0: an empty sum, zeros written
    out = dev(np.full((3, 8), 7.0, dtype=np.float32))
    lib.forward(dev(np.zeros((3, 0), dtype=np.float32)), dev(np.zeros((8, 0), dtype=np.float32)),
                dev(np.zeros((8, 0), dtype=np.uint8)), out=out)
    assert np.all(host(out) == 0.0)
    # M == 0: nothing to do
    r = lib.forward(dev(np.zeros((0, 64), dtype=np.float32)), s, b)
    assert tuple(r.shape) == (0, 8)
    # N % 8 != 0 and K % 64 != 0 are rejected before any launch
    with pytest.raises(lib.Nf4Error):
        lib.forward(dev(np.ones((2, 64), dtype=np.float32)), dev(np.ones((4, 1), dtype=np.float32)),
                    dev(np.zeros((4, 32), dtype=np.uint8)))
    st = lib._lib.nf4_forward(dev(np.ones((2, 96), dtype=np.float32)).data_ptr(), s.data_ptr(), b.data_ptr(),
                              dev(np.zeros((2, 8), dtype=np.float32)).data_ptr(), 2, 8, 96,
                              torch.cuda.current_stream().cuda_stream)
    assert st == lib.NF4_ERR_SHAPE


# --- streaming kernel (1 <= M <= 16) -------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (3, 72, 192), (8, 64, 512), (16, 200, 640), (5, 1000, 448),
                                   (16, 3584, 512), (7, 128, 3584)])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_forward_stream_ragged_and_split(lib, M, N, K, splits):
    """16-column wave strips with N tails (rows past N read as zero), K % 128 == 64 (a half step at the
    end of K), one to many 128-wide steps per chunk, every K chunking."""
    a, s, b = fwd_inputs(M, N, K, seed=5 * M + N + 3 * K + splits)
    out = lib.forward(dev(a), dev(s), dev(b), splits=splits, kernel="stream")
    gpu = host(out)
    ref, S = oracle.forward(a, s, b, M, N, K)
    lim = 2e-3 * S + 1e-6
    err = np.abs(gpu.astype(np.float64) - ref)
    assert (err <= lim).all(), f"stream s{splits} {M}x{N}x{K}: worst {np.max(err / lim)}"
    w16 = oracle.dequant(s, b, N, K).astype(np.float16).astype(np.float64)
    a16 = a.astype(np.float16).astype(np.float64)
    ref16, S16 = a16 @ w16.T, np.abs(a16) @ np.abs(w16).T
    assert (np.abs(gpu - ref16) <= (K / 8 + 64) * 2.0 ** -24 * S16 + 1e-30).all()


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("N,K", [(18944, 3584), (3584, 18944)])
def test_forward_stream_skinny_configs_full(lib, M, N, K):
    """The skinny sweep's layer shapes in the forward orientation, default plan, every output checked."""
    b = synth.random_code_bytes(N, K, seed=N + M)
    s = synth.random_scales_uniform(N, K, seed=N + M + 1)
    a = synth.grad_out_normal(M, K, seed=N + M + 2)
    check_forward(lib, a, s, b, M, N, K, what=f"forward stream {M}x{N}x{K}")


def test_forward_stream_default_equals_forced_plan_bitwise(lib):
    """The default plan for M <= 16 is the streaming kernel with the planner's split; forcing the same split
    reproduces it bit for bit, and repeated calls are bitwise equal."""
    M, N, K = 16, 3584, 18944
    a, s, b = fwd_inputs(M, N, K, seed=123)
    ad, sd, bd = dev(a), dev(s), dev(b)
    base = host(lib.forward(ad, sd, bd))
    again = host(lib.forward(ad, sd, bd))
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))
    found = False
    for sp in range(1, 65):  # the planner considers 1 .. 64 chunks
        r = host(lib.forward(ad, sd, bd, splits=sp, kernel="stream"))
        if np.array_equal(r.view(np.uint32), base.view(np.uint32)):
            found = True
            break
    assert found


def test_forward_stream_rejects_large_m(lib):
    a = dev(np.ones((17, 64), dtype=np.float32))
    s = dev(np.ones((8, 1), dtype=np.float32))
    b = dev(np.zeros((8, 32), dtype=np.uint8))
    with pytest.raises(lib.Nf4Error):
        lib.forward(a, s, b, splits=1, kernel="stream")


@pytest.mark.parametrize("M", [1, 8, 16])
def test_forward_grouped_matches_separate_calls(lib, M):
    """M <= 16: the streaming problems of a group run as one grid, each bitwise equal to its own nf4_forward
    call (split and unsplit chunk plans, K % 128 == 64); N == 0 and K == 0 problems keep their contracts;
    every output within the bound.  Run twice: the second pass reuses the arrival counters."""
    shapes = [(2048, 1536), (520, 1344), (4096, 384), (96, 64), (0, 128), (256, 0), (18944, 3584), (3584, 18944)]
    data = [fwd_inputs(M, N, K, seed=13 * M + N + K) for (N, K) in shapes]
    devs = [(dev(a), dev(s), dev(b)) for a, s, b in data]
    seps = [host(lib.forward(*d)) for d in devs]
    for rnd in range(2):
        outs = [torch.full((M, N), float("nan"), device="cuda") for (N, K) in shapes]
        lib.forward_grouped(devs, outs=outs)
        for (N, K), (a, s, b), o, sep in zip(shapes, data, outs, seps):
            gpu = host(o)
            assert np.array_equal(gpu.view(np.uint32), sep.view(np.uint32)), (rnd, M, N, K)
            if rnd == 0 and N * K <= 4096 * 1536:
                ref, S = oracle.forward(a, s, b, M, N, K)
                assert np.all(np.abs(gpu.astype(np.float64) - ref) <= 2e-3 * S + 1e-6), (M, N, K)


def test_forward_grouped_shares_the_conversion_of_common_activations(lib):
    """M > 16: problems with the same activations (q, k, v of a layer; gate and up) share one conversion of `a`
    inside the grouped call; every result is bitwise that of its own nf4_forward call, including problems
    whose plan splits K (partials reused between problems) and an unshared one in between."""
    M = 600
    x = dev(synth.grad_out_normal(M, 448, seed=81))
    y = dev(synth.grad_out_normal(M, 320, seed=82))
    ws = []
    for j, (N, K) in enumerate([(512, 448), (128, 448), (128, 448), (264, 320), (1024, 448), (1024, 320)]):
        _, s, b = fwd_inputs(1, N, K, seed=90 + j)
        ws.append((dev(s), dev(b)))
    problems = [(x,) + ws[0], (x,) + ws[1], (x,) + ws[2], (y,) + ws[3], (x,) + ws[4], (y,) + ws[5]]
    outs = lib.forward_grouped(problems)
    for p, o in zip(problems, outs):
        ref = host(lib.forward(*p))
        assert np.array_equal(host(o).view(np.uint32), ref.view(np.uint32))
    a, s, b = host(x), host(ws[0][0]), host(ws[0][1])
    check_forward(lib, a, s, b, M, 512, 448, what="grouped shared-a problem 0")


def test_forward_grouped_large_m_and_errors(lib):
    """M > 16 problems run as nf4_forward runs them; more than 8 problems and mixed M are rejected."""
    M = 40
    shapes = [(256, 512), (136, 320)]
    data = [fwd_inputs(M, N, K, seed=70 + N) for (N, K) in shapes]
    devs = [(dev(a), dev(s), dev(b)) for a, s, b in data]
    outs = lib.forward_grouped(devs)
    for d, o in zip(devs, outs):
        assert np.array_equal(host(o).view(np.uint32), host(lib.forward(*d)).view(np.uint32))
    assert lib.forward_grouped([]) == []
    with pytest.raises(ValueError):
        lib.forward_grouped([devs[0]] * 9)
    a2 = dev(synth.grad_out_normal(8, 512, seed=1))
    with pytest.raises(ValueError):
        lib.forward_grouped([devs[0], (a2, devs[0][1], devs[0][2])])
