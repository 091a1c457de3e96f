"""Race check of the kernels' LDS use: the race-check build against the release build, bit for bit.

The race-check build (``libnf4bwd_barriers.so``, the same sources compiled with
NF4_EXTRA_BARRIERS) separates every LDS phase of every kernel with an extra
barrier -- a workgroup barrier between the ticks of the wide and forward
kernels' stages, a wave-level drain around the streaming kernel's private
tables -- so no wave can read LDS that another wave (or the same wave's
later phase) has not finished writing or reading.  The release kernels rely
on one barrier per stage and on the order of their own accesses; if one of
those orderings were missing, the release build's results would depend on
timing, and would differ from the race-check build's.  Every kernel variant
is called through the C ABI of both libraries on the same inputs (ragged
tails, N splits) and the outputs must be bitwise equal.
"""

import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KERNELS = {"tile": 0, "skinny": 1, "wide": 3, "stream": 4, "wide16": 5, "unfused": 6, "mid": 9, "small": 10}


@pytest.fixture(scope="module")
def libs(lib):
    return lib._lib, lib.load_library(lib.BARRIER_LIB_PATH)


def _inputs(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (g, s, b)]


def _grad_a(cl, g, s, b, M, N, K, kernel, rb, splits):
    out = torch.full((M, K), float("nan"), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = cl.nf4_grad_a_forced(g.data_ptr(), s.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, KERNELS[kernel],
                              rb, splits, ctypes.c_void_p(st))
    assert rc == 0, rc
    return out


CASES = [
    ("tile", 1, 1, 200, 384, 768), ("tile", 2, 2, 513, 640, 256), ("tile", 1, 3, 300, 100, 320),
    ("skinny", 0, 3, 16, 1000, 512), ("skinny", 0, 1, 5, 200, 192),
    ("stream", 0, 1, 16, 3000, 512), ("stream", 0, 5, 8, 4100, 384), ("stream", 0, 3, 1, 257, 320),
    ("wide", 1, 1, 600, 1024, 448), ("wide", 1, 3, 1030, 256, 1088),
    ("wide16", 1, 1, 1030, 2048, 384), ("wide16", 1, 2, 513, 640, 320), ("wide16", 1, 1, 31, 128, 128),
    ("unfused", 1, 2, 600, 1024, 448),
    ("mid", 1, 1, 600, 1024, 448), ("mid", 3, 2, 513, 640, 320), ("mid", 1, 3, 1030, 256, 1088),
    ("small", 1, 1, 600, 1024, 448), ("small", 1, 2, 129, 640, 320),
]


@pytest.mark.parametrize("kernel,rb,splits,M,N,K", CASES)
def test_race_check_build_matches_release_grad_a(libs, kernel, rb, splits, M, N, K):
    rel, chk = libs
    g, s, b = _inputs(M, N, K, seed=M + 3 * N + K + splits)
    a = _grad_a(rel, g, s, b, M, N, K, kernel, rb, splits)
    c = _grad_a(chk, g, s, b, M, N, K, kernel, rb, splits)
    torch.cuda.synchronize()
    assert not torch.isnan(a).any()
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


@pytest.mark.parametrize("kernel,splits,M,N,K", [(0, 1, 600, 1024, 448), (0, 3, 1030, 520, 1088),
                                                 (1, 1, 16, 2048, 1536), (1, 3, 5, 520, 1344),
                                                 (2, 1, 600, 1024, 448), (2, 2, 257, 520, 640),
                                                 (3, 1, 600, 1024, 448), (3, 3, 129, 264, 1088)])
def test_race_check_build_matches_release_forward(libs, kernel, splits, M, N, K):
    rel, chk = libs
    _, s, b = _inputs(1, N, K, seed=M + N + K)
    a = torch.randn((M, K), device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for cl in (rel, chk):
        c = torch.full((M, N), float("nan"), device="cuda")
        rc = cl.nf4_forward_forced(a.data_ptr(), s.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, kernel, splits, st)
        assert rc == 0, rc
        outs.append(c)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
