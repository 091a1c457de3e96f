"""nf4_grad_a_noalloc through the C ABI: the entry point for callers that cannot allocate.

It runs nf4_grad_a's launch plan with its scratch (split partials, arrival
counters, fp16 A fragments) in the library's static device array, so its
results must equal nf4_grad_a's bit for bit, and lie within the oracle's bound
|gpu - ref| <= 2e-3 * S + 1e-6.  Calls follow each other on one stream with
different, then smaller, shapes: the array keeps the previous call's contents,
so a call that did not clear or fully rewrite what it reads would show up.
A shape whose plan needs more scratch than the array holds is refused with
NF4_ERR_SCRATCH and leaves its output untouched.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    return g, s, b


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# pairs of calls in a row, the second smaller, over the kinds of plan nf4_grad_a makes: the streaming kernel
# with its in-kernel split sum (9, then 8 N-chunks sharing the arrival counters); 256 x 128 tiles with fp16 A
# fragments and 8 N-chunks of partials in the scratch, twice; 128 x 128 tiles unsplit (fragments only), then
# 256 x 128 tiles unsplit; 256 x 128 tiles in 4 N-chunks, then 128 x 128 tiles unsplit
SEQUENCES = [
    [(16, 18944, 3584), (4, 3000, 512)],
    [(600, 2048, 768), (100, 1024, 384)],
    [(2048, 1536, 1536), (1030, 256, 1088)],
    [(1024, 3584, 3584), (300, 1024, 3584)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join("x".join(map(str, c)) for c in s))
def test_noalloc_matches_nf4_grad_a_on_calls_in_a_row(lib, seq):
    for i, (M, N, K) in enumerate(seq):
        g, s, b = _inputs(M, N, K, seed=1000 + 10 * i + M)
        gd, sd, bd = _dev(g), _dev(s), _dev(b)
        want = lib.grad_a(gd, sd, bd)
        out = torch.full((M, K), float("nan"), device="cuda")
        lib.grad_a_noalloc(gd, sd, bd, out)
        torch.cuda.synchronize()
        got, ref_out = out.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref_out.view(np.uint32)), (i, M, N, K)
        ref, S = oracle.grad_a(g, s, b, M, N, K)
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= 2e-3 * S + 1e-6), (i, M, N, K, float(np.max(err / (2e-3 * S + 1e-6))))


def test_noalloc_refuses_a_plan_larger_than_its_scratch(lib):
    M, N, K = 4096, 18944, 3584  # fp16 A fragments alone: 2 * 4096 * 18944 bytes = 148 MiB > 128 MiB
    plan = lib.grad_a_plan(M, N, K)
    assert plan["kernel"] == "wide16"
    gd = torch.zeros((M, N), device="cuda")
    sd = torch.ones((N, K // 64), device="cuda")
    bd = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    out = torch.full((M, K), float("nan"), device="cuda")
    with pytest.raises(lib.Nf4Error) as ei:
        lib.grad_a_noalloc(gd, sd, bd, out)
    assert ei.value.status == lib.NF4_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # a small call afterwards still works
    g, s, b = _inputs(64, 256, 256, seed=5)
    o = torch.empty((64, 256), device="cuda")
    lib.grad_a_noalloc(_dev(g), _dev(s), _dev(b), o)
    ref, S = oracle.grad_a(g, s, b, 64, 256, 256)
    assert np.all(np.abs(o.cpu().numpy().astype(np.float64) - ref) <= 2e-3 * S + 1e-6)
