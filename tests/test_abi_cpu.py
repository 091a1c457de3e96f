"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, validates arguments before touching the device, and plans
launches on the host."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(nf4_\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def nb():
    import dequant_backward_gemm_amd as nb
    return nb


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("nf4_grad_a", "nf4_dequant", "nf4_pack", "nf4_status_string"):
        assert want in names, names


def test_library_exports_every_declared_symbol(nb):
    lib = ctypes.CDLL(nb.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) <= set(nb.EXPORTED_SYMBOLS) | {"nf4_status_string"}


def test_status_strings(nb):
    for s in range(7):
        assert nb.status_string(s) and "unknown" not in nb.status_string(s)
    assert "capture" in nb.status_string(nb.NF4_ERR_CAPTURE)
    assert "scratch" in nb.status_string(nb.NF4_ERR_SCRATCH)
    assert "unknown" in nb.status_string(99)


def test_validation_runs_before_any_device_work(nb):
    # Bogus but aligned non-null addresses: validation must reject before use.
    p = 0x1000
    hs = None
    # K not a multiple of 64
    assert nb.grad_a_raw(p, p, p, p, 4, 4, 65, hs) == nb.NF4_ERR_SHAPE
    assert nb.dequant_raw(p, p, p, 4, 100, hs) == nb.NF4_ERR_SHAPE
    assert nb.pack_raw(p, p, p, 4, 32, hs) == nb.NF4_ERR_SHAPE
    # negative sizes
    assert nb.grad_a_raw(p, p, p, p, -1, 4, 64, hs) == nb.NF4_ERR_SHAPE
    assert nb.grad_a_raw(p, p, p, p, 4, -4, 64, hs) == nb.NF4_ERR_SHAPE
    assert nb.dequant_raw(p, p, p, -1, 64, hs) == nb.NF4_ERR_SHAPE
    # sizes beyond the index range
    assert nb.grad_a_raw(p, p, p, p, 1 << 31, 4, 64, hs) == nb.NF4_ERR_SHAPE
    # null pointers with non-empty arrays
    assert nb.grad_a_raw(None, p, p, p, 4, 4, 64, hs) == nb.NF4_ERR_NULL
    assert nb.grad_a_raw(p, None, p, p, 4, 4, 64, hs) == nb.NF4_ERR_NULL
    assert nb.grad_a_raw(p, p, None, p, 4, 4, 64, hs) == nb.NF4_ERR_NULL
    assert nb.grad_a_raw(p, p, p, None, 4, 4, 64, hs) == nb.NF4_ERR_NULL
    assert nb.dequant_raw(None, p, p, 4, 64, hs) == nb.NF4_ERR_NULL
    assert nb.pack_raw(p, p, None, 4, 64, hs) == nb.NF4_ERR_NULL
    # misaligned pointers
    assert nb.grad_a_raw(p + 4, p, p, p, 4, 4, 64, hs) == nb.NF4_ERR_ALIGN
    assert nb.grad_a_raw(p, p, p, p + 8, 4, 4, 64, hs) == nb.NF4_ERR_ALIGN
    assert nb.dequant_raw(p, p + 1, p, 4, 64, hs) == nb.NF4_ERR_ALIGN
    assert nb.pack_raw(p + 2, p, p, 4, 64, hs) == nb.NF4_ERR_ALIGN
    # empty problems: nothing to do, nothing enqueued, even with null pointers
    assert nb.grad_a_raw(None, None, None, None, 0, 4, 64, hs) == nb.NF4_OK
    assert nb.grad_a_raw(None, None, None, None, 4, 4, 0, hs) == nb.NF4_OK
    assert nb.dequant_raw(None, None, None, 0, 64, hs) == nb.NF4_OK
    assert nb.pack_raw(None, None, None, 4, 0, hs) == nb.NF4_OK
    # N == 0 needs only the output pointer
    assert nb.grad_a_raw(None, None, None, None, 4, 0, 64, hs) == nb.NF4_ERR_NULL


@pytest.mark.parametrize("M,N,K", [(1, 18944, 3584), (16, 3584, 18944), (64, 256, 256), (2048, 1536, 1536),
                                   (1100, 1024, 1088), (1024, 1536, 1536),
                                   (4096, 8960, 1536), (4096, 1536, 8960), (8192, 512, 3584), (8192, 18944, 3584),
                                   (8192, 3584, 18944), (17, 100, 192), (3, 0, 64)])
def test_plan_is_consistent(nb, M, N, K):
    _check_plan(nb, M, N, K)


def test_plan_is_consistent_on_random_shapes(nb):
    """The same invariants over 2000 seeded random shapes, from skinny to the full step's sizes, N ragged or a
    multiple of 64, K any multiple of 64 (host-only: the planner runs no device work)."""
    rng = np.random.default_rng(77)
    for _ in range(2000):
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 600), rng.integers(600, 9000)]))
        N = int(rng.choice([rng.integers(0, 20000), 64 * rng.integers(1, 300)]))
        K = 64 * int(rng.integers(1, 300))
        _check_plan(nb, M, N, K)


def _check_plan(nb, M, N, K):
    p = nb.grad_a_plan(M, N, K)
    if N == 0:
        assert p["kernel"] == "zero_fill"
        return
    if M <= 16:
        assert p["kernel"] in ("skinny", "stream")
    else:
        assert p["kernel"] in ("tile", "wide", "wide16", "mid", "small")
    if p["kernel"] in ("wide", "wide16", "mid", "small"):  # only where the wide kernel's preconditions hold
        assert N % 64 == 0 and M * N * 4 < 2 ** 31 and N * K // 2 < 2 ** 31
    assert p["splits"] >= 1
    assert p["n_chunk"] * p["splits"] >= N > p["n_chunk"] * (p["splits"] - 1)
    tiles_k = -(-K // 256)
    if p["kernel"] == "skinny":
        assert p["n_chunk"] % 128 == 0
        assert p["grid"] == tiles_k * p["splits"]
    elif p["kernel"] == "stream":
        assert p["n_chunk"] % 32 == 0
        assert p["grid"] == -(-K // 128) * p["splits"]
    elif p["kernel"] == "tile":
        assert p["n_chunk"] % 64 == 0
        bm = 128 * p["rb"]
        assert p["grid"] == -(-M // bm) * tiles_k * p["splits"]
    else:
        assert p["n_chunk"] % 64 == 0 and p["rb"] == 1
        bm, bk = {"mid": 256, "small": 128}.get(p["kernel"], 512), 128
        assert p["grid"] == -(-M // bm) * -(-K // bk) * p["splits"]


@pytest.mark.parametrize("M,N,K,kernel,splits", [
    (8192, 3584, 3584, "wide16", 1), (8192, 512, 3584, "mid", 1), (8192, 18944, 3584, "wide16", 1),
    (8192, 3584, 18944, "wide16", 1), (2048, 1536, 1536, "small", 1), (4096, 8960, 1536, "wide16", 2),
    (4096, 1536, 8960, "mid", 1), (1, 18944, 3584, "stream", 9), (16, 3584, 18944, "stream", 3)])
def test_plan_choices_of_the_configurations(nb, M, N, K, kernel, splits):
    """The plans measured fastest on MI355X for the benchmark's configurations (the full step's projections,
    the attention projection, the MLP pair, the skinny sweep): a change of the cost model that moves one of
    them has to be measured again."""
    p = nb.grad_a_plan(M, N, K)
    assert (p["kernel"], p["splits"]) == (kernel, splits), p



def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says why, before touching any device."""
    import subprocess
    import sys
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(here, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
