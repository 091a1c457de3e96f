"""Python binding over the NF4 input-gradient C ABI (``include/nf4bwd.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libnf4bwd.so``.  PyTorch supplies device memory and the current
stream.  Importing this module loads the in-tree library and fails loudly if
it is missing; there is no fallback of any kind.

    grad_a(grad_out, scales, codes)          -> fp32 [M, K]
    grad_a_grouped([(grad_out, scales, codes), ...])  -> [fp32 [M, K_i], ...]  (shared M, up to 8)
    forward(a, scales, codes)                -> fp32 [M, N]   (the same layer's forward product)
    forward_grouped([(a, scales, codes), ...])  -> [fp32 [M, N_i], ...]  (shared M, up to 8)
    dequant(scales, codes, N, K)             -> fp32 [N, K]
    pack(w)                                  -> (scales fp32 [N, K/64], codes uint8 [N, K/2])
    rms_norm_backward(x, gamma, rms, dy)     -> (dx fp32 [rows, H], dgamma fp32 [H])
    grad_a_plan(M, N, K), grad_a_forced(...), release_workspaces()

Tensors must be contiguous, on the current CUDA (HIP) device, 16-byte
aligned, with the dtypes and shapes the C ABI states.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libnf4bwd.so")
# the race-check build (every LDS phase separated by an extra barrier); tests only
BARRIER_LIB_PATH = os.path.join(_PKG_DIR, "libnf4bwd_barriers.so")

NF4_OK, NF4_ERR_NULL, NF4_ERR_SHAPE, NF4_ERR_ALIGN, NF4_ERR_HIP, NF4_ERR_CAPTURE, NF4_ERR_SCRATCH = 0, 1, 2, 3, 4, 5, 6
NOALLOC_SCRATCH_BYTES = 128 << 20

EXPORTED_SYMBOLS = ("nf4_grad_a", "nf4_dequant", "nf4_pack", "nf4_status_string", "nf4_grad_a_plan",
                    "nf4_grad_a_forced", "nf4_release_workspaces", "nf4_forward", "nf4_forward_forced",
                    "nf4_grad_a_grouped", "nf4_rms_norm_backward", "nf4_forward_grouped", "nf4_grad_a_noalloc")
GROUP_MAX = 8


class _Problem(ctypes.Structure):
    _fields_ = [("grad_out", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("grad_a", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _ForwardProblem(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("c", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class Nf4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load a build of the C-ABI library (the release one by default) with its argument types declared."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python dequant_backward_gemm_amd/build.py` "
            "(hipcc, gfx950). There is no CPU fallback.")
    # One HIP runtime per process: PyTorch ships its own libamdhip64, and the
    # library must bind to that copy, since it works on torch's memory and
    # streams.  Loaded first, the library would pull in the system runtime,
    # and every launch on torch's memory would then fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.nf4_grad_a.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.nf4_grad_a.restype = ctypes.c_int
    lib.nf4_grad_a_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.nf4_grad_a_noalloc.restype = ctypes.c_int
    lib.nf4_dequant.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.nf4_dequant.restype = ctypes.c_int
    lib.nf4_pack.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.nf4_pack.restype = ctypes.c_int
    lib.nf4_status_string.argtypes = [ctypes.c_int]
    lib.nf4_status_string.restype = ctypes.c_char_p
    lib.nf4_grad_a_plan.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int)]
    lib.nf4_grad_a_plan.restype = ctypes.c_int
    ci = ctypes.c_int
    lib.nf4_grad_a_forced.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, vp]
    lib.nf4_grad_a_forced.restype = ctypes.c_int
    lib.nf4_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.nf4_forward.restype = ctypes.c_int
    lib.nf4_forward_forced.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.nf4_forward_forced.restype = ctypes.c_int
    lib.nf4_forward_grouped.argtypes = [vp, ci, i64, vp]
    lib.nf4_forward_grouped.restype = ctypes.c_int
    lib.nf4_rms_norm_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp]
    lib.nf4_rms_norm_backward.restype = ctypes.c_int
    lib.nf4_grad_a_grouped.argtypes = [ctypes.c_void_p, ci, i64, vp]
    lib.nf4_grad_a_grouped.restype = ctypes.c_int
    lib.nf4_release_workspaces.argtypes = []
    lib.nf4_release_workspaces.restype = ctypes.c_int
    return lib


_lib = load_library(LIB_PATH)


def status_string(status: int) -> str:
    return _lib.nf4_status_string(int(status)).decode()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        # the raw-handle query skips building a Stream object (a few us per call)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, what: str) -> None:
    if status != NF4_OK:
        raise Nf4Error(status, what)


def _require(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def grad_a_raw(grad_out_ptr, scales_ptr, codes_ptr, grad_a_ptr, M, N, K, stream_handle) -> int:
    """Direct C-ABI call with raw pointers; returns the nf4_status."""
    return _lib.nf4_grad_a(grad_out_ptr, scales_ptr, codes_ptr, grad_a_ptr, M, N, K, stream_handle)


def dequant_raw(scales_ptr, codes_ptr, w_ptr, N, K, stream_handle) -> int:
    return _lib.nf4_dequant(scales_ptr, codes_ptr, w_ptr, N, K, stream_handle)


def pack_raw(w_ptr, scales_ptr, codes_ptr, N, K, stream_handle) -> int:
    return _lib.nf4_pack(w_ptr, scales_ptr, codes_ptr, N, K, stream_handle)


def grad_a(grad_out, scales, codes, out=None, stream=None):
    """grad_A[M, K] = grad_out[M, N] . dequant(codes, scales)[N, K] (fp32)."""
    import torch
    M, N = grad_out.shape
    K = codes.shape[1] * 2
    _require(grad_out, torch.float32, (M, N), "grad_out")
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=grad_out.device)
    _require(out, torch.float32, (M, K), "out")
    _check(grad_a_raw(_ptr(grad_out), _ptr(scales), _ptr(codes), _ptr(out), M, N, K, _stream_handle(stream)),
           "nf4_grad_a")
    return out


def grad_a_noalloc(grad_out, scales, codes, out, stream=None):
    """grad_a through nf4_grad_a_noalloc: no device allocation by the library (its scratch is a static
    device array); `out` must be given.  Raises Nf4Error (status NF4_ERR_SCRATCH) when the shape needs more
    scratch than that array holds."""
    import torch
    M, N = grad_out.shape
    K = codes.shape[1] * 2
    _require(grad_out, torch.float32, (M, N), "grad_out")
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    _require(out, torch.float32, (M, K), "out")
    _check(_lib.nf4_grad_a_noalloc(_ptr(grad_out), _ptr(scales), _ptr(codes), _ptr(out), M, N, K,
                                   _stream_handle(stream)), "nf4_grad_a_noalloc")
    return out


def grad_a_grouped(problems, outs=None, stream=None):
    """grad_A of several problems sharing M in as few launches as possible.

    problems: sequence of (grad_out [M, N], scales [N, K/64], codes [N, K/2]); returns the list of grad_A
    [M, K] tensors (or fills `outs`)."""
    import torch
    if len(problems) > GROUP_MAX:
        raise ValueError(f"at most {GROUP_MAX} problems per group")
    arr = (_Problem * max(1, len(problems)))()
    res = []
    M = problems[0][0].shape[0] if problems else 0
    for i, (g, s, c) in enumerate(problems):
        Mi, N = g.shape
        K = c.shape[1] * 2
        if Mi != M:
            raise ValueError("all problems of a group share M")
        _require(g, torch.float32, (M, N), "grad_out")
        _require(s, torch.float32, (N, K // 64), "scales")
        _require(c, torch.uint8, (N, K // 2), "codes")
        o = outs[i] if outs is not None else torch.empty((M, K), dtype=torch.float32, device=g.device)
        _require(o, torch.float32, (M, K), "out")
        arr[i] = _Problem(_ptr(g), _ptr(s), _ptr(c), _ptr(o), N, K)
        res.append(o)
    _check(_lib.nf4_grad_a_grouped(ctypes.cast(arr, ctypes.c_void_p), len(problems), M, _stream_handle(stream)),
           "nf4_grad_a_grouped")
    return res


def grad_a_forced(grad_out, scales, codes, kernel: str, rb: int = 2, splits: int = 1, out=None, stream=None):
    """grad_a with a forced launch plan (kernel "tile", "skinny", "wide", "stream", "wide16", "unfused": the
    comparison path with a separate fp16 dequant pass, "lines": line streaming with `rb` of each lane's 4
    rows decoded in registers, "mid": 256 x 128 tiles with `rb` k-steps of A fragments in flight, or
    "small": 128 x 128 tiles, `rb` 1); for tests and tuning."""
    import torch
    M, N = grad_out.shape
    K = codes.shape[1] * 2
    _require(grad_out, torch.float32, (M, N), "grad_out")
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=grad_out.device)
    _require(out, torch.float32, (M, K), "out")
    kid = {"tile": 0, "skinny": 1, "wide": 3, "stream": 4, "wide16": 5, "unfused": 6, "lines": 8, "mid": 9,
           "small": 10}[kernel]
    _check(_lib.nf4_grad_a_forced(_ptr(grad_out), _ptr(scales), _ptr(codes), _ptr(out), M, N, K, kid, rb, splits,
                                  _stream_handle(stream)), "nf4_grad_a_forced")
    return out


FORWARD_KERNELS = {"tile": 0, "stream": 1, "mid": 2, "small": 3}


def forward(a, scales, codes, out=None, stream=None, splits: int = 0, kernel: str = "auto"):
    """c[M, N] = a[M, K] . dequant(codes, scales)[N, K]^T (fp32).

    splits > 0 forces the K chunk count; kernel "tile" (512 x 128 tiles), "mid" (256 x 128), "small"
    (128 x 128) or "stream" forces the kernel ("auto" with a forced split count takes streaming for
    M <= 16, 512 x 128 tiles otherwise)."""
    import torch
    M, K = a.shape
    N = codes.shape[0]
    _require(a, torch.float32, (M, K), "a")
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _require(out, torch.float32, (M, N), "out")
    if splits > 0 or kernel != "auto":
        if kernel == "auto":
            kernel = "stream" if 1 <= M <= 16 else "tile"
        st = _lib.nf4_forward_forced(_ptr(a), _ptr(scales), _ptr(codes), _ptr(out), M, N, K,
                                     FORWARD_KERNELS[kernel], max(splits, 1), _stream_handle(stream))
    else:
        st = _lib.nf4_forward(_ptr(a), _ptr(scales), _ptr(codes), _ptr(out), M, N, K, _stream_handle(stream))
    _check(st, "nf4_forward")
    return out


def forward_grouped(problems, outs=None, stream=None):
    """Forward products of several problems sharing M in as few launches as possible (M <= 16: one grid of the
    streaming kernel; larger M: problems with the same `a` tensor share one conversion of it), each result
    bitwise that of forward().

    problems: sequence of (a [M, K], scales [N, K/64], codes [N, K/2]); returns the list of c [M, N] tensors
    (or fills `outs`)."""
    import torch
    if len(problems) > GROUP_MAX:
        raise ValueError(f"at most {GROUP_MAX} problems per group")
    arr = (_ForwardProblem * max(1, len(problems)))()
    res = []
    M = problems[0][0].shape[0] if problems else 0
    for i, (a, s, c) in enumerate(problems):
        Mi, K = a.shape
        N = c.shape[0]
        if Mi != M:
            raise ValueError("all problems of a group share M")
        _require(a, torch.float32, (M, K), "a")
        _require(s, torch.float32, (N, K // 64), "scales")
        _require(c, torch.uint8, (N, K // 2), "codes")
        o = outs[i] if outs is not None else torch.empty((M, N), dtype=torch.float32, device=a.device)
        _require(o, torch.float32, (M, N), "out")
        arr[i] = _ForwardProblem(_ptr(a), _ptr(s), _ptr(c), _ptr(o), N, K)
        res.append(o)
    _check(_lib.nf4_forward_grouped(ctypes.cast(arr, ctypes.c_void_p), len(problems), M, _stream_handle(stream)),
           "nf4_forward_grouped")
    return res


def rms_norm_backward(x, gamma, rms, dy, dx=None, dgamma=None, stream=None):
    """(dx [rows, H], dgamma [H]) of RMSNorm; rms is the forward pass's sqrt(mean(x^2) + eps) per row."""
    import torch
    rows, H = x.shape
    _require(x, torch.float32, (rows, H), "x")
    _require(gamma, torch.float32, (H,), "gamma")
    _require(rms, torch.float32, (rows,), "rms")
    _require(dy, torch.float32, (rows, H), "dy")
    if dx is None:
        dx = torch.empty((rows, H), dtype=torch.float32, device=x.device)
    if dgamma is None:
        dgamma = torch.empty((H,), dtype=torch.float32, device=x.device)
    _require(dx, torch.float32, (rows, H), "dx")
    _require(dgamma, torch.float32, (H,), "dgamma")
    _check(_lib.nf4_rms_norm_backward(_ptr(x), _ptr(gamma), _ptr(rms), _ptr(dy), _ptr(dx), _ptr(dgamma), rows, H,
                                      _stream_handle(stream)), "nf4_rms_norm_backward")
    return dx, dgamma


def dequant(scales, codes, out=None, stream=None):
    """w[N, K] = fl32(scales[n, k/64] * NF4[code(n, k)])."""
    import torch
    N = codes.shape[0]
    K = codes.shape[1] * 2
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    _require(out, torch.float32, (N, K), "out")
    _check(dequant_raw(_ptr(scales), _ptr(codes), _ptr(out), N, K, _stream_handle(stream)), "nf4_dequant")
    return out


def pack(w, scales=None, codes=None, stream=None):
    """NF4-quantise fp32 weights w[N, K] -> (scales [N, K/64], codes [N, K/2])."""
    import torch
    N, K = w.shape
    _require(w, torch.float32, (N, K), "w")
    if scales is None:
        scales = torch.empty((N, K // 64), dtype=torch.float32, device=w.device)
    if codes is None:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    _require(scales, torch.float32, (N, K // 64), "scales")
    _require(codes, torch.uint8, (N, K // 2), "codes")
    _check(pack_raw(_ptr(w), _ptr(scales), _ptr(codes), N, K, _stream_handle(stream)), "nf4_pack")
    return scales, codes


def release_workspaces() -> None:
    """Free the library's cached split-N workspaces (waits for the devices that hold one)."""
    _check(_lib.nf4_release_workspaces(), "nf4_release_workspaces")


def grad_a_plan(M: int, N: int, K: int) -> dict:
    """Launch plan nf4_grad_a uses for a shape (host-only, no device work)."""
    out = (ctypes.c_int * 5)()
    _check(_lib.nf4_grad_a_plan(M, N, K, out), "nf4_grad_a_plan")
    kernel = {0: "tile", 1: "skinny", 2: "zero_fill", 3: "wide", 4: "stream", 5: "wide16", 6: "unfused",
              8: "lines", 9: "mid", 10: "small"}[out[0]]
    return {"kernel": kernel, "rb": out[1], "splits": out[2], "n_chunk": out[3], "grid": out[4]}
