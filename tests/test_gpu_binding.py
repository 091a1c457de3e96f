"""The Python binding loaded before PyTorch: it must bind to the HIP runtime PyTorch ships (one runtime per
process), or every launch on torch's memory fails."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import dequant_backward_gemm_amd as nb   # before torch
import numpy as np
import torch
import oracle, synth
N, K = 96, 192
w = synth.weights_normal(N, K, 7)
s, b = oracle.pack(w, N, K)
out = nb.dequant(torch.from_numpy(s).cuda(), torch.from_numpy(b).cuda())
torch.cuda.synchronize()
assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.dequant(s, b, N, K).view(np.uint32))
print("binding-first ok")
"""


def test_binding_imported_before_torch():
    r = subprocess.run([sys.executable, "-c", _SCRIPT, ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "binding-first ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
