"""The C ABI used from C++ alone: fa355_c_example (built next to the library from
csrc/c_example.cpp) runs the forward, the persistent forward, the backward and a
decoding call through the header's functions and checks identities that need no
reference implementation, plus the documented error codes (GPU)."""

import os
import subprocess

import pytest

from io_aware_exact_attention_amd import build

pytestmark = pytest.mark.gpu


def test_c_example():
    import torch
    if torch.cuda.device_count() == 0:   # counting devices does not initialise the GPU
        pytest.skip("no GPU visible")
    assert os.path.exists(build.EXAMPLE_OUT), "fa355_c_example is not built (run build())"
    res = subprocess.run([build.EXAMPLE_OUT], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c_example ok" in res.stdout
