"""Register budget of every kernel in libfa355, from the compiler's own report.

The hot kernels are designed for two waves per SIMD (two 4-wave work-groups per
CU, 256 registers per lane) with nothing spilled: a spill to scratch memory
turns register traffic into memory traffic inside the key loop (the d = 128
non-causal forward once spilled 232 bytes per lane and ran at 58% of its
spill-free speed, with bitwise the same results, so no parity test notices).
This compiles the device code with the same flags as the library, asks for
the per-kernel resource remarks, and checks them.  CPU only (hipcc
cross-compiles for gfx950); about 15 s.
"""

from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from io_aware_exact_attention_amd import build as fa_build

# kernels whose schedules assume two waves per SIMD
TWO_WAVE_KERNELS = ("fa_fwd_kernel", "fa_fwd_persistent_kernel", "fa_fwd_split_kernel", "fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel",
                    "fa_bwd_fused_kernel", "fa_bwd_dq_persistent_kernel", "fa_bwd_dkdv_persistent_kernel")


def _remarks():
    try:
        cc = fa_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in fa_build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [cc, *flags, "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
               fa_build.SRC, "-o", os.path.join(tmp, "dev.o")]
        res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: +(.+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = val
            kernels[cur] = {}
        elif cur is not None:
            kernels[cur][key] = val
    return kernels


@pytest.fixture(scope="module")
def kernels():
    k = _remarks()
    assert k, "the compiler printed no resource remarks"
    return k


def test_every_kernel_reported(kernels):
    names = " ".join(kernels)
    for base in TWO_WAVE_KERNELS + ("fa_decode_split_kernel", "fa_fwd_fp8_kernel"):
        assert base in names, f"no resource remark for {base}"


def test_no_scratch_spills(kernels):
    bad = {n: (r.get("ScratchSize [bytes/lane]"), r.get("VGPRs Spill")) for n, r in kernels.items()
           if r.get("ScratchSize [bytes/lane]") != "0" or r.get("VGPRs Spill") != "0"}
    assert not bad, f"kernels that spill registers to scratch (bytes/lane, VGPRs): {bad}"


def test_hot_kernels_keep_two_waves_per_simd(kernels):
    low = {n: r.get("Occupancy [waves/SIMD]") for n, r in kernels.items()
           if any(b in n for b in TWO_WAVE_KERNELS) and int(r.get("Occupancy [waves/SIMD]", "0")) < 2}
    assert not low, f"hot kernels below two waves per SIMD: {low}"
