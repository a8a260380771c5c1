"""Register budget of the HIP kernels (CPU: device-only compiles with the
build's flags, no GPU).  The prefill tile keeps ~250 VGPRs live; a change
that pushes a kernel over the 256-VGPR budget makes the compiler spill
accumulators to scratch memory, which runs correctly but several times
slower -- so spills are checked here, where they are cheap to see."""
import os
import re
import shutil
import subprocess

import pytest

from fp8_block_scaled_token_amd import build as B

# kernels allowed a small scratch area (bytes per lane), by name pattern
ALLOWED = {}


def _usage(src):
    cmd = [B.hipcc()] + B.compile_flags() + B.EXTRA_FLAGS.get(src, []) + [
        "--cuda-device-only", "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
        "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm_fast.hip", "gemm_decode.hip", "gemm_kernels.hip", "quant_kernels.hip"])
def test_no_scratch_spills(src):
    usage = _usage(src)
    assert usage, "no kernels found in the compiler's resource report"
    for name, scratch in usage.items():
        limit = next((v for k, v in ALLOWED.items() if re.search(k, name)), 0)
        assert scratch <= limit, f"{name}: {scratch} bytes of scratch per lane"
