"""CPU: the opt-in kernel variant still compiles for gfx950.

The 32-query-row forward kernel (kernel32.h) is built only with
-DATTN_JVP_ROWS32_D128=1; the default library never compiles it, so this
test keeps it from falling behind the shared headers it uses.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

from attention_jvp_amd import build

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_rows32_variant_compiles():
    src = os.path.join(build.CSRC, "inst_bf16_qk128.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "r32.o")
        flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
        cmd = [HIPCC] + flags + ["-DATTN_JVP_ROWS32_D128=1", "--cuda-device-only", "-c", src,
                                 "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        assert os.path.getsize(out) > 0
