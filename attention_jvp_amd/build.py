"""Build step: compile the HIP sources into libattn_jvp.so for gfx950.

    python -m attention_jvp_amd.build

Each translation unit (the host API and one unit of kernel instances per
head dim) compiles in its own hipcc process, in parallel; the objects are
then linked into one shared library.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
UNITS = ["attn_jvp.hip", "inst_bf16_qk16.hip", "inst_bf16_qk32.hip", "inst_bf16_qk64.hip",
         "inst_bf16_qk128.hip", "inst_bf16_qk256.hip", "inst_fp32.hip", "merge.hip",
         "inst_bwd.hip"]
SOURCES = [os.path.join(CSRC, u) for u in UNITS]
HEADERS = [os.path.join(CSRC, h) for h in ("kernel.h", "dispatch.h", "inst.h", "bwd.h")] + [
    os.path.join(ROOT, "include", "attn_jvp.h")]
OUTPUT = os.path.join(HERE, "libattn_jvp.so")

# Packed fp32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ArchVGPRs: the online rescale multiplies them
    # with VALU ops, and AGPR accumulators would be copied every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose=False, jobs=None):
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="attn_jvp_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            futs = [pool.submit(_run, [hipcc()] + HIPCC_FLAGS + ["-c", s, "-o", o], verbose)
                    for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        out_tmp = OUTPUT + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out_tmp],
             verbose)
        os.replace(out_tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
