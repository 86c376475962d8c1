"""Build step: compile the HIP sources into libattn_jvp.so for gfx950.

    python -m attention_jvp_amd.build

Each translation unit (the launching entry points, one unit of kernel
instances per head dim, the merge and backward kernels) compiles in its own
hipcc process, in parallel; the host-only unit (validation and planning,
plain C++) with the host compiler.  The objects are then linked into one
shared library, together with a generated unit that exports the digest of
the sources and flags it was built from (``attn_jvp_build_id``), so that the
loader can refuse a library older than the sources beside it.
"""

import concurrent.futures
import hashlib
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
UNITS = ["attn_jvp.hip", "inst_bf16_qk16.hip", "inst_bf16_qk32.hip", "inst_bf16_qk64.hip",
         "inst_bf16_qk128.hip", "inst_bf16_qk256.hip", "inst_fp32.hip", "merge.hip",
         "inst_bwd.hip"]
HOST_UNITS = ["host.cpp"]
SOURCES = [os.path.join(CSRC, u) for u in UNITS]
HOST_SOURCES = [os.path.join(CSRC, u) for u in HOST_UNITS]
OUTPUT = os.path.join(HERE, "libattn_jvp.so")

# Packed fp32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ArchVGPRs: the online rescale multiplies them
    # with VALU ops, and AGPR accumulators would be copied every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + INCLUDE,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def host_cxx():
    return os.environ.get("CXX", "g++")


def source_files():
    """Every file the library is built from: the sources under csrc/ and the
    public header, in a fixed order."""
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h", ".cpp")))
    return [os.path.join(CSRC, n) for n in names] + [os.path.join(INCLUDE, "attn_jvp.h")]


def source_digest():
    """sha256 over the names and contents of source_files() and the compiler
    flags."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    flags = [f for f in HIPCC_FLAGS + HOST_FLAGS if not f.startswith("-I")]
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("compile failed: " + " ".join(cmd[-3:]))


def build(verbose=False, jobs=None):
    jobs = jobs or min(len(SOURCES) + 2, max(1, len(os.sched_getaffinity(0))))
    digest = source_digest()
    with tempfile.TemporaryDirectory(prefix="attn_jvp_build_") as tmp:
        stamp = os.path.join(tmp, "build_id.cpp")
        with open(stamp, "w") as f:
            f.write('extern "C" const char *attn_jvp_build_id(void) { return "%s"; }\n' % digest)
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        host_objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in HOST_SOURCES + [stamp]]
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            futs = [pool.submit(_run, [hipcc()] + HIPCC_FLAGS + ["-c", s, "-o", o], verbose)
                    for s, o in zip(SOURCES, objs)]
            futs += [pool.submit(_run, [host_cxx()] + HOST_FLAGS + ["-c", s, "-o", o], verbose)
                     for s, o in zip(HOST_SOURCES + [stamp], host_objs)]
            for fut in futs:
                fut.result()
        out_tmp = OUTPUT + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + host_objs +
             ["-o", out_tmp], verbose)
        os.replace(out_tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
