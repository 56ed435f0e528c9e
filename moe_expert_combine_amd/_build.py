"""Build of the HIP library (gfx950) with hipcc; no torch extension machinery.

The library is a plain shared object exporting the C ABI of
``include/moe_combine.h``; it is built in-tree next to this file.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_combine.so")
SOURCES = [os.path.join(CSRC, "moe_combine.hip")]
DEPS = SOURCES + [os.path.join(CSRC, "combine_kernels.h"),
                  os.path.join(CSRC, "dispatch_kernels.h"),
                  os.path.join(ROOT, "include", "moe_combine.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # packed fp32 instructions stay off (hipcc would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def hipcc_command(out=LIB, extra=()):
    return [HIPCC] + FLAGS + list(extra) + SOURCES + ["-o", out]


def build(verbose=False):
    """Compile the library (always; callers decide when to rebuild)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for the MoE combine library")
    os.replace(tmp, LIB)
    return LIB


def stale():
    """True if the library is missing or older than a source it depends on."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
