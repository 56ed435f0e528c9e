"""Build of the HIP library (gfx950) with hipcc; no torch extension machinery.

The library is a plain shared object exporting the C ABI of
``include/moe_combine.h``; it is built in-tree next to this file. After a
successful build, ``libmoe_combine.so.srchash`` records the sha256 of the
exact source bytes and compiler flags it was built from; ``stale()``
compares that record with the sources as they are now, so an edited source
is never silently served by an older binary (file times are not trusted:
copies of the tree need not keep them).
"""
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_combine.so")
STAMP = LIB + ".srchash"
SOURCES = [os.path.join(CSRC, "moe_combine.hip"), os.path.join(CSRC, "check_args.cpp")]
DEPS = SOURCES + [os.path.join(CSRC, "combine_kernels.h"),
                  os.path.join(CSRC, "dispatch_kernels.h"),
                  os.path.join(CSRC, "host_check.h"),
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


def source_hash():
    """sha256 over the compiler flags and the bytes of every source file the
    library is built from."""
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for d in DEPS:
        h.update(os.path.basename(d).encode() + b"\0")
        with open(d, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build(verbose=False):
    """Compile the library (always; callers decide when to rebuild) and
    record the hash of the sources it was compiled from."""
    want = source_hash()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for the MoE combine library")
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w") as f:
        f.write(want + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


def stale():
    """True if the library is missing or was not built from the sources as
    they are now (by content, not by file time)."""
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return True
    with open(STAMP) as f:
        return f.read().strip() != source_hash()


if __name__ == "__main__":
    print(build(verbose=True))
