"""Host sanitizers (CPU only): the oracle's pins against an AddressSanitizer
+ UndefinedBehaviorSanitizer build of oracle.c, and a fuzz of the argument
validator (check_args.cpp, pure host code) built the same way. Any report
aborts the child process, which fails the test.

The same runs by hand, from the repository root:
  LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
    MOE_ORACLE_SANITIZE=1 python -m pytest tests/test_oracle_pins.py -q
  g++ -std=c++17 -O1 -fsanitize=address,undefined -fno-sanitize-recover=all -fPIC \\
    -shared -Iinclude moe_expert_combine_amd/csrc/check_args.cpp -o /tmp/libcheck_san.so
  LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
    python tests/_sanitize_check_args.py /tmp/libcheck_san.so
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def _env():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("libasan is not installed")
    env = dict(os.environ, LD_PRELOAD=asan, MOE_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    return env


def _clean(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan():
    env = _env()
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"],
                   cwd=ROOT, env=dict(env, LD_PRELOAD=""), check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q",
                        "-p", "no:cacheprovider", "-x"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = _clean(r)
    assert " passed" in out and " failed" not in out


def test_argument_validator_under_asan_and_ubsan(tmp_path):
    env = _env()
    lib = tmp_path / "libcheck_san.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-Wall", "-Wextra"] + SAN_FLAGS
                   + ["-I", os.path.join(ROOT, "include"),
                      os.path.join(ROOT, "moe_expert_combine_amd", "csrc", "check_args.cpp"),
                      "-o", str(lib)], check=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_sanitize_check_args.py"),
                        str(lib)], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert "random calls clean" in _clean(r)
