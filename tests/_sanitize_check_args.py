"""Run under the host sanitizers by tests/test_sanitizers.py (not collected by
pytest): calls moe_combine_check_args of a host-only, sanitizer-instrumented
build of check_args.cpp on the valid calls, the rejection table and a
random fuzz of every kind, including extreme sizes. Any sanitizer report
aborts the process."""
import ctypes
import os
import random
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moe_expert_combine_amd as mc          # noqa: E402  (the library itself is not loaded)
from tests.test_abi import B, REJECT, good   # noqa: E402

L = ctypes.CDLL(sys.argv[1])
L.moe_combine_check_args.argtypes = [ctypes.POINTER(mc.CallArgs)]
L.moe_combine_check_args.restype = ctypes.c_int
L.moe_combine_last_error.restype = ctypes.c_char_p


def check(kind, fields):
    a = mc.CallArgs(kind=mc.KIND[kind], **fields)
    st = L.moe_combine_check_args(ctypes.byref(a))
    return st, L.moe_combine_last_error().decode()


n = 0
for kind in mc.KIND:
    assert check(kind, good(kind))[0] == 0, kind
for kind, change, status, frag in REJECT:
    st, msg = check(kind, dict(good(kind), **change))
    assert st == status and frag in msg, (kind, change, st, msg)
rnd = random.Random(5)
extreme = [-(1 << 31), -1, 0, 1, 7, 8, 31, 32, 33, 4096, 4097, (1 << 28), (1 << 28) + 8,
           (1 << 31) - 1]
for kind in mc.KIND:
    base = good(kind)
    ptrs = [k for k, v in base.items() if isinstance(v, int) and v >= B]
    sizes = [k for k in ("hidden", "top_k", "ep_size", "n_in", "num_experts") if k in base]
    wide = [k for k in ("num_tokens", "max_tokens_per_rank") if k in base]
    for _ in range(3000):
        a = dict(base)
        for _ in range(rnd.randint(1, 4)):
            r = rnd.random()
            if r < 0.4:
                a[rnd.choice(ptrs)] = rnd.choice([None, 8, 1 << 63, (1 << 64) - 16,
                                                  rnd.randrange(0, 1 << 48)])
            elif r < 0.7:
                a[rnd.choice(sizes)] = rnd.choice(extreme)
            else:
                a[rnd.choice(wide)] = rnd.choice(extreme + [(1 << 62), -(1 << 62)])
        check(kind, a)
        n += 1
print("check_args sanitizer run: %d random calls clean" % n, flush=True)
