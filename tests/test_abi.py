"""C-ABI library: loads, exports every declared symbol, rejects bad arguments
before touching the GPU (no compute call is made here), fails loudly when
missing, and shares no code with the oracle. Runs without a GPU."""
import ctypes
import os
import re

import pytest
import torch

import moe_expert_combine_amd as mc
from moe_expert_combine_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_combine.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_combine", "moe_combine_residual_rmsnorm", "moe_combine_mxfp8",
              "moe_combine_residual_rmsnorm_mxfp8", "moe_combine_mxfp4",
              "moe_reduce_dense", "moe_reduce_dense_residual_rmsnorm",
              "moe_dispatch", "moe_dispatch_workspace_size",
              "moe_combine_describe_launch", "moe_combine_check_args", "moe_combine_abi_version",
              "moe_combine_status_string", "moe_combine_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mc.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert mc.abi_version() == 2


def test_status_strings():
    L = mc.lib()
    assert L.moe_combine_status_string(0) == b"MOE_OK"
    assert L.moe_combine_status_string(1) == b"MOE_ERR_INVALID_ARG"
    assert L.moe_combine_status_string(3) == b"MOE_ERR_HIP"
    assert L.moe_combine_status_string(99) == b"MOE_ERR_UNKNOWN"


# Fake, well-aligned device addresses: every call below is rejected (or is a
# zero-token no-op) before any HIP call, so nothing is dereferenced.
A = 1 << 20


def call_combine(payload=A, src=A, w=A, shared=None, out=2 * A, T=4, H=64, k=2,
                 ep=1, mtpr=8):
    return mc.lib().moe_combine(payload, src, w, shared, out, T, H, k, ep, mtpr, None)


@pytest.mark.parametrize("kw,msg", [
    (dict(T=-1), "num_tokens"),
    (dict(H=0), "hidden"),
    (dict(H=12), "hidden"),
    (dict(H=(1 << 28) + 8), "hidden"),
    (dict(k=0), "top_k"),
    (dict(k=33), "top_k"),
    (dict(ep=0), "ep_size"),
    (dict(mtpr=0), "max_tokens_per_rank"),
    (dict(payload=None), "payload"),
    (dict(src=None), "src_info"),
    (dict(out=None), "out"),
    (dict(payload=A + 8), "aligned"),
    (dict(src=A + 4), "aligned"),
    (dict(w=A + 2), "aligned"),
    (dict(out=A + 8), "aligned"),
    (dict(shared=A + 8), "aligned"),
    (dict(out=A), "alias"),
])
def test_moe_combine_rejects_bad_arguments(kw, msg):
    assert call_combine(**kw) == INVALID
    assert msg in mc.lib().moe_combine_last_error().decode()


def test_zero_tokens_is_a_no_op():
    assert call_combine(T=0, out=None, payload=None, src=None) == OK
    L = mc.lib()
    assert L.moe_combine_mxfp8(None, None, None, None, None, None, 0, 64, 2, 1, 8, None) == OK
    assert L.moe_combine_residual_rmsnorm(None, None, None, None, None, None, 1e-6, 0.0,
                                          None, None, 0, 64, 2, 1, 8, None) == OK


def test_rmsnorm_argument_errors():
    L = mc.lib()
    f = lambda ro, no, res=3 * A, g=4 * A, eps=1e-6: L.moe_combine_residual_rmsnorm(
        A, A, A, None, res, g, eps, 0.0, ro, no, 4, 64, 2, 1, 8, None)
    assert f(5 * A, 5 * A) == INVALID            # residual_out == norm_out
    assert f(5 * A, 3 * A) == INVALID            # norm_out == residual_in
    assert f(None, 6 * A) == INVALID
    assert f(5 * A, 6 * A, g=None) == INVALID
    assert f(5 * A, 6 * A, eps=-1.0) == INVALID
    assert f(5 * A + 2, 6 * A) == INVALID


def test_mxfp8_argument_errors():
    L = mc.lib()
    f = lambda H=64, o=5 * A, s=6 * A: L.moe_combine_mxfp8(A, A, A, None, o, s, 4, H, 2, 1, 8, None)
    assert f(H=40) == INVALID                    # not a multiple of 32
    assert "multiple of 32" in L.moe_combine_last_error().decode()
    assert f(o=None) == INVALID
    assert f(s=None) == INVALID
    assert f(o=5 * A + 4) == INVALID
    assert f(s=5 * A) == INVALID                 # scales alias codes


def test_mxfp4_argument_errors():
    L = mc.lib()
    f = lambda H=64, o=5 * A, s=6 * A: L.moe_combine_mxfp4(A, A, A, None, o, s, 4, H, 2, 1, 8, None)
    assert f(H=48) == INVALID
    assert f(o=None) == INVALID
    assert f(s=None) == INVALID
    assert f(o=5 * A + 2) == INVALID              # 4-byte alignment
    assert f(s=5 * A) == INVALID
    assert "multiple of 32" in (L.moe_combine_last_error().decode() if f(H=40) else "multiple of 32")
    assert L.moe_combine_mxfp4(None, None, None, None, None, None, 0, 64, 2, 1, 8, None) == OK
    assert "masked=0" in mc.describe_launch(4, 16384, 7168, 8)


def test_reduce_dense_argument_errors():
    L = mc.lib()
    f = lambda x=A, n=4, s=A, tok=None, o=2 * A, T=4, H=64: L.moe_reduce_dense(x, n, s, tok, o, T, H, None)
    assert f(n=0) == INVALID and "n_in" in L.moe_combine_last_error().decode()
    assert f(n=33) == INVALID
    assert f(x=None) == INVALID
    assert f(o=None) == INVALID
    assert f(o=A) == INVALID                       # out aliases inputs
    assert f(H=12) == INVALID
    assert f(x=A + 8) == INVALID
    assert f(tok=A + 8) == INVALID
    assert f(T=0, x=None, o=None) == OK
    g = lambda ro=5 * A, no=6 * A, res=3 * A: L.moe_reduce_dense_residual_rmsnorm(
        A, 4, None, None, res, 4 * A, 1e-6, 0.0, ro, no, 4, 64, None)
    assert g(no=5 * A) == INVALID
    assert g(res=None) == INVALID
    assert g(no=3 * A) == INVALID


def test_dispatch_argument_errors_and_workspace_size():
    L = mc.lib()
    n = (4096 * 8 // 256 * 256 + 4096 * 8) * 4     # chunk offsets [chunks, E] + pair ranks [T * k]
    assert mc.dispatch_workspace_size(4096, 8, 256, 8, 4224) == (n + 255) // 256 * 256
    assert mc.dispatch_workspace_size(1, 1, 8, 1, 1) == 256     # rounded to 256 B
    assert mc.dispatch_workspace_size(-1, 8, 8, 1, 1) == 0
    ws = mc.dispatch_workspace_size(4, 2, 8, 2, 8)

    def f(x=A, ids=A, T=4, H=64, k=2, E=8, ep=2, mtpr=8, pay=2 * A, src=3 * A, cnt=None, w=4 * A, wb=ws):
        return L.moe_dispatch(x, ids, T, H, k, E, ep, mtpr, pay, src, cnt, w, wb, None)
    assert f(E=9, ep=2) == INVALID    # ep must divide E
    assert f(E=5000) == INVALID
    assert f(k=0) == INVALID
    assert f(H=12) == INVALID
    assert f(mtpr=0) == INVALID
    assert f(w=None) == INVALID
    assert f(wb=ws - 4) == INVALID and "workspace too small" in L.moe_combine_last_error().decode()
    assert f(src=3 * A + 4) == INVALID
    assert f(pay=A) == INVALID        # payload aliases x
    assert f(T=0, x=None, ids=None, pay=None, src=None, w=None) == OK


def test_rmsnorm_mxfp8_argument_errors():
    L = mc.lib()

    def f(ro=5 * A, no=None, o=6 * A, sc=7 * A, H=64, res=3 * A, g=4 * A, eps=1e-6):
        return L.moe_combine_residual_rmsnorm_mxfp8(A, A, A, None, res, g, eps, 1.0, ro, no,
                                                     o, sc, 4, H, 2, 1, 8, None)
    assert f(H=40) == INVALID                 # not a multiple of 32
    assert f(ro=None) == INVALID
    assert f(o=None) == INVALID
    assert f(sc=None) == INVALID
    assert f(g=None) == INVALID
    assert f(no=6 * A) == INVALID             # norm_out aliases out_fp8
    assert f(o=3 * A) == INVALID              # out_fp8 aliases residual_in
    assert f(sc=5 * A) == INVALID             # scales alias residual_out
    assert f(o=6 * A + 4) == INVALID          # misaligned codes
    assert f(eps=-1.0) == INVALID
    assert L.moe_combine_residual_rmsnorm_mxfp8(None, None, None, None, None, None, 1e-6, 0.0,
                                                None, None, None, None, 0, 64, 2, 1, 8, None) == OK


def test_describe_launch_shapes():
    d = mc.describe_launch(0, 4096, 7168, 8)
    assert "threads=64 vec_per_thread=2 chunks=7 blocks=28672 slot_tile=8 masked=0" == d
    d = mc.describe_launch(0, 100, 4096, 8)
    assert "chunks=4" in d and "masked=0" in d
    d = mc.describe_launch(1, 2048, 7168, 8)
    assert "threads=256 vec_per_thread=4 chunks=1 blocks=2048 slot_tile=2 masked=1" in d
    assert "threads=256 vec_per_thread=4 chunks=1 blocks=2048 slot_tile=2 masked=1" in mc.describe_launch(3, 2048, 7168, 8)
    # shorter and longer rows keep the narrowest shape that covers them
    assert "threads=512 vec_per_thread=1 chunks=1 blocks=8 slot_tile=4 masked=0" in mc.describe_launch(1, 8, 4096, 8)
    assert "threads=512 vec_per_thread=4" in mc.describe_launch(1, 8, 16384, 8)
    assert "threads=384 vec_per_thread=8" in mc.describe_launch(1, 8, 24576, 8)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(3, 4, 48, 2)
    d = mc.describe_launch(2, 16384, 7168, 8)
    assert "masked=0" in d
    d = mc.describe_launch(0, 5, 264, 3)          # ragged: 33 vectors
    assert "masked=1" in d and "slot_tile=4" in d
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(2, 4, 48, 2)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(1, 4, 8 * 8 * 512 + 8, 2)
    assert "threads=512 vec_per_thread=8" in mc.describe_launch(1, 4, 8 * 8 * 512, 2)
    assert "slot_tile=2" in mc.describe_launch(1, 4, 8 * 8 * 512, 8)


def test_tile_override_env(monkeypatch):
    monkeypatch.setenv("MOE_COMBINE_TILE", "256x2")
    assert "threads=256 vec_per_thread=2 chunks=2" in mc.describe_launch(0, 10, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "64x1")
    with pytest.raises(mc.MoeCombineError):      # RMSNorm needs the whole row
        mc.describe_launch(1, 10, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "128x4")
    assert "slot_tile=4" in mc.describe_launch(0, 10, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "1024x4")  # over the V>=4 budget -> ignored
    assert "threads=64 vec_per_thread=2" in mc.describe_launch(0, 10, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "448x2x4")
    assert "threads=448 vec_per_thread=2 chunks=1 blocks=20 slot_tile=4" in mc.describe_launch(1, 20, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "448x2x8")  # explicit slot tile wins
    assert "slot_tile=8" in mc.describe_launch(1, 20, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "448x2x3")  # bad slot tile -> ignored (default shape)
    assert "threads=256 vec_per_thread=4" in mc.describe_launch(1, 20, 7168, 8)
    assert "slot_tile=2" in mc.describe_launch(1, 20, 7168, 8)
    monkeypatch.setenv("MOE_COMBINE_TILE", "100x3")   # invalid -> ignored
    assert "threads=64 vec_per_thread=2" in mc.describe_launch(0, 10, 7168, 8)


def test_binding_rejects_host_tensors_and_bad_dtypes():
    p = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    s = torch.zeros((2, 1, 2), dtype=torch.int32)
    with pytest.raises(ValueError):
        mc.moe_combine(p, s)
    with pytest.raises(ValueError):
        mc.moe_combine_mxfp8(p.float(), s)
    with pytest.raises(ValueError):
        mc.moe_reduce_dense(torch.zeros((2, 4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        mc.moe_dispatch(torch.zeros((4, 64), dtype=torch.bfloat16),
                        torch.zeros((4, 2), dtype=torch.int32), 8, 2, 8)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library (and no compiler) calls raise."""
    monkeypatch.setattr(_build, "LIB", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_build, "HIPCC", str(tmp_path / "no-hipcc"))
    monkeypatch.setattr(mc, "_lib", None)
    with pytest.raises(Exception):
        mc.lib()


def test_stale_library_is_rebuilt_or_refused(monkeypatch, tmp_path):
    """A source whose bytes differ from the ones the library was built from
    makes the loader rebuild; if the rebuild fails, loading raises instead
    of serving the old binary."""
    extra = tmp_path / "extra.h"
    extra.write_text("// one\n")
    stamp = tmp_path / "lib.srchash"
    monkeypatch.setattr(_build, "DEPS", _build.DEPS + [str(extra)])
    monkeypatch.setattr(_build, "STAMP", str(stamp))
    stamp.write_text(_build.source_hash() + "\n")
    assert not _build.stale()
    extra.write_text("// two\n")                       # a source changes
    assert _build.stale()
    calls = []

    def fake_build(verbose=False):
        calls.append(1)
        stamp.write_text(_build.source_hash() + "\n")
        return _build.LIB
    monkeypatch.setattr(_build, "build", fake_build)
    mc._load()
    assert calls == [1] and not _build.stale()
    mc._load()                                         # fresh now: no rebuild
    assert calls == [1]
    extra.write_text("// three\n")

    def failing_build(verbose=False):
        raise RuntimeError("hipcc failed")
    monkeypatch.setattr(_build, "build", failing_build)
    with pytest.raises(RuntimeError):
        mc._load()

    def no_op_build(verbose=False):
        return _build.LIB
    monkeypatch.setattr(_build, "build", no_op_build)
    with pytest.raises(RuntimeError, match="does not match its sources"):
        mc._load()


def _py_sources(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith((".py", ".hip", ".h", ".c", ".cpp")):
                yield os.path.join(dp, f)


def test_product_and_oracle_share_no_code():
    for f in _py_sources("moe_expert_combine_amd"):
        txt = open(f).read()
        assert not re.search(r"\boracle\b", txt), f
    for f in _py_sources("oracle"):
        txt = open(f).read()
        assert "moe_expert_combine_amd" not in txt and "combine_kernels" not in txt, f
        assert "import gen" not in txt, f
    for f in _py_sources("gen"):
        txt = open(f).read()
        assert "import oracle" not in txt and "moe_expert_combine_amd" not in txt, f


def test_describe_dispatch_launch(monkeypatch):
    monkeypatch.delenv("MOE_DISPATCH_PATH", raising=False)
    monkeypatch.delenv("MOE_DISPATCH_TILE", raising=False)
    d = mc.describe_launch(5, 4096, 7168, 8)
    assert d == ("path=place place_blocks=128 scatter_threads=64 scatter_vec_per_thread=2 "
                 "scatter_blocks=28672")
    assert mc.describe_launch(5, 8192, 7168, 8).startswith("path=place ")      # 65536 pairs
    assert mc.describe_launch(5, 8193, 7168, 8).startswith("path=count_scan ")
    monkeypatch.setenv("MOE_DISPATCH_PATH", "count_scan")
    assert mc.describe_launch(5, 16, 64, 2).startswith("path=count_scan ")
    monkeypatch.setenv("MOE_DISPATCH_PATH", "place")
    assert mc.describe_launch(5, 16384, 7168, 8).startswith("path=place place_blocks=512 ")
    monkeypatch.setenv("MOE_DISPATCH_TILE", "448x2")
    assert "scatter_threads=448 scatter_vec_per_thread=2 scatter_blocks=16384" in \
        mc.describe_launch(5, 16384, 7168, 8)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(8, 16, 64, 2)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(5, 16, 12, 2)
    # the local reduce launches like the combine with top_k = n_in
    assert mc.describe_launch(6, 4096, 7168, 8) == mc.describe_launch(0, 4096, 7168, 8)
    assert mc.describe_launch(7, 2048, 7168, 8) == mc.describe_launch(1, 2048, 7168, 8)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(6, 16, 64, 33)


# ------------------------------------------------ moe_combine_check_args

def test_call_args_layout_matches_the_header(tmp_path):
    """The ctypes mirror of moe_call_args_t has the C struct's size and field
    offsets (a C program built against the header prints them)."""
    import subprocess
    fields = [f[0] for f in mc.CallArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "moe_combine.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(moe_call_args_t));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(moe_call_args_t, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(mc.CallArgs)
    assert out[1:] == [getattr(mc.CallArgs, f).offset for f in fields]


B = 1 << 24    # spacing of the fake pointers below: far apart, no overlap


def good(kind):
    """Valid arguments of each kind (T=4, H=64), every buffer at its own B."""
    dims = dict(num_tokens=4, hidden=64)
    comb = dict(dims, top_k=2, ep_size=2, max_tokens_per_rank=8, payload=B, src_info=2 * B,
                router_weights=3 * B, shared_out=4 * B)
    rms = dict(residual_in=5 * B, gamma=6 * B, eps=1e-6, weight_bias=1.0,
               residual_out=7 * B, norm_out=8 * B)
    red = dict(dims, n_in=3, inputs=B, scales=3 * B, token_input=4 * B)
    return {
        "combine": dict(comb, out=9 * B),
        "combine_residual_rmsnorm": dict(comb, **rms),
        "combine_mxfp8": dict(comb, out_fp8=9 * B, out_scales=10 * B),
        "combine_residual_rmsnorm_mxfp8": dict(comb, **rms, out_fp8=9 * B, out_scales=10 * B),
        "combine_mxfp4": dict(comb, out_fp4=9 * B, out_scales=10 * B),
        "dispatch": dict(dims, top_k=2, num_experts=8, ep_size=2, max_tokens_per_rank=8, x=B,
                         topk_ids=2 * B, payload=3 * B, src_info=4 * B, recv_counts=5 * B,
                         workspace=6 * B, workspace_bytes=mc.dispatch_workspace_size(4, 2, 8, 2, 8)),
        "reduce_dense": dict(red, out=9 * B),
        "reduce_dense_residual_rmsnorm": dict(red, **rms),
    }[kind]


@pytest.mark.parametrize("kind", sorted(mc.KIND))
def test_check_args_accepts_valid_calls_of_every_kind(kind):
    st, msg = mc.check_args(kind, **good(kind))
    assert st == OK, msg
    # zero tokens needs no pointer at all
    z = {k: v for k, v in good(kind).items() if not isinstance(v, int) or v < B}
    z["num_tokens"] = 0
    assert mc.check_args(kind, **z)[0] == OK


# (kind, changes, status, message fragment): sizes, required pointers,
# alignment, and partial byte-range overlaps of outputs with inputs and with
# each other
REJECT = [
    ("combine", dict(num_tokens=-1), INVALID, "num_tokens"),
    ("combine", dict(hidden=12), INVALID, "hidden"),
    ("combine", dict(top_k=33), INVALID, "top_k"),
    ("combine", dict(ep_size=0), INVALID, "ep_size"),
    ("combine", dict(max_tokens_per_rank=0), INVALID, "max_tokens_per_rank"),
    ("combine", dict(out=None), INVALID, "out is NULL"),
    ("combine", dict(out=9 * B + 8), INVALID, "aligned"),
    ("combine", dict(out=B + 2 * 8 * 64 * 2 - 16), INVALID, "out aliases payload"),   # last 16 B of payload
    ("combine", dict(out=2 * B + 48), INVALID, "out aliases src_info"),             # inside [T, k, 2]
    ("combine", dict(out=3 * B - 496), INVALID, "out aliases router_weights"),      # ends inside it
    ("combine", dict(out=3 * B - 512), OK, ""),                                     # ends right before it
    ("combine", dict(out=4 * B + 256), INVALID, "out aliases shared_out"),
    ("combine", dict(out=B + 2 * 8 * 64 * 2), OK, ""),                              # just past payload
    ("combine_residual_rmsnorm", dict(hidden=32776), UNSUPPORTED, "too large"),
    ("combine_residual_rmsnorm", dict(eps=-1.0), INVALID, "eps"),
    ("combine_residual_rmsnorm", dict(gamma=None), INVALID, "required"),
    ("combine_residual_rmsnorm", dict(residual_out=5 * B), OK, ""),                 # in place
    ("combine_residual_rmsnorm", dict(residual_out=5 * B + 16), INVALID, "residual_out aliases residual_in"),
    ("combine_residual_rmsnorm", dict(norm_out=7 * B + 128), INVALID, "norm_out aliases residual_out"),
    ("combine_residual_rmsnorm", dict(norm_out=6 * B + 64), INVALID, "norm_out aliases gamma"),
    ("combine_mxfp8", dict(hidden=48), INVALID, "multiple of 32"),
    ("combine_mxfp8", dict(out_fp8=9 * B + 4), INVALID, "aligned"),
    ("combine_mxfp8", dict(out_scales=9 * B + 255), INVALID, "out_scales aliases out_fp8"),
    ("combine_mxfp8", dict(out_scales=9 * B + 256), OK, ""),                         # just past the codes
    ("combine_mxfp8", dict(out_scales=None), INVALID, "required"),
    ("combine_residual_rmsnorm_mxfp8", dict(out_fp8=7 * B + 8), INVALID, "out_fp8 aliases residual_out"),
    ("combine_residual_rmsnorm_mxfp8", dict(out_scales=8 * B + 500), INVALID, "out_scales aliases norm_out"),
    ("combine_residual_rmsnorm_mxfp8", dict(norm_out=None), OK, ""),
    ("combine_residual_rmsnorm_mxfp8", dict(out_fp8=None), INVALID, "required"),
    ("combine_mxfp4", dict(out_fp4=9 * B + 2), INVALID, "aligned"),
    ("combine_mxfp4", dict(out_scales=9 * B + 127), INVALID, "out_scales aliases out_fp4"),
    ("combine_mxfp4", dict(out_scales=9 * B + 128), OK, ""),
    ("dispatch", dict(num_experts=9), INVALID, "ep_size must divide"),
    ("dispatch", dict(workspace_bytes=4), INVALID, "workspace too small"),
    ("dispatch", dict(payload=B + 256), INVALID, "payload aliases x"),
    ("dispatch", dict(recv_counts=4 * B + 8), INVALID, "recv_counts aliases src_info"),
    ("dispatch", dict(workspace=3 * B + 2 * 8 * 64 * 2 - 4), INVALID, "workspace aliases payload"),
    ("dispatch", dict(src_info=2 * B + 4), INVALID, "aligned"),
    ("reduce_dense", dict(n_in=0), INVALID, "n_in"),
    ("reduce_dense", dict(inputs=None), INVALID, "inputs is NULL"),
    ("reduce_dense", dict(out=B + 3 * 4 * 64 * 2 - 2), INVALID, "aligned"),
    ("reduce_dense", dict(out=B + 3 * 4 * 64 * 2 - 16), INVALID, "out aliases inputs"),
    ("reduce_dense", dict(out=3 * B), INVALID, "out aliases scales"),
    ("reduce_dense_residual_rmsnorm", dict(residual_out=4 * B + 32), INVALID, "residual_out aliases token_input"),
    ("reduce_dense_residual_rmsnorm", dict(norm_out=5 * B), INVALID, "norm_out aliases residual_in"),
]


@pytest.mark.parametrize("kind,change,status,frag", REJECT)
def test_check_args_rejections(kind, change, status, frag):
    st, msg = mc.check_args(kind, **dict(good(kind), **change))
    assert st == status, msg
    assert frag in msg


def _entry_call(kind, a):
    """The entry point of a kind, called with the same arguments."""
    L, g = mc.lib(), a.get
    T, H = g("num_tokens", 0), g("hidden", 0)
    comb = (g("payload"), g("src_info"), g("router_weights"), g("shared_out"))
    dims = (T, H, g("top_k", 0), g("ep_size", 0), g("max_tokens_per_rank", 0), None)
    rms = (g("residual_in"), g("gamma"), g("eps", 0.0), g("weight_bias", 0.0))
    if kind == "combine":
        return L.moe_combine(*comb, g("out"), *dims)
    if kind == "combine_residual_rmsnorm":
        return L.moe_combine_residual_rmsnorm(*comb, *rms, g("residual_out"), g("norm_out"), *dims)
    if kind == "combine_mxfp8":
        return L.moe_combine_mxfp8(*comb, g("out_fp8"), g("out_scales"), *dims)
    if kind == "combine_residual_rmsnorm_mxfp8":
        return L.moe_combine_residual_rmsnorm_mxfp8(*comb, *rms, g("residual_out"), g("norm_out"),
                                                    g("out_fp8"), g("out_scales"), *dims)
    if kind == "combine_mxfp4":
        return L.moe_combine_mxfp4(*comb, g("out_fp4"), g("out_scales"), *dims)
    if kind == "dispatch":
        return L.moe_dispatch(g("x"), g("topk_ids"), T, H, g("top_k", 0), g("num_experts", 0),
                              g("ep_size", 0), g("max_tokens_per_rank", 0), g("payload"),
                              g("src_info"), g("recv_counts"), g("workspace"),
                              g("workspace_bytes", 0), None)
    red = (g("inputs"), g("n_in", 0), g("scales"), g("token_input"))
    if kind == "reduce_dense":
        return L.moe_reduce_dense(*red, g("out"), T, H, None)
    return L.moe_reduce_dense_residual_rmsnorm(*red, *rms, g("residual_out"), g("norm_out"), T, H, None)


@pytest.mark.parametrize("kind", sorted(mc.KIND))
def test_entry_points_reject_what_check_args_rejects(kind):
    """Random perturbations of a valid call (pointers moved into other
    buffers or misaligned, sizes out of range, pointers dropped): whenever
    moe_combine_check_args rejects a call, the entry point rejects it with
    the same status and message, before any HIP call."""
    import random
    import zlib
    rnd = random.Random(zlib.crc32(kind.encode()))
    base = good(kind)
    ptrs = [k for k, v in base.items() if isinstance(v, int) and v >= B]
    sizes = [k for k in ("num_tokens", "hidden", "top_k", "ep_size", "max_tokens_per_rank",
                         "n_in", "num_experts") if k in base]
    rejected = 0
    for _ in range(300):
        a = dict(base)
        for _ in range(rnd.randint(1, 3)):
            r = rnd.random()
            if r < 0.5:
                p = rnd.choice(ptrs)
                a[p] = rnd.choice([v for k, v in base.items() if k in ptrs]) + rnd.choice([0, 2, 4, 8, 16, 64, 256, 1024])
            elif r < 0.8:
                sz = rnd.choice(sizes)
                a[sz] = rnd.choice([-1, 0, 1, 3, 8, 12, 33, 40, 64, 4096, 1 << 31])
            else:
                a[rnd.choice(ptrs)] = None
        try:
            st, msg = mc.check_args(kind, **a)
        except (OverflowError, TypeError):
            continue
        if st == OK:
            continue
        rejected += 1
        assert _entry_call(kind, a) == st, (a, msg)
        assert mc.lib().moe_combine_last_error().decode() == msg
    assert rejected > 100
