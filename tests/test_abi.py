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
              "moe_combine_describe_launch", "moe_combine_abi_version",
              "moe_combine_status_string", "moe_combine_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mc.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert mc.abi_version() == 1


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
    assert "threads=448 vec_per_thread=2 chunks=1 blocks=2048 slot_tile=4" in d
    assert "threads=448 vec_per_thread=2 chunks=1 blocks=2048 slot_tile=2" in mc.describe_launch(3, 2048, 7168, 8)
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
    monkeypatch.setenv("MOE_COMBINE_TILE", "448x2x3")  # bad slot tile -> ignored
    assert "threads=448 vec_per_thread=2" in mc.describe_launch(1, 20, 7168, 8)
    assert "slot_tile=4" in mc.describe_launch(1, 20, 7168, 8)
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
        mc.describe_launch(6, 16, 64, 2)
    with pytest.raises(mc.MoeCombineError):
        mc.describe_launch(5, 16, 12, 2)
