"""The allocation-free dispatch (moe_dispatch_noalloc, library-held device
scratch) against moe_dispatch with a caller workspace, through the C ABI:
slot map, every payload row (placed and untouched) and the accumulated
receive counts must be bit-identical, on two calls in a row, the second
smaller than the first, on both placement paths (only the count + scan path
keeps data in the scratch)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_combine_amd as mc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(T, H, k, E, drop, seed):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[rng.random((T, k)) < drop] = -1
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    return x.to(DEV), torch.from_numpy(ids).to(DEV)


def _outputs(T, H, k, E, ep, mtpr):
    pay = torch.full((ep, mtpr, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    src = torch.full((T, k, 2), -7, dtype=torch.int32, device=DEV)
    cnt = torch.arange(E, dtype=torch.int32, device=DEV)          # counts accumulate onto this
    return pay, src, cnt


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("path", ["count_scan", "place"])
def test_noalloc_dispatch_matches_workspace_dispatch(monkeypatch, path):
    monkeypatch.setenv("MOE_DISPATCH_PATH", path)
    L = mc.lib()
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: None if t is None else t.data_ptr()
    # the second call is smaller, so stale scratch contents from the first
    # would show if the kernels read anything they did not write
    for (T, H, k, E, ep, mtpr, drop, seed) in [(3000, 1024, 8, 256, 8, 3100, 0.05, 1),
                                               (700, 512, 6, 64, 4, 900, 0.2, 2)]:
        x, ids = _inputs(T, H, k, E, drop, seed)
        ref_pay, ref_src, ref_cnt = _outputs(T, H, k, E, ep, mtpr)
        mc.moe_dispatch(x, ids, E, ep, mtpr, payload=ref_pay, src_info=ref_src, recv_counts=ref_cnt)
        pay, src, cnt = _outputs(T, H, k, E, ep, mtpr)
        st = L.moe_dispatch_noalloc(P(x), P(ids), T, H, k, E, ep, mtpr, P(pay), P(src), P(cnt), stream)
        assert st == 0, L.moe_combine_last_error().decode()
        torch.cuda.synchronize()
        what = f"{path} T={T}"
        np.testing.assert_array_equal(_bits(src), _bits(ref_src), err_msg=what + " src_info")
        np.testing.assert_array_equal(_bits(pay), _bits(ref_pay), err_msg=what + " payload")
        np.testing.assert_array_equal(_bits(cnt), _bits(ref_cnt), err_msg=what + " recv_counts")
        assert (_bits(src)[..., 0] >= 0).sum() > 0.5 * T * k


def test_noalloc_dispatch_rejects_calls_beyond_its_scratch(monkeypatch):
    """A count + scan dispatch needing more than the 8 MiB scratch is
    rejected before any launch (4096 experts, 2^19 pairs: 34 MiB)."""
    monkeypatch.setenv("MOE_DISPATCH_PATH", "count_scan")
    L = mc.lib()
    A = 1 << 30
    T, k, E = 65536, 8, 4096
    assert mc.dispatch_workspace_size(T, k, E, 8, 70000) > (8 << 20)
    st = L.moe_dispatch_noalloc(A, 2 * A, T, 1024, k, E, 8, 70000, 4 * A, 3 * A, None, None)
    assert st == 2 and "scratch" in L.moe_combine_last_error().decode()
