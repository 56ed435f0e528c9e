"""MI355X-native MoE expert combine: thin Python binding of the C ABI.

Every function here only checks and marshals arguments (dtype, shape, device,
contiguity) and calls the entry point of the same name in
``libmoe_combine.so`` (hand-written HIP kernels for gfx950, declared in
``include/moe_combine.h``) on torch's current HIP stream. All arithmetic runs
in those kernels. There is no fallback: if the library cannot be loaded,
every call raises.

Layouts (see the header for the full contract):
  payload        bf16  [ep_size, max_tokens_per_rank, hidden]
  src_info       int32 [num_tokens, top_k, 2]   (rank, row); rank < 0, or a slot outside
                                                the payload, is dropped
  router_weights fp32  [num_tokens, top_k]      or None (unit weights)
  shared_out     bf16  [num_tokens, hidden]     or None
Outputs may be passed in with at least num_tokens rows; only the first
num_tokens rows are written.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

__all__ = ["moe_combine", "moe_combine_residual_rmsnorm", "moe_combine_mxfp8",
           "moe_combine_residual_rmsnorm_mxfp8", "moe_combine_mxfp4",
           "moe_reduce_dense", "moe_reduce_dense_residual_rmsnorm",
           "moe_dispatch", "moe_dispatch_noalloc", "dispatch_workspace_size",
           "describe_launch", "check_args", "CallArgs", "KIND", "abi_version", "lib",
           "library_path", "MoeCombineError"]

# Entry-point kinds (MOE_KIND_* in include/moe_combine.h).
KIND = {"combine": 0, "combine_residual_rmsnorm": 1, "combine_mxfp8": 2,
        "combine_residual_rmsnorm_mxfp8": 3, "combine_mxfp4": 4, "dispatch": 5,
        "reduce_dense": 6, "reduce_dense_residual_rmsnorm": 7}


class CallArgs(ctypes.Structure):
    """moe_call_args_t: the arguments of one entry-point call, by name
    (pointers as integers, sizes as ints)."""
    _fields_ = [("kind", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_tokens", ctypes.c_int64), ("top_k", ctypes.c_int32),
                ("ep_size", ctypes.c_int32), ("max_tokens_per_rank", ctypes.c_int64),
                ("n_in", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("eps", ctypes.c_float), ("weight_bias", ctypes.c_float)] + [
        (n, ctypes.c_void_p) for n in (
            "payload", "src_info", "router_weights", "shared_out", "inputs", "scales",
            "token_input", "residual_in", "gamma", "x", "topk_ids", "out", "residual_out",
            "norm_out", "out_fp8", "out_fp4", "out_scales", "recv_counts", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t)]

library_path = _build.LIB


class MoeCombineError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn, status, msg):
        self.status = status
        super().__init__(f"{fn}: {_status_name(status)}: {msg}")


_lib = None


def _load():
    """Load the library. If it is missing, or was built from other sources
    than the ones in the tree, rebuild it first; if that fails, raise:
    a stale binary is never loaded."""
    if _build.stale():
        _build.build()
        if _build.stale():
            raise RuntimeError(f"{_build.LIB} does not match its sources after a rebuild")
    L = ctypes.CDLL(_build.LIB)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    dims = [I64, I32, I32, I32, I64, P]
    L.moe_combine.argtypes = [P, P, P, P, P] + dims
    L.moe_combine_residual_rmsnorm.argtypes = [P, P, P, P, P, P, F, F, P, P] + dims
    L.moe_combine_mxfp8.argtypes = [P, P, P, P, P, P] + dims
    L.moe_combine_residual_rmsnorm_mxfp8.argtypes = [P, P, P, P, P, P, F, F, P, P, P, P] + dims
    L.moe_combine_mxfp4.argtypes = [P, P, P, P, P, P] + dims
    L.moe_reduce_dense.argtypes = [P, I32, P, P, P, I64, I32, P]
    L.moe_reduce_dense.restype = ctypes.c_int
    L.moe_reduce_dense_residual_rmsnorm.argtypes = [P, I32, P, P, P, P, F, F, P, P, I64, I32, P]
    L.moe_reduce_dense_residual_rmsnorm.restype = ctypes.c_int
    L.moe_dispatch_workspace_size.argtypes = [I64, I32, I32, I32, I64]
    L.moe_dispatch_workspace_size.restype = ctypes.c_size_t
    L.moe_dispatch.argtypes = [P, P, I64, I32, I32, I32, I32, I64, P, P, P, P, ctypes.c_size_t, P]
    L.moe_dispatch.restype = ctypes.c_int
    L.moe_dispatch_noalloc.argtypes = [P, P, I64, I32, I32, I32, I32, I64, P, P, P, P]
    L.moe_dispatch_noalloc.restype = ctypes.c_int
    for f in ("moe_combine", "moe_combine_residual_rmsnorm", "moe_combine_mxfp8",
              "moe_combine_residual_rmsnorm_mxfp8", "moe_combine_mxfp4"):
        getattr(L, f).restype = ctypes.c_int
    L.moe_combine_check_args.argtypes = [ctypes.POINTER(CallArgs)]
    L.moe_combine_check_args.restype = ctypes.c_int
    L.moe_combine_describe_launch.argtypes = [ctypes.c_int, I64, I32, I32, ctypes.c_char_p, I32]
    L.moe_combine_describe_launch.restype = ctypes.c_int
    L.moe_combine_abi_version.argtypes = []
    L.moe_combine_abi_version.restype = ctypes.c_int
    L.moe_combine_status_string.argtypes = [ctypes.c_int]
    L.moe_combine_status_string.restype = ctypes.c_char_p
    L.moe_combine_last_error.argtypes = []
    L.moe_combine_last_error.restype = ctypes.c_char_p
    return L


def lib():
    """The loaded ctypes library (loaded on first use)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _status_name(st):
    return lib().moe_combine_status_string(st).decode()


def _check(fn, st):
    if st != 0:
        raise MoeCombineError(fn, st, lib().moe_combine_last_error().decode())


def abi_version() -> int:
    return lib().moe_combine_abi_version()


def check_args(kind, **fields):
    """moe_combine_check_args: validate one call's arguments on the host
    (sizes, required pointers, alignment, byte-range overlap) without
    touching the GPU. ``kind`` is a name of KIND or its number; fields are
    the entry point's parameter names (pointers as ints). Returns the status
    and the library's message."""
    a = CallArgs(kind=KIND.get(kind, kind) if isinstance(kind, str) else kind, **fields)
    st = lib().moe_combine_check_args(ctypes.byref(a))
    return st, lib().moe_combine_last_error().decode()


def describe_launch(kind: int, num_tokens: int, hidden: int, top_k: int) -> str:
    """Launch shape an entry point would use (kind as in KIND: 0 bf16,
    1 RMSNorm, 2 MXFP8, 3 RMSNorm + MXFP8, 4 MXFP4, 5 dispatch, 6 and 7 the
    local reduce, with top_k = n_in)."""
    buf = ctypes.create_string_buffer(256)
    _check("moe_combine_describe_launch",
           lib().moe_combine_describe_launch(kind, num_tokens, hidden, top_k, buf, 256))
    return buf.value.decode()


# ----------------------------------------------------------------- checks

def _need(t, name, dtype, device, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")


def _common(payload, src_info, router_weights, shared_out):
    if not isinstance(payload, torch.Tensor) or payload.device.type != "cuda":
        raise ValueError("payload must be a GPU tensor")
    dev = payload.device
    _need(payload, "payload", torch.bfloat16, dev, 3)
    _need(src_info, "src_info", torch.int32, dev, 3)
    if src_info.shape[2] != 2:
        raise ValueError("src_info must be [num_tokens, top_k, 2]")
    ep, mtpr, H = payload.shape
    T, k, _ = src_info.shape
    if router_weights is not None:
        _need(router_weights, "router_weights", torch.float32, dev, 2)
        if tuple(router_weights.shape) != (T, k):
            raise ValueError(f"router_weights must be [{T}, {k}]")
    if shared_out is not None:
        _need(shared_out, "shared_out", torch.bfloat16, dev, 2)
        if tuple(shared_out.shape) != (T, H):
            raise ValueError(f"shared_out must be [{T}, {H}]")
    return dev, (T, H, k, ep, mtpr)


def _out(t, name, dtype, dev, T, cols, make):
    if t is None:
        return make()
    _need(t, name, dtype, dev, 2)
    if t.shape[0] < T or t.shape[1] != cols:
        raise ValueError(f"{name} must be [>= {T}, {cols}] (got {tuple(t.shape)})")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


# ------------------------------------------------------------ entry points

def moe_combine(payload, src_info, router_weights=None, shared_out=None, out=None):
    """bf16 combine; returns ``out`` ([num_tokens, hidden] bf16 if None)."""
    dev, (T, H, k, ep, mtpr) = _common(payload, src_info, router_weights, shared_out)
    out = _out(out, "out", torch.bfloat16, dev, T, H,
               lambda: torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    _check("moe_combine", lib().moe_combine(
        _ptr(payload), _ptr(src_info), _ptr(router_weights), _ptr(shared_out), _ptr(out),
        T, H, k, ep, mtpr, _stream(dev)))
    return out


def moe_combine_residual_rmsnorm(payload, src_info, router_weights, shared_out,
                                 residual_in, gamma, eps, weight_bias=0.0,
                                 residual_out=None, norm_out=None):
    """Combine + residual add + RMSNorm; returns (residual_out, norm_out).
    ``weight_bias`` None means 0.0; ``residual_out`` may be ``residual_in``."""
    dev, (T, H, k, ep, mtpr) = _common(payload, src_info, router_weights, shared_out)
    _need(residual_in, "residual_in", torch.bfloat16, dev, 2)
    if residual_in.shape[0] < T or residual_in.shape[1] != H:
        raise ValueError(f"residual_in must be [>= {T}, {H}]")
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    if gamma.shape[0] != H:
        raise ValueError(f"gamma must be [{H}]")
    mk = lambda: torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    residual_out = _out(residual_out, "residual_out", torch.bfloat16, dev, T, H, mk)
    norm_out = _out(norm_out, "norm_out", torch.bfloat16, dev, T, H, mk)
    wb = 0.0 if weight_bias is None else float(weight_bias)
    _check("moe_combine_residual_rmsnorm", lib().moe_combine_residual_rmsnorm(
        _ptr(payload), _ptr(src_info), _ptr(router_weights), _ptr(shared_out),
        _ptr(residual_in), _ptr(gamma), float(eps), wb, _ptr(residual_out),
        _ptr(norm_out), T, H, k, ep, mtpr, _stream(dev)))
    return residual_out, norm_out


def moe_combine_mxfp8(payload, src_info, router_weights=None, shared_out=None,
                      out_fp8=None, out_scales=None):
    """MXFP8 combine; returns (out_fp8 float8_e4m3fn [T, H], out_scales uint8
    [T, H/32] UE8M0, linear layout)."""
    dev, (T, H, k, ep, mtpr) = _common(payload, src_info, router_weights, shared_out)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP8")
    out_fp8 = _out(out_fp8, "out_fp8", torch.float8_e4m3fn, dev, T, H,
                   lambda: torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev))
    out_scales = _out(out_scales, "out_scales", torch.uint8, dev, T, H // 32,
                      lambda: torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    _check("moe_combine_mxfp8", lib().moe_combine_mxfp8(
        _ptr(payload), _ptr(src_info), _ptr(router_weights), _ptr(shared_out),
        _ptr(out_fp8), _ptr(out_scales), T, H, k, ep, mtpr, _stream(dev)))
    return out_fp8, out_scales


def moe_combine_residual_rmsnorm_mxfp8(payload, src_info, router_weights, shared_out,
                                       residual_in, gamma, eps, weight_bias=0.0,
                                       residual_out=None, out_fp8=None, out_scales=None,
                                       norm_out=None, want_norm_out=False):
    """Combine + residual add + RMSNorm, normalised row quantised to MXFP8.
    Returns (residual_out, out_fp8, out_scales, norm_out); norm_out (bf16) is
    written only if passed in or ``want_norm_out`` is set, else None."""
    dev, (T, H, k, ep, mtpr) = _common(payload, src_info, router_weights, shared_out)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP8")
    _need(residual_in, "residual_in", torch.bfloat16, dev, 2)
    if residual_in.shape[0] < T or residual_in.shape[1] != H:
        raise ValueError(f"residual_in must be [>= {T}, {H}]")
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    if gamma.shape[0] != H:
        raise ValueError(f"gamma must be [{H}]")
    mk = lambda: torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    residual_out = _out(residual_out, "residual_out", torch.bfloat16, dev, T, H, mk)
    out_fp8 = _out(out_fp8, "out_fp8", torch.float8_e4m3fn, dev, T, H,
                   lambda: torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev))
    out_scales = _out(out_scales, "out_scales", torch.uint8, dev, T, H // 32,
                      lambda: torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    if norm_out is not None or want_norm_out:
        norm_out = _out(norm_out, "norm_out", torch.bfloat16, dev, T, H, mk)
    wb = 0.0 if weight_bias is None else float(weight_bias)
    _check("moe_combine_residual_rmsnorm_mxfp8", lib().moe_combine_residual_rmsnorm_mxfp8(
        _ptr(payload), _ptr(src_info), _ptr(router_weights), _ptr(shared_out),
        _ptr(residual_in), _ptr(gamma), float(eps), wb, _ptr(residual_out),
        _ptr(norm_out), _ptr(out_fp8), _ptr(out_scales), T, H, k, ep, mtpr, _stream(dev)))
    return residual_out, out_fp8, out_scales, norm_out


def moe_combine_mxfp4(payload, src_info, router_weights=None, shared_out=None,
                      out_fp4=None, out_scales=None):
    """MXFP4 combine; returns (out_fp4 uint8 [T, H/2], two e2m1 codes per
    byte with element 2i in the low nibble, out_scales uint8 [T, H/32] UE8M0)."""
    dev, (T, H, k, ep, mtpr) = _common(payload, src_info, router_weights, shared_out)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP4")
    out_fp4 = _out(out_fp4, "out_fp4", torch.uint8, dev, T, H // 2,
                   lambda: torch.empty((T, H // 2), dtype=torch.uint8, device=dev))
    out_scales = _out(out_scales, "out_scales", torch.uint8, dev, T, H // 32,
                      lambda: torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    _check("moe_combine_mxfp4", lib().moe_combine_mxfp4(
        _ptr(payload), _ptr(src_info), _ptr(router_weights), _ptr(shared_out),
        _ptr(out_fp4), _ptr(out_scales), T, H, k, ep, mtpr, _stream(dev)))
    return out_fp4, out_scales


def _dense(inputs, scales, token_input):
    if not isinstance(inputs, torch.Tensor) or inputs.device.type != "cuda":
        raise ValueError("inputs must be a GPU tensor")
    dev = inputs.device
    _need(inputs, "inputs", torch.bfloat16, dev, 3)
    n_in, T, H = inputs.shape
    if scales is not None:
        _need(scales, "scales", torch.float32, dev, 2)
        if tuple(scales.shape) != (T, n_in):
            raise ValueError(f"scales must be [{T}, {n_in}]")
    if token_input is not None:
        _need(token_input, "token_input", torch.bfloat16, dev, 2)
        if tuple(token_input.shape) != (T, H):
            raise ValueError(f"token_input must be [{T}, {H}]")
    return dev, n_in, T, H


def moe_reduce_dense(inputs, scales=None, token_input=None, out=None):
    """Weighted sum of expert-major inputs [n_in, T, H] (unit scales if None:
    the plain sum of n_in partial buffers), plus token_input; bf16 [T, H]."""
    dev, n_in, T, H = _dense(inputs, scales, token_input)
    out = _out(out, "out", torch.bfloat16, dev, T, H,
               lambda: torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    _check("moe_reduce_dense", lib().moe_reduce_dense(
        _ptr(inputs), n_in, _ptr(scales), _ptr(token_input), _ptr(out), T, H, _stream(dev)))
    return out


def moe_reduce_dense_residual_rmsnorm(inputs, scales, token_input, residual_in, gamma, eps,
                                      weight_bias=0.0, residual_out=None, norm_out=None):
    """moe_reduce_dense + residual add + RMSNorm; returns (residual_out, norm_out)."""
    dev, n_in, T, H = _dense(inputs, scales, token_input)
    _need(residual_in, "residual_in", torch.bfloat16, dev, 2)
    if residual_in.shape[0] < T or residual_in.shape[1] != H:
        raise ValueError(f"residual_in must be [>= {T}, {H}]")
    _need(gamma, "gamma", torch.bfloat16, dev, 1)
    if gamma.shape[0] != H:
        raise ValueError(f"gamma must be [{H}]")
    mk = lambda: torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    residual_out = _out(residual_out, "residual_out", torch.bfloat16, dev, T, H, mk)
    norm_out = _out(norm_out, "norm_out", torch.bfloat16, dev, T, H, mk)
    wb = 0.0 if weight_bias is None else float(weight_bias)
    _check("moe_reduce_dense_residual_rmsnorm", lib().moe_reduce_dense_residual_rmsnorm(
        _ptr(inputs), n_in, _ptr(scales), _ptr(token_input), _ptr(residual_in), _ptr(gamma),
        float(eps), wb, _ptr(residual_out), _ptr(norm_out), T, H, _stream(dev)))
    return residual_out, norm_out


def dispatch_workspace_size(num_tokens: int, top_k: int, num_experts: int, ep_size: int,
                            max_tokens_per_rank: int) -> int:
    return int(lib().moe_dispatch_workspace_size(num_tokens, top_k, num_experts, ep_size,
                                                 max_tokens_per_rank))


def moe_dispatch(x, topk_ids, num_experts, ep_size, max_tokens_per_rank, payload=None,
                 src_info=None, recv_counts=None, workspace=None):
    """Forward scatter: returns (payload bf16 [ep, mtpr, H], src_info int32
    [T, k, 2]). recv_counts (int32 [E]) is accumulated in place if given.
    A workspace is allocated with torch when none is passed."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(topk_ids, "topk_ids", torch.int32, dev, 2)
    T, H = x.shape
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must be [T, top_k]")
    k = topk_ids.shape[1]
    if payload is None:
        payload = torch.zeros((ep_size, max_tokens_per_rank, H), dtype=torch.bfloat16, device=dev)
    _need(payload, "payload", torch.bfloat16, dev, 3)
    if tuple(payload.shape) != (ep_size, max_tokens_per_rank, H):
        raise ValueError(f"payload must be [{ep_size}, {max_tokens_per_rank}, {H}]")
    if src_info is None:
        src_info = torch.empty((T, k, 2), dtype=torch.int32, device=dev)
    _need(src_info, "src_info", torch.int32, dev, 3)
    if tuple(src_info.shape) != (T, k, 2):
        raise ValueError(f"src_info must be [{T}, {k}, 2]")
    if recv_counts is not None:
        _need(recv_counts, "recv_counts", torch.int32, dev, 1)
        if recv_counts.shape[0] != num_experts:
            raise ValueError(f"recv_counts must be [{num_experts}]")
    need = dispatch_workspace_size(T, k, num_experts, ep_size, max_tokens_per_rank)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)
    _check("moe_dispatch", lib().moe_dispatch(
        _ptr(x), _ptr(topk_ids), T, H, k, num_experts, ep_size, max_tokens_per_rank,
        _ptr(payload), _ptr(src_info), _ptr(recv_counts), _ptr(workspace), workspace.numel(),
        _stream(dev)))
    return payload, src_info


def moe_dispatch_noalloc(x, topk_ids, num_experts, ep_size, payload, src_info, recv_counts=None):
    """moe_dispatch without a workspace: the library's own device scratch
    (8 MiB per GPU) holds the count + scan path's intermediates, and nothing
    is allocated. payload [ep, mtpr, H] and src_info [T, k, 2] are the
    caller's outputs; recv_counts (int32 [E]) accumulates if given. Calls
    that may overlap on one GPU race on the shared scratch."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    dev = x.device
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(topk_ids, "topk_ids", torch.int32, dev, 2)
    T, H = x.shape
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must be [T, top_k]")
    k = topk_ids.shape[1]
    _need(payload, "payload", torch.bfloat16, dev, 3)
    if payload.shape[0] != ep_size or payload.shape[2] != H:
        raise ValueError(f"payload must be [{ep_size}, max_tokens_per_rank, {H}]")
    _need(src_info, "src_info", torch.int32, dev, 3)
    if tuple(src_info.shape) != (T, k, 2):
        raise ValueError(f"src_info must be [{T}, {k}, 2]")
    if recv_counts is not None:
        _need(recv_counts, "recv_counts", torch.int32, dev, 1)
        if recv_counts.shape[0] != num_experts:
            raise ValueError(f"recv_counts must be [{num_experts}]")
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        _ptr(x), _ptr(topk_ids), T, H, k, num_experts, ep_size, payload.shape[1],
        _ptr(payload), _ptr(src_info), _ptr(recv_counts), _stream(dev)))
    return payload, src_info
