"""CPU oracle of the MoE expert combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, scalar, OpenMP over tokens,
compiled without implicit fused multiply-add); this module only marshals numpy
arrays to it through ctypes. What each function computes, with the passages of
the documentation pages it follows, is stated in ``oracle.c``:

* ``combine``                   -- bf16 combine (routed fp32 sum, optional
                                   shared expert, RNE to bf16);
* ``combine_residual_rmsnorm``  -- + residual add and RMSNorm (weight_bias);
* ``combine_mxfp8``             -- + MXFP8 e4m3 codes and UE8M0 scales / 32;
* ``combine_residual_rmsnorm_mxfp8`` -- RMSNorm whose normalised row is also
                                   quantised to MXFP8;
* ``combine_mxfp4``             -- + MXFP4 e2m1 codes (two per byte) and
                                   UE8M0 scales / 32;
* ``reduce_dense``              -- weighted sum of expert-major dense inputs
                                   [n_in, T, H] (+ token input, + residual
                                   and RMSNorm): the local reduce;
* ``dispatch``                  -- the forward scatter the combine inverts
                                   (stable by expert, capacity, receive counts);
* ``routed_sum_f32``            -- the fp32 sum before any epilogue;
* ``bf16_rne``, ``e4m3_rne_sat``, ``mx_exponent``, ``e2m1_rne_sat``,
  ``mx4_exponent`` -- the scalar conversions.

Inputs are numpy arrays: bf16 tensors as uint16 bit patterns, ``src_info``
int32 [T, k, 2] (rank, row) with rank < 0 = dropped slot, ``weights`` float32
[T, k] or None (unit weights).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")

# MOE_ORACLE_SANITIZE=1 selects a build with the host AddressSanitizer and
# UndefinedBehaviorSanitizer (same arithmetic flags); a process that loads it
# must have libasan preloaded (tests/test_sanitizers.py does this).
SANITIZE = os.environ.get("MOE_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o",
           _LIB_PATH, "-lm"]
SANITIZE_FLAGS = ["-fsanitize=address,undefined,float-cast-overflow",
                  "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc if the library is missing or stale."""
    if (force or not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = GCC_CMD[:-3] + (SANITIZE_FLAGS if SANITIZE else []) + ["-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        F = ctypes.c_float
        common = [P, P, P, P]
        dims = [I64, I64, I, I, I64, I]
        lib.oracle_routed_sum_f32.argtypes = common + [P] + dims
        lib.oracle_combine.argtypes = common + [P] + dims
        lib.oracle_combine_residual_rmsnorm.argtypes = (
            common + [P, P, F, F, P, P] + dims)
        lib.oracle_combine_mxfp8.argtypes = common + [P, P] + dims
        lib.oracle_combine_residual_rmsnorm_mxfp8.argtypes = (
            common + [P, P, F, F, P, P, P, P] + dims)
        lib.oracle_combine_mxfp4.argtypes = common + [P, P] + dims
        lib.oracle_reduce_dense.argtypes = [P, I, P, P, P, P, F, F, P, P, I64, I64]
        lib.oracle_reduce_dense.restype = I
        lib.oracle_dispatch.argtypes = [P, P, I64, I64, I, I, I, I64, P, P, P]
        lib.oracle_dispatch.restype = I
        for f in ("oracle_routed_sum_f32", "oracle_combine",
                  "oracle_combine_residual_rmsnorm", "oracle_combine_mxfp8",
                  "oracle_combine_residual_rmsnorm_mxfp8", "oracle_combine_mxfp4"):
            getattr(lib, f).restype = I
        lib.oracle_bf16_rne.argtypes = [F]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_e4m3_rne_sat.argtypes = [F]
        lib.oracle_e4m3_rne_sat.restype = ctypes.c_uint8
        lib.oracle_mx_exponent.argtypes = [F]
        lib.oracle_mx_exponent.restype = I
        lib.oracle_mx4_exponent.argtypes = [F]
        lib.oracle_mx4_exponent.restype = I
        lib.oracle_e2m1_rne_sat.argtypes = [F]
        lib.oracle_e2m1_rne_sat.restype = ctypes.c_uint8
        lib.oracle_set_num_threads.argtypes = [I]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


def _prep(payload, src_info, weights, shared):
    payload = np.ascontiguousarray(payload, dtype=np.uint16)
    src_info = np.ascontiguousarray(src_info, dtype=np.int32)
    if payload.ndim != 3 or src_info.ndim != 3 or src_info.shape[2] != 2:
        raise ValueError("payload [ep, mtpr, H] and src_info [T, k, 2] expected")
    ep, mtpr, H = payload.shape
    T, k, _ = src_info.shape
    if weights is not None:
        weights = np.ascontiguousarray(weights, dtype=np.float32)
        if weights.shape != (T, k):
            raise ValueError("weights must be [T, k]")
    if shared is not None:
        shared = np.ascontiguousarray(shared, dtype=np.uint16)
        if shared.shape != (T, H):
            raise ValueError("shared must be [T, H]")
    return payload, src_info, weights, shared, (T, H, k, ep, mtpr)


def _rc(rc):
    if rc == 1:
        raise OracleError("slot map points outside the payload")
    if rc:
        raise OracleError("invalid arguments (%d)" % rc)


def routed_sum_f32(payload, src_info, weights=None, shared=None, checked=True):
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    acc = np.empty((T, H), dtype=np.float32)
    _rc(_L().oracle_routed_sum_f32(_ptr(payload), _ptr(src_info), _ptr(weights),
                                   _ptr(shared), _ptr(acc), T, H, k, ep, mtpr,
                                   int(checked)))
    return acc


def combine(payload, src_info, weights=None, shared=None, checked=True):
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    out = np.empty((T, H), dtype=np.uint16)
    _rc(_L().oracle_combine(_ptr(payload), _ptr(src_info), _ptr(weights),
                            _ptr(shared), _ptr(out), T, H, k, ep, mtpr,
                            int(checked)))
    return out


def combine_residual_rmsnorm(payload, src_info, weights, shared, residual,
                             gamma, eps, weight_bias=0.0, checked=True):
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    if residual.shape != (T, H) or gamma.shape != (H,):
        raise ValueError("residual [T, H] and gamma [H] expected")
    ro = np.empty((T, H), dtype=np.uint16)
    no = np.empty((T, H), dtype=np.uint16)
    _rc(_L().oracle_combine_residual_rmsnorm(
        _ptr(payload), _ptr(src_info), _ptr(weights), _ptr(shared),
        _ptr(residual), _ptr(gamma), float(eps),
        float(0.0 if weight_bias is None else weight_bias), _ptr(ro), _ptr(no),
        T, H, k, ep, mtpr, int(checked)))
    return ro, no


def combine_mxfp8(payload, src_info, weights=None, shared=None, checked=True):
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP8")
    codes = np.empty((T, H), dtype=np.uint8)
    scales = np.empty((T, H // 32), dtype=np.uint8)
    _rc(_L().oracle_combine_mxfp8(_ptr(payload), _ptr(src_info), _ptr(weights),
                                  _ptr(shared), _ptr(codes), _ptr(scales), T, H,
                                  k, ep, mtpr, int(checked)))
    return codes, scales


def combine_residual_rmsnorm_mxfp8(payload, src_info, weights, shared, residual,
                                   gamma, eps, weight_bias=0.0, checked=True):
    """Returns (residual_out bf16 bits, norm_out bf16 bits, codes, scales)."""
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP8")
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    if residual.shape != (T, H) or gamma.shape != (H,):
        raise ValueError("residual [T, H] and gamma [H] expected")
    ro = np.empty((T, H), dtype=np.uint16)
    no = np.empty((T, H), dtype=np.uint16)
    codes = np.empty((T, H), dtype=np.uint8)
    scales = np.empty((T, H // 32), dtype=np.uint8)
    _rc(_L().oracle_combine_residual_rmsnorm_mxfp8(
        _ptr(payload), _ptr(src_info), _ptr(weights), _ptr(shared),
        _ptr(residual), _ptr(gamma), float(eps),
        float(0.0 if weight_bias is None else weight_bias), _ptr(ro), _ptr(no),
        _ptr(codes), _ptr(scales), T, H, k, ep, mtpr, int(checked)))
    return ro, no, codes, scales


def combine_mxfp4(payload, src_info, weights=None, shared=None, checked=True):
    """Returns (packed e2m1 codes uint8 [T, H/2], UE8M0 scales uint8 [T, H/32])."""
    payload, src_info, weights, shared, (T, H, k, ep, mtpr) = _prep(
        payload, src_info, weights, shared)
    if H % 32:
        raise ValueError("hidden must be a multiple of 32 for MXFP4")
    codes = np.empty((T, H // 2), dtype=np.uint8)
    scales = np.empty((T, H // 32), dtype=np.uint8)
    _rc(_L().oracle_combine_mxfp4(_ptr(payload), _ptr(src_info), _ptr(weights),
                                  _ptr(shared), _ptr(codes), _ptr(scales), T, H,
                                  k, ep, mtpr, int(checked)))
    return codes, scales


def reduce_dense(x, scales=None, tok=None, residual=None, gamma=None, eps=1e-6,
                 weight_bias=0.0):
    """x: bf16 bits [n_in, T, H]; scales fp32 [T, n_in] or None; tok bf16
    [T, H] or None. Returns out bf16 [T, H], or (residual_out, norm_out)
    when residual and gamma are given."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n_in, T, H = x.shape
    if scales is not None:
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        assert scales.shape == (T, n_in)
    if tok is not None:
        tok = np.ascontiguousarray(tok, dtype=np.uint16)
        assert tok.shape == (T, H)
    out = np.empty((T, H), dtype=np.uint16)
    no = None
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        no = np.empty((T, H), dtype=np.uint16)
    _rc(_L().oracle_reduce_dense(_ptr(x), n_in, _ptr(scales), _ptr(tok), _ptr(residual),
                                 _ptr(gamma), float(eps),
                                 float(0.0 if weight_bias is None else weight_bias),
                                 _ptr(out), _ptr(no), T, H))
    return out if residual is None else (out, no)


def dispatch(x, topk_ids, E, ep, mtpr, payload=None, recv_counts=None):
    """x bf16 bits [T, H]; topk_ids int32 [T, k] (-1 = dropped slot).
    Returns (payload [ep, mtpr, H], src_info [T, k, 2], recv_counts [E]);
    ``payload`` / ``recv_counts`` given are updated in place (rows no pair
    is placed in keep their contents; counts accumulate)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, H = x.shape
    k = topk_ids.shape[1]
    if payload is None:
        payload = np.zeros((ep, mtpr, H), dtype=np.uint16)
    if recv_counts is None:
        recv_counts = np.zeros(E, dtype=np.int32)
    src = np.empty((T, k, 2), dtype=np.int32)
    _rc(_L().oracle_dispatch(_ptr(x), _ptr(topk_ids), T, H, k, E, ep, mtpr,
                             _ptr(payload), _ptr(src), _ptr(recv_counts)))
    return payload, src, recv_counts


def e2m1_rne_sat(x: float) -> int:
    return int(_L().oracle_e2m1_rne_sat(float(x)))


def mx4_exponent(amax: float) -> int:
    return int(_L().oracle_mx4_exponent(float(amax)))


def bf16_rne(x: float) -> int:
    return int(_L().oracle_bf16_rne(float(x)))


def e4m3_rne_sat(x: float) -> int:
    return int(_L().oracle_e4m3_rne_sat(float(x)))


def mx_exponent(amax: float) -> int:
    return int(_L().oracle_mx_exponent(float(amax)))


def set_threads(n: int) -> None:
    _L().oracle_set_num_threads(int(n))


def max_threads() -> int:
    return int(_L().oracle_max_threads())
