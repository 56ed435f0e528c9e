"""Pins of the CPU oracle to facts fixed outside it (no GPU needed).

Each test checks the oracle against something other than itself: hand-worked
fixtures under ``tests/golden``, closed forms, invariants, exact-rational brute
force (``tests/_brute.py``), library routines (torch CPU casts, float64
``rms_norm``) and error bounds. Every part of the oracle is covered by at least
one pin that a plausible mistake (dropped term, wrong sign or index, swapped
operand, wrong rounding or tie rule) would break.
"""
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

import gen
import oracle
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def to_bf16_bits(x):
    """float array -> bf16 bits via torch's CPU cast (RNE)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ulp_dist_bf16(a, b):
    """Distance in bf16 steps on the monotone integer line (NaN -> huge)."""
    def key(u):
        u = np.asarray(u, dtype=np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    d = np.abs(key(a) - key(b))
    nan_a = (np.asarray(a) & 0x7FFF) > 0x7F80
    nan_b = (np.asarray(b) & 0x7FFF) > 0x7F80
    d = np.where(nan_a & nan_b, 0, d)
    return np.where(nan_a ^ nan_b, 1 << 20, d)


def _num(tok):
    tok = tok.strip()
    if tok == "nan":
        return float("nan")
    if "^" in tok:
        neg = tok.startswith("-")
        t = tok.lstrip("-")
        if "*" in t:
            m, p = t.split("*")
            v = float(m) * 2.0 ** int(p.split("^")[1])
        else:
            v = 2.0 ** int(t.split("^")[1])
        return -v if neg else v
    return float(tok)


def load_fixture(name):
    lines = [l.rstrip("\n") for l in open(os.path.join(GOLDEN, name))]
    lines = [l for l in lines if l.strip() and not l.startswith("#")]
    fx = {"rows": {}, "slots": {}, "expect": {}, "residual": {}, "cases": [],
          "x": {}, "scales": {}, "codes": {}, "expect_residual": {}}
    cur = None
    for l in lines:
        head, _, body = l.partition(":")
        hs = head.split()
        if hs[0] == "dims":
            fx["dims"] = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in hs[1:]}
        elif hs[0] == "row":
            fx["rows"][(int(hs[1]), int(hs[2]))] = [_num(v) for v in body.split()]
        elif hs[0] == "slot":
            r, row, w = body.split()
            fx["slots"][(int(hs[1]), int(hs[2]))] = (int(r), int(row), float(w))
        elif hs[0] == "expect":
            fx["expect"][int(hs[1])] = [_num(v) for v in body.split()]
        elif hs[0] == "residual":
            fx["residual"][int(hs[1])] = [_num(v) for v in body.split()]
        elif hs[0] == "gamma":
            fx["gamma"] = [_num(v) for v in body.split()]
        elif hs[0] == "expect_residual":
            fx["expect_residual"][int(hs[1])] = [_num(v) for v in body.split()]
        elif hs[0] == "case":
            cur = {"name": hs[1], "norm": {}}
            for kv in hs[2:]:
                k_, v_ = kv.split("=")
                cur[k_] = float(v_)
            fx["cases"].append(cur)
        elif hs[0] == "expect_norm":
            cur["norm"][int(hs[1])] = [_num(v) for v in body.split()]
        elif hs[0] == "x":
            b = body.split()
            fx["x"][int(hs[1])] = (("negate", int(b[1])) if b[0] == "negate"
                                   else [_num(v) for v in b])
        elif hs[0] == "scales":
            fx["scales"][int(hs[1])] = [int(v) for v in body.split()]
        elif hs[0] == "codes" and cur is not None:
            cur.setdefault("codes", {})[int(hs[1])] = [int(v, 16) for v in body.split()]
        elif hs[0] == "codes":
            fx["codes"][int(hs[1])] = [int(v, 16) for v in body.split()]
        elif hs[0] == "scale":
            cur.setdefault("scale", {})[int(hs[1])] = [int(v) for v in body.split()]
        else:
            raise ValueError(l)
    return fx


def build_arrays(fx):
    d = fx["dims"]
    payload = np.zeros((d["ep"], d["mtpr"], d["H"]), dtype=np.uint16)
    for (r, row), vals in fx["rows"].items():
        payload[r, row] = to_bf16_bits(vals)
    src = np.full((d["T"], d["k"], 2), -1, dtype=np.int32)
    w = np.zeros((d["T"], d["k"]), dtype=np.float32)
    for (t, j), (r, row, wj) in fx["slots"].items():
        src[t, j] = (r, row)
        w[t, j] = wj
    return payload, src, w


# ------------------------------------------------------- golden fixtures

def test_golden_combine():
    fx = load_fixture("combine_small.txt")
    payload, src, w = build_arrays(fx)
    out = oracle.combine(payload, src, w)
    for t, vals in fx["expect"].items():
        np.testing.assert_array_equal(out[t], to_bf16_bits(vals), err_msg=f"token {t}")


def test_golden_rmsnorm():
    fx = load_fixture("rmsnorm_small.txt")
    payload, src, w = build_arrays(fx)
    res = np.stack([to_bf16_bits(fx["residual"][t]) for t in sorted(fx["residual"])])
    gamma = to_bf16_bits(fx["gamma"])
    assert len(fx["cases"]) == 4
    for case in fx["cases"]:
        ro, no = oracle.combine_residual_rmsnorm(
            payload, src, w, None, res, gamma, case["eps"], case["weight_bias"])
        for t, vals in fx["expect_residual"].items():
            np.testing.assert_array_equal(ro[t], to_bf16_bits(vals))
        for t, vals in case["norm"].items():
            np.testing.assert_array_equal(no[t], to_bf16_bits(vals),
                                          err_msg=case["name"])


def test_golden_mxfp8():
    fx = load_fixture("mxfp8_small.txt")
    d = fx["dims"]
    x0 = np.array(fx["x"][0], dtype=np.float32)
    assert fx["x"][1] == ("negate", 0)
    payload = np.stack([to_bf16_bits(x0), to_bf16_bits(-x0)])[None]
    # bf16 must hold every hand value exactly, else the fixture is wrong
    np.testing.assert_array_equal(bf16_to_f32(payload[0, 0]), x0)
    _, src, w = build_arrays({"dims": d, "rows": {}, "slots": fx["slots"]})
    codes, scales = oracle.combine_mxfp8(payload, src, w)
    for t in range(2):
        assert list(scales[t]) == fx["scales"][t], f"scales token {t}"
        assert list(codes[t]) == fx["codes"][t], f"codes token {t}"


# ------------------------------------------------------ P1: inverse map

@pytest.mark.parametrize("ep,mtpr_pad", [(1, 0), (4, 37), (8, 128)])
@pytest.mark.parametrize("unit", ["none", "ones"])
def test_inverse_permutation_bit_exact(ep, mtpr_pad, unit):
    """top_k = 1 with weight 1: combine(dispatch(x)) returns x exactly
    (the combine is the inverse of the dispatch scatter)."""
    rng = np.random.default_rng(11)
    T, H, E = 97, 64, 16
    x = to_bf16_bits(rng.standard_normal((T, H)) * 3)
    topk = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    src, loads = gen.dispatch_slots(topk, np.zeros((T, 1), bool), E, ep, None)
    mtpr = int(loads.max()) + mtpr_pad
    payload = gen.scatter_rows(src, x[:, None, :], ep, mtpr,
                               fill=np.full((ep, mtpr, H), 0x7FC0, np.uint16))
    w = None if unit == "none" else np.ones((T, 1), np.float32)
    out = oracle.combine(payload, src, w)
    np.testing.assert_array_equal(out, x)


# --------------------------------------------- P2: identity experts

def test_identity_experts_sum_of_weights():
    """Every expert returns its input row unchanged: out = bf16(x * sum_j w_j)
    within one bf16 step (only the fp32 accumulation separates them)."""
    rng = np.random.default_rng(5)
    T, H, E, k, ep = 64, 256, 32, 8, 4
    x = to_bf16_bits(rng.standard_normal((T, H)))
    inp = gen.make_inputs(dict(T=T, H=H, E=E, ep=ep, k=k), seed=3)
    payload = gen.scatter_rows(inp.src_info, np.repeat(x[:, None, :], k, axis=1),
                               ep, inp.mtpr)
    out = oracle.combine(payload, inp.src_info, inp.weights)
    ws = inp.weights.astype(np.float64).sum(axis=1)
    ref = to_bf16_bits(bf16_to_f32(x).astype(np.float64) * ws[:, None])
    assert ulp_dist_bf16(out, ref).max() <= 1


# ------------------------------------------------------------ P3: drops

def test_drop_equals_zero_weight_and_all_dropped():
    inp = gen.make_inputs(dict(T=40, H=128, E=16, ep=2, k=4, shared_sd=0.5), seed=7)
    rng = np.random.default_rng(0)
    mask = rng.random((inp.T, inp.k)) < 0.3
    src_d = inp.src_info.copy()
    src_d[mask] = -1
    w0 = inp.weights.copy()
    w0[mask] = 0.0
    for shared in (None, inp.shared):
        a = oracle.combine(inp.payload, src_d, inp.weights, shared)
        b = oracle.combine(inp.payload, inp.src_info, w0, shared)
        np.testing.assert_array_equal(a, b)
    src_all = np.full_like(inp.src_info, -1)
    z = oracle.combine(inp.payload, src_all, inp.weights)
    assert (z == 0).all()                     # +0.0 exactly
    s = oracle.combine(inp.payload, src_all, inp.weights, inp.shared)
    np.testing.assert_array_equal(s, inp.shared)


# ------------------------------------------------ P4: layout invariance

def test_layout_invariance():
    """The same (token, slot) rows placed under different ep_size, capacity
    and row order give bit-identical output: accumulation follows slot order,
    not payload order."""
    rng = np.random.default_rng(9)
    T, H, E, k = 50, 96, 24, 6
    rows = to_bf16_bits(rng.standard_normal((T, k, H)))
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    outs = []
    for ep, pad, shuffle in [(1, 0, False), (4, 5, False), (8, 64, True), (2, 1, True)]:
        src, loads = gen.dispatch_slots(topk, np.zeros((T, k), bool), E, ep, None)
        mtpr = int(loads.max()) + pad
        if shuffle:
            perm = np.stack([rng.permutation(mtpr) for _ in range(ep)])
            v = src[..., 0] >= 0
            src[..., 1][v] = perm[src[..., 0][v], src[..., 1][v]]
        payload = gen.scatter_rows(src, rows, ep, mtpr)
        outs.append(oracle.combine(payload, src, w))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


# ------------------------------------------------- P5: exact arithmetic

def test_exact_dyadic_sums():
    """Small integers * 2^-4 with weights in {1/8, ..., 8/8}: every fp32
    operation is exact, so the output is the exact sum rounded once to bf16."""
    rng = np.random.default_rng(21)
    T, H, k, ep, mtpr = 30, 64, 8, 2, 200
    vals = rng.integers(-16, 17, size=(ep, mtpr, H)) / 16.0
    payload = to_bf16_bits(vals)
    assert (bf16_to_f32(payload) == vals).all()
    src = np.stack([rng.integers(0, ep, (T, k)), rng.integers(0, mtpr, (T, k))],
                   axis=-1).astype(np.int32)
    w = (rng.integers(1, 9, size=(T, k)) / 8.0).astype(np.float32)
    out = oracle.combine(payload, src, w)
    exact = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            exact[t] += w[t, j] * vals[src[t, j, 0], src[t, j, 1]]
    np.testing.assert_array_equal(out, to_bf16_bits(exact))


# ------------------------------------------ P6: exact-rational brute force

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_routed_sum(seed):
    """fp32 fused multiply-add chain in exact rationals, one rounding per
    step, ascending slot order; then bf16 via torch's cast."""
    inp = gen.make_inputs(dict(T=5, H=16, E=6, ep=2, k=3, shared_sd=2.0,
                               drop_frac=0.2), seed=seed)
    pf = bf16_to_f32(inp.payload)
    sf = bf16_to_f32(inp.shared)
    ref = np.array(_brute.brute_routed_sum(pf, inp.src_info, inp.weights, sf),
                   dtype=np.float32)
    acc = oracle.routed_sum_f32(inp.payload, inp.src_info, inp.weights, inp.shared)
    np.testing.assert_array_equal(acc.view(np.uint32), ref.view(np.uint32))
    out = oracle.combine(inp.payload, inp.src_info, inp.weights, inp.shared)
    np.testing.assert_array_equal(out, to_bf16_bits(ref))


def test_round_f32_brute_matches_numpy_on_doubles():
    """The brute-force rounding agrees with the double->float cast."""
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-40, 38, 500),
                         [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** -149 * 1.5]])
    for x in xs:
        assert _brute.round_f32(Fraction(float(x))) == float(np.float32(x))


def test_fp32_accumulation_error_bound():
    """The fp32 sum is within the recursive-summation bound of the exact sum
    (k roundings of relative size <= 2^-24 each)."""
    inp = gen.make_inputs(dict(T=256, H=512, E=64, ep=8, k=8, shared_sd=0.5), seed=4)
    acc = oracle.routed_sum_f32(inp.payload, inp.src_info, inp.weights, inp.shared)
    pf = bf16_to_f32(inp.payload).astype(np.float64)
    exact = np.zeros((inp.T, inp.H))
    absum = np.zeros((inp.T, inp.H))
    for j in range(inp.k):
        r, row = inp.src_info[:, j, 0], inp.src_info[:, j, 1]
        term = inp.weights[:, j, None].astype(np.float64) * pf[r, row]
        exact += term
        absum += np.abs(term)
    sh = bf16_to_f32(inp.shared).astype(np.float64)
    exact += sh
    absum += np.abs(sh)
    bound = (inp.k + 1) * 2.0 ** -24 * absum * 1.0001
    assert (np.abs(acc - exact) <= bound).all()


# --------------------------------------------- P7: unoccupied rows unread

def test_unoccupied_rows_never_read():
    c = dict(T=64, H=256, E=32, ep=4, k=4, unoccupied="nan", drop_frac=0.25,
             shared_sd=0.5, residual_sd=1.0, gamma_sd=0.1)
    inp = gen.make_inputs(c, seed=2, mtpr=512)
    assert ((inp.payload & 0x7FFF) > 0x7F80).any()
    out = oracle.combine(inp.payload, inp.src_info, inp.weights, inp.shared)
    assert not ((out & 0x7FFF) > 0x7F80).any()
    ro, no = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                             inp.shared, inp.residual, inp.gamma, 1e-6, 1.0)
    assert not ((ro & 0x7FFF) > 0x7F80).any() and not ((no & 0x7FFF) > 0x7F80).any()
    codes, scales = oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights, inp.shared)
    assert not ((codes & 0x7F) == 0x7F).any() and not (scales == 0xFF).any()


def test_checked_mode_rejects_out_of_range_slots():
    inp = gen.make_inputs("tiny", 0)
    bad = inp.src_info.copy()
    bad[3, 1] = (0, inp.mtpr)        # row past capacity
    with pytest.raises(oracle.OracleError):
        oracle.combine(inp.payload, bad, inp.weights)
    bad = inp.src_info.copy()
    bad[0, 0] = (inp.ep, 0)          # rank past ep_size
    with pytest.raises(oracle.OracleError):
        oracle.combine(inp.payload, bad, inp.weights)


# ----------------------------------------------------------- P8-P10: RMSNorm

def _rms_inputs(seed=1, T=24, H=512, **kw):
    c = dict(T=T, H=H, E=32, ep=4, k=8, residual_sd=1.0, gamma_sd=0.1)
    c.update(kw)
    return gen.make_inputs(c, seed=seed)


def test_rmsnorm_constant_gamma_closed_form():
    """gamma == c, weight_bias 0: RMS(norm_out) = c * sqrt(ms / (ms + eps))."""
    inp = _rms_inputs()
    c, eps = 1.5, 0.25
    gamma = to_bf16_bits(np.full(inp.H, c))
    ro, no = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                             None, inp.residual, gamma, eps, 0.0)
    x = bf16_to_f32(ro).astype(np.float64)
    ms = (x * x).mean(axis=1)
    y = bf16_to_f32(no).astype(np.float64)
    rms = np.sqrt((y * y).mean(axis=1))
    np.testing.assert_allclose(rms, c * np.sqrt(ms / (ms + eps)), rtol=2.0 ** -8)


def test_rmsnorm_weight_bias_identity():
    """(gamma == 0, weight_bias 1) is bit-identical to (gamma == 1, wb 0)."""
    inp = _rms_inputs(seed=2)
    g0 = to_bf16_bits(np.zeros(inp.H))
    g1 = to_bf16_bits(np.ones(inp.H))
    a = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights, None,
                                        inp.residual, g0, 1e-6, 1.0)
    b = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights, None,
                                        inp.residual, g1, 1e-6, 0.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_rmsnorm_matches_torch_float64(wb):
    """torch.nn.functional.rms_norm in float64 on residual_out, with weight
    gamma + weight_bias, rounded to bf16, is within one bf16 step; the
    residual stream equals bf16(fp32 sum + residual) exactly."""
    inp = _rms_inputs(seed=3, shared_sd=0.5)
    ro, no = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                             inp.shared, inp.residual, inp.gamma,
                                             inp.eps, wb)
    acc = oracle.routed_sum_f32(inp.payload, inp.src_info, inp.weights, inp.shared)
    s = torch.from_numpy(acc) + torch.from_numpy(bf16_to_f32(inp.residual))
    np.testing.assert_array_equal(
        ro, s.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    x = torch.from_numpy(bf16_to_f32(ro)).double()
    g = (torch.from_numpy(bf16_to_f32(inp.gamma)) + wb).double()
    ref = torch.nn.functional.rms_norm(x, (inp.H,), weight=g, eps=inp.eps)
    refb = ref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d = ulp_dist_bf16(no, refb)
    assert d.max() <= 1
    # both round double -> fp32 -> bf16, so only summation order separates
    # them: almost every element is identical. Normalising the unrounded
    # fp32 sum instead of residual_out would move about a quarter of them.
    assert (d != 0).mean() <= 1e-3


def test_rmsnorm_scale_invariance_eps0():
    """With eps = 0, scaling payload and residual by 2^j scales residual_out by
    2^j exactly and leaves norm_out bit-identical."""
    inp = _rms_inputs(seed=4)
    base = oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                           None, inp.residual, inp.gamma, 0.0, 0.0)
    for j in (-5, 3, 11):
        sc = lambda b: to_bf16_bits(bf16_to_f32(b).astype(np.float64) * 2.0 ** j)
        ro, no = oracle.combine_residual_rmsnorm(sc(inp.payload), inp.src_info,
                                                 inp.weights, None, sc(inp.residual),
                                                 inp.gamma, 0.0, 0.0)
        np.testing.assert_array_equal(ro, sc(base[0]))
        np.testing.assert_array_equal(no, base[1])


# ------------------------------------------------------------- P11-P14: MXFP8

def test_mx_exponent_closed_form():
    rng = np.random.default_rng(8)
    vals = np.concatenate([
        np.float32(2.0) ** np.arange(-149, 128, dtype=np.float64).astype(np.float32),
        (rng.random(2000) * 10.0 ** rng.integers(-44, 38, 2000)).astype(np.float32)])
    for a in vals:
        a = float(a)
        if a == 0.0:
            continue
        e = _brute.floor_log2(Fraction(a)) - 8
        assert oracle.mx_exponent(a) == max(-127, min(127, e)), a
    for n in range(-100, 100):
        assert oracle.mx_exponent(2.0 ** n) + 127 == max(0, n + 119)
    assert oracle.mx_exponent(0.0) == -127
    assert oracle.mx_exponent(float("nan")) + 127 == 0xFF
    assert oracle.mx_exponent(float("inf")) + 127 == 0xFF


def test_e4m3_exhaustive_over_bf16_patterns():
    """Every bf16 bit pattern (as an fp32 value) against nearest-code search."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    q = (bits << 16).view(np.float32)
    fin = np.isfinite(q)
    ref = _brute.nearest_e4m3_vec(q[fin].astype(np.float64))
    got = np.array([oracle.e4m3_rne_sat(float(v)) for v in q[fin]], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)
    for v in q[~fin]:
        c = oracle.e4m3_rne_sat(float(v))
        if np.isnan(v):
            assert c & 0x7F == 0x7F
        else:
            assert c & 0x7F == 0x7E and (c >> 7) == (v < 0)


def test_e4m3_random_fp32_and_scalar_brute():
    rng = np.random.default_rng(12)
    q = (rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 10, 20000)).astype(np.float32)
    got = np.array([oracle.e4m3_rne_sat(float(v)) for v in q], dtype=np.uint8)
    np.testing.assert_array_equal(got, _brute.nearest_e4m3_vec(q.astype(np.float64)))
    for v in q[:300]:
        assert oracle.e4m3_rne_sat(float(v)) == _brute.nearest_e4m3(float(v))


def test_e4m3_matches_torch_cast_after_clamp():
    """torch's CPU float8_e4m3fn cast of clamp(q, -448, 448)."""
    rng = np.random.default_rng(13)
    q = np.concatenate([(rng.standard_normal(50000) * 2.0 ** rng.integers(-12, 10, 50000)),
                        np.arange(-520, 520, 0.5)]).astype(np.float32)
    t = torch.from_numpy(q).clamp(-448, 448).to(torch.float8_e4m3fn)
    ref = t.view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_rne_sat(float(v)) for v in q], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_mxfp8_blocks_brute_force_and_bounds():
    """Tiny shapes: scales and codes from the exact-rational routed sum by
    search; every block then satisfies the MX invariants and the e4m3 error
    bound."""
    inp = gen.make_inputs(dict(T=6, H=64, E=8, ep=2, k=3, hot_row_frac=0.2,
                               hot_scale=64.0), seed=5)
    pf = bf16_to_f32(inp.payload)
    acc = np.array(_brute.brute_routed_sum(pf, inp.src_info, inp.weights), np.float64)
    codes, scales = oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights)
    for t in range(inp.T):
        for b in range(inp.H // 32):
            blk = acc[t, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = -127 if amax == 0 else max(-127, _brute.floor_log2(Fraction(amax)) - 8)
            assert scales[t, b] == e + 127
            for i, v in enumerate(blk):
                q = v * 2.0 ** -e
                c = int(codes[t, 32 * b + i])
                assert c == _brute.nearest_e4m3(q)
                dec = _brute.e4m3_decode(c)
                if abs(q) < 448:
                    E = max(_brute.floor_log2(Fraction(abs(q))) if q else -6, -6)
                    assert abs(dec - q) <= 0.5 * 2.0 ** (E - 3)
                else:
                    assert abs(dec) == 448.0
            if amax > 0 and e > -127:
                assert 256 <= amax * 2.0 ** -e < 512


def test_mxfp8_full_pipeline_consistency():
    """Codes and scales equal the scalar conversions applied to the oracle's
    own fp32 sums (links the fused path to the pinned scalar functions), on a
    generated workload with hot rows, drops and a shared expert."""
    inp = gen.make_inputs(dict(T=48, H=256, E=32, ep=4, k=8, hot_row_frac=0.05,
                               drop_frac=0.1, shared_sd=0.5), seed=6)
    codes, scales = oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights, inp.shared)
    acc = oracle.routed_sum_f32(inp.payload, inp.src_info, inp.weights, inp.shared)
    blocks = acc.reshape(inp.T, -1, 32)
    amax = np.abs(blocks).max(axis=2)
    e = np.vectorize(oracle.mx_exponent)(amax)
    np.testing.assert_array_equal(scales, (e + 127).astype(np.uint8))
    q = blocks * np.exp2(-e.astype(np.float64))[..., None]
    ref = _brute.nearest_e4m3_vec(q.reshape(-1)).reshape(inp.T, inp.H)
    np.testing.assert_array_equal(codes, ref)


# ------------------------------------------- RMSNorm + MXFP8 of the norm

def test_golden_rmsnorm_mxfp8():
    fx = load_fixture("rmsnorm_mxfp8_small.txt")
    payload, src, w = build_arrays(fx)
    res = to_bf16_bits(fx["residual"][0])[None]
    gamma = to_bf16_bits(fx["gamma"])
    assert len(fx["cases"]) == 2
    for case in fx["cases"]:
        ro, no, codes, scales = oracle.combine_residual_rmsnorm_mxfp8(
            payload, src, w, None, res, gamma, case["eps"], case["weight_bias"])
        np.testing.assert_array_equal(ro[0], to_bf16_bits([2, -2] * 16))
        assert list(scales[0]) == case["scale"][0], case["name"]
        assert list(codes[0]) == case["codes"][0], case["name"]


@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_rmsnorm_mxfp8_matches_independent_recomputation(wb):
    """The normalised row recomputed in numpy (exact sum of squares, float64
    scaling, fp32 rounding) and quantised by code search equals the oracle's
    codes and scales; residual_out and norm_out equal the RMSNorm oracle's."""
    inp = _rms_inputs(seed=7, T=16, H=1024, shared_sd=0.5)
    ro, no, codes, scales = oracle.combine_residual_rmsnorm_mxfp8(
        inp.payload, inp.src_info, inp.weights, inp.shared, inp.residual,
        inp.gamma, inp.eps, wb)
    ro2, no2 = oracle.combine_residual_rmsnorm(
        inp.payload, inp.src_info, inp.weights, inp.shared, inp.residual,
        inp.gamma, inp.eps, wb)
    np.testing.assert_array_equal(ro, ro2)
    np.testing.assert_array_equal(no, no2)
    x = bf16_to_f32(ro).astype(np.float64)
    ss = np.array([math.fsum(r * r) for r in x])
    rstd = 1.0 / np.sqrt(ss / inp.H + np.float64(np.float32(inp.eps)))
    g = (bf16_to_f32(inp.gamma) + np.float32(wb)).astype(np.float64)
    n = (x * rstd[:, None] * g[None, :]).astype(np.float32)
    np.testing.assert_array_equal(no, to_bf16_bits(n))
    blocks = n.astype(np.float64).reshape(inp.T, -1, 32)
    amax = np.abs(blocks).max(axis=2)
    e = np.array([[-127 if a == 0 else max(-127, _brute.floor_log2(Fraction(float(a))) - 8)
                   for a in row] for row in amax])
    np.testing.assert_array_equal(scales, (e + 127).astype(np.uint8))
    q = blocks * np.exp2(-e.astype(np.float64))[..., None]
    np.testing.assert_array_equal(codes, _brute.nearest_e4m3_vec(q.reshape(-1)).reshape(inp.T, inp.H))


# --------------------------------------------------------------- MXFP4

E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def nearest_e2m1(q):
    """Nearest e2m1 code by search over the 8 magnitudes (ties -> even code,
    saturating at 6), sign from q."""
    a = min(abs(Fraction(q)), Fraction(100)) if math.isfinite(q) else Fraction(100)
    best, bd = None, None
    for c, v in enumerate(E2M1_VALUES):
        d = abs(a - Fraction(v))
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x8 if math.copysign(1.0, q) < 0 else 0)


def test_golden_mxfp4():
    fx = load_fixture("mxfp4_small.txt")
    d = fx["dims"]
    x0 = np.array(fx["x"][0], dtype=np.float32)
    payload = to_bf16_bits(x0)[None, None]
    np.testing.assert_array_equal(bf16_to_f32(payload[0, 0]), x0)
    _, src, w = build_arrays({"dims": d, "rows": {}, "slots": fx["slots"]})
    codes, scales = oracle.combine_mxfp4(payload, src, w)
    assert list(scales[0]) == fx["scales"][0]
    assert list(codes[0]) == fx["codes"][0]


def test_e2m1_exhaustive_over_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    q = (bits << 16).view(np.float32)
    vals = np.array(E2M1_VALUES)
    fin = q[np.isfinite(q)].astype(np.float64)
    a = np.minimum(np.abs(fin), 100.0)
    dist = np.abs(a[:, None] - vals[None, :])
    dmin = dist.min(axis=1, keepdims=True)
    tie = dist == dmin
    even = tie & (np.arange(8)[None, :] % 2 == 0)
    ref = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
    ref = ref | np.where(np.signbit(fin), 8, 0)
    got = np.array([oracle.e2m1_rne_sat(float(v)) for v in fin])
    np.testing.assert_array_equal(got, ref)
    for v in q[~np.isfinite(q)][:50]:
        assert oracle.e2m1_rne_sat(float(v)) & 0x7 == 0x7
    for v in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.3, 5.9, -7.0, 1e30]:
        assert oracle.e2m1_rne_sat(v) == nearest_e2m1(v), v


def test_mx4_exponent_closed_form():
    rng = np.random.default_rng(9)
    for a in np.concatenate([2.0 ** np.arange(-149, 128),
                             rng.random(500) * 10.0 ** rng.integers(-44, 38, 500)]).astype(np.float32):
        a = float(a)
        if a == 0:
            continue
        e = _brute.floor_log2(Fraction(a)) - 2
        assert oracle.mx4_exponent(a) == max(-127, min(127, e)), a
    assert oracle.mx4_exponent(0.0) == -127
    assert oracle.mx4_exponent(float("nan")) == 128


def test_mxfp4_blocks_brute_force():
    """Tiny shapes: scales and packed codes from the exact-rational routed sum
    by search, plus the e2m1 error bound and block invariants."""
    inp = gen.make_inputs(dict(T=5, H=64, E=8, ep=2, k=3, hot_row_frac=0.2,
                               hot_scale=64.0, shared_sd=0.5), seed=8)
    pf = bf16_to_f32(inp.payload)
    acc = np.array(_brute.brute_routed_sum(pf, inp.src_info, inp.weights,
                                           bf16_to_f32(inp.shared)), np.float64)
    codes, scales = oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared)
    for t in range(inp.T):
        for b in range(inp.H // 32):
            blk = acc[t, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = -127 if amax == 0 else max(-127, _brute.floor_log2(Fraction(amax)) - 2)
            assert scales[t, b] == e + 127
            if amax > 0 and e > -127:
                assert 4 <= amax * 2.0 ** -e < 8
            for i in range(32):
                byte = int(codes[t, (32 * b + i) // 2])
                c = (byte >> 4) if i % 2 else (byte & 0xF)
                q = blk[i] * 2.0 ** -e
                assert c == nearest_e2m1(q), (t, b, i, q)


# ------------------------------------------------- dense / local reduce

def _dense_case(seed, n_in=6, T=20, H=256):
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((n_in, T, H)))
    sc = rng.random((T, n_in)).astype(np.float32)
    tok = to_bf16_bits(rng.standard_normal((T, H)) * 0.5)
    res = to_bf16_bits(rng.standard_normal((T, H)))
    gam = to_bf16_bits(1 + 0.1 * rng.standard_normal(H))
    ident = np.stack([np.broadcast_to(np.arange(n_in, dtype=np.int32), (T, n_in)),
                      np.broadcast_to(np.arange(T, dtype=np.int32)[:, None], (T, n_in))], axis=-1)
    return x, sc, tok, res, gam, np.ascontiguousarray(ident)


def test_reduce_dense_equals_combine_with_identity_map():
    """Input i of token t read through the slot map (i, t): the combine's
    pinned definition gives the same bits, with and without scales, token
    input, residual + RMSNorm."""
    x, sc, tok, res, gam, ident = _dense_case(0)
    for s_, t_ in [(sc, tok), (None, None), (sc, None), (None, tok)]:
        np.testing.assert_array_equal(oracle.reduce_dense(x, s_, t_),
                                      oracle.combine(x, ident, s_, t_))
    ro, no = oracle.reduce_dense(x, sc, tok, res, gam, 1e-6, 1.0)
    ro2, no2 = oracle.combine_residual_rmsnorm(x, ident, sc, tok, res, gam, 1e-6, 1.0)
    np.testing.assert_array_equal(ro, ro2)
    np.testing.assert_array_equal(no, no2)


def test_reduce_dense_special_cases():
    x, sc, tok, res, gam, ident = _dense_case(1, n_in=1)
    np.testing.assert_array_equal(oracle.reduce_dense(x), x[0])           # one input
    x4 = np.zeros((4,) + x.shape[1:], np.uint16)
    x4[2] = x[0]
    np.testing.assert_array_equal(oracle.reduce_dense(x4), x[0])          # others zero
    # exact dyadic sums
    rng = np.random.default_rng(2)
    v = rng.integers(-8, 9, size=(5, 7, 64)) / 8.0
    s = (rng.integers(1, 5, size=(7, 5)) / 4.0).astype(np.float32)
    exact = np.einsum("ti,ith->th", s.astype(np.float64), v)
    np.testing.assert_array_equal(oracle.reduce_dense(to_bf16_bits(v), s), to_bf16_bits(exact))


# ------------------------------------------------------------- dispatch

@pytest.mark.parametrize("E,ep,k,cap,drop", [(16, 1, 1, None, 0.0), (32, 4, 4, None, 0.2),
                                              (64, 8, 8, 40, 0.1), (8, 2, 3, 5, 0.0)])
def test_dispatch_matches_generator_slot_map(E, ep, k, cap, drop):
    """The oracle's expert-by-expert placement equals the generator's stable
    argsort construction (two independent statements of the same order)."""
    rng = np.random.default_rng(E + k)
    T, H = 70, 16
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    dropped = rng.random((T, k)) < drop
    src_g, loads = gen.dispatch_slots(topk, dropped, E, ep, cap)
    mtpr = cap if cap else int(loads.max())
    ids = np.where(dropped, -1, topk).astype(np.int32)
    x = to_bf16_bits(rng.standard_normal((T, H)))
    payload, src, counts = oracle.dispatch(x, ids, E, ep, mtpr)
    np.testing.assert_array_equal(src, src_g)
    v = src[..., 0] >= 0
    tok = np.broadcast_to(np.arange(T)[:, None], (T, k))
    np.testing.assert_array_equal(payload[src[..., 0][v], src[..., 1][v]], x[tok[v]])
    assert counts.sum() == v.sum()
    np.testing.assert_array_equal(counts, np.bincount(ids[v], minlength=E))
    # rows of each rank are 0..n-1 with no gaps, and never past capacity
    for r in range(ep):
        rows = np.sort(src[..., 1][src[..., 0] == r])
        np.testing.assert_array_equal(rows, np.arange(rows.size))
        assert rows.size <= mtpr


def test_dispatch_then_combine_is_identity_and_counts_accumulate():
    rng = np.random.default_rng(4)
    T, H, E, ep = 90, 32, 12, 3
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    x = to_bf16_bits(rng.standard_normal((T, H)))
    counts = np.zeros(E, np.int32)
    fill = np.full((ep, 64, H), 0x7FC0, np.uint16)
    payload, src, counts = oracle.dispatch(x, ids, E, ep, 64, payload=fill, recv_counts=counts)
    np.testing.assert_array_equal(oracle.combine(payload, src, None), x)
    _, _, counts2 = oracle.dispatch(x, ids, E, ep, 64, recv_counts=counts.copy())
    np.testing.assert_array_equal(counts2, 2 * counts)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(x, np.full((T, 1), E, np.int32), E, ep, 64)


# ------------------------------------------------- non-finite values
#
# The pages fix the bf16 output and the MX formats but say nothing of NaN or
# infinity; the reading taken (a NaN or inf block gets the UE8M0 NaN byte
# 0xFF, its codes taken at e = 0; bf16 rounding keeps NaN a NaN and rounds
# past the largest finite value to infinity) is pinned here against
# hand-worked fixtures and torch's CPU bf16 cast. The sign and payload of a
# NaN result are not fixed (IEEE 754 leaves them open), so NaN outputs are
# compared as "is a NaN" only.

_REP = re.compile(r"\{([^}]*)\}\*(\d+)")


def _fnum(tok):
    t = tok.strip()
    if t in ("inf", "+inf"):
        return math.inf
    if t == "-inf":
        return -math.inf
    return _num(t)


def load_nonfinite(name):
    """Parser of the non-finite fixtures (grammar stated in their headers)."""
    fx = {"rows": [], "rowfill": {}, "slots": {}, "expect": {}, "residual": [],
          "residualfill": {}, "expect_residual": {}, "cases": [],
          "mx8_scales": {}, "mx8_codes": {}, "mx4_scales": {}, "mx4_codes": {}}
    cur = fx
    for raw in open(os.path.join(GOLDEN, name)):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        head, _, body = line.partition(":")
        hs = head.split()
        at = 0
        if len(hs) > 1 and hs[-1].startswith("@"):
            at, hs = int(hs[-1][1:]), hs[:-1]
        toks = _REP.sub(lambda m: " ".join([m.group(1)] * int(m.group(2))), body).split()
        key = hs[0]
        if key == "dims":
            fx["dims"] = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in hs[1:]}
        elif key == "case":
            cur = {"name": hs[1], "expect_norm": {}, "mx8_scales": {}, "mx8_codes": {}}
            for kv in hs[2:]:
                cur[kv.split("=")[0]] = float(kv.split("=")[1])
            fx["cases"].append(cur)
        elif key == "row":
            fx["rows"].append(((int(hs[1]), int(hs[2])), at, [_fnum(v) for v in toks]))
        elif key == "rowfill":
            fx["rowfill"][(int(hs[1]), int(hs[2]))] = _fnum(toks[0])
        elif key == "slot":
            fx["slots"][(int(hs[1]), int(hs[2]))] = (int(toks[0]), int(toks[1]), _fnum(toks[2]))
        elif key == "residual":
            fx["residual"].append((int(hs[1]), at, [_fnum(v) for v in toks]))
        elif key == "residualfill":
            fx["residualfill"][int(hs[1])] = _fnum(toks[0])
        elif key == "gamma":
            fx["gamma"] = [_fnum(v) for v in toks]
        elif key in ("expect", "expect_residual", "expect_norm"):
            tgt = cur if key == "expect_norm" else fx
            tgt[key].setdefault(int(hs[1]), []).append((at, [_fnum(v) for v in toks]))
        elif key in ("mx8_scales", "mx4_scales"):
            cur[key][int(hs[1])] = [int(v) for v in toks]
        elif key in ("mx8_codes", "mx4_codes"):
            cur[key].setdefault(int(hs[1]), []).append((at, toks))
        else:
            raise ValueError(raw)
    return fx


def _exact_bf16(vals):
    """bf16 bits of hand values that bf16 must hold exactly (NaN aside)."""
    v = np.asarray(vals, dtype=np.float64)
    b = to_bf16_bits(v)
    fin = ~np.isnan(v)
    np.testing.assert_array_equal(bf16_to_f32(b)[fin].astype(np.float64), v[fin],
                                  err_msg="fixture value not exact in bf16")
    return b


def _placed(entries, n, fill=0.0):
    """Row of n values from (offset, values) pieces over a fill value."""
    row = np.full(n, fill, dtype=np.float64)
    for at, vals in entries:
        row[at:at + len(vals)] = vals
    return row


def nonfinite_arrays(fx):
    """payload bf16 bits, src_info, weights (and residual, gamma if given)."""
    d = fx["dims"]
    pay = np.zeros((d["ep"], d["mtpr"], d["H"]), np.float64)
    for (r, i), v in fx["rowfill"].items():
        pay[r, i] = v
    for (r, i), at, vals in fx["rows"]:
        pay[r, i, at:at + len(vals)] = vals
    payload = _exact_bf16(pay.reshape(-1)).reshape(pay.shape)
    src = np.full((d["T"], d["k"], 2), -1, np.int32)
    w = np.zeros((d["T"], d["k"]), np.float32)
    for (t, j), (r, row, wj) in fx["slots"].items():
        src[t, j] = (r, row)
        w[t, j] = np.float32(wj)
        assert float(w[t, j]) == wj, "weight not exact in fp32"
    res = gam = None
    if fx["residualfill"] or fx["residual"]:
        res = np.zeros((d["T"], d["H"]), np.float64)
        for t, v in fx["residualfill"].items():
            res[t] = v
        for t, at, vals in fx["residual"]:
            res[t, at:at + len(vals)] = vals
        res = _exact_bf16(res.reshape(-1)).reshape(res.shape)
        gam = _exact_bf16(fx["gamma"])
    return payload, src, w, res, gam


def assert_bf16_expect(got, entries, H, what):
    """Exact bits where a number is expected (signed zeros included), any NaN
    where "nan" is expected."""
    exp = _placed(entries, H)
    nan = np.isnan(exp)
    got_nan = (got & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal(got_nan, nan, err_msg=f"{what}: NaN positions")
    np.testing.assert_array_equal(got[~nan], to_bf16_bits(exp[~nan]), err_msg=what)


def assert_codes_expect(got, entries, n, width, what):
    """e4m3 bytes (width 8) or e2m1 nibbles (width 4); "nn" / "n" accept the
    NaN-block code 0x7F / 7 with either sign; unset entries expect code 0."""
    exp = ["0"] * n
    for at, toks in entries:
        exp[at:at + len(toks)] = toks
    mag = 0x7F if width == 8 else 0x7
    for i, (g, e) in enumerate(zip(got, exp)):
        if e.strip("n") == "":
            assert int(g) & mag == mag, f"{what}[{i}]: {int(g):#x}, expected a NaN code"
        else:
            assert int(g) == int(e, 16), f"{what}[{i}]: {int(g):#x} != {e}"


def _unpack_e2m1(packed):
    p = packed.astype(np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[0], -1)


def test_golden_nonfinite_combine():
    """NaN / +-inf blocks of the MX outputs take byte 0xFF and codes at e = 0;
    bf16 keeps NaN, rounds the halfway point above the largest bf16 to inf
    and the point just below it to 0x7F7F."""
    fx = load_nonfinite("nonfinite_combine_small.txt")
    d = fx["dims"]
    payload, src, w, _, _ = nonfinite_arrays(fx)
    out = oracle.combine(payload, src, w)
    c8, s8 = oracle.combine_mxfp8(payload, src, w)
    c4, s4 = oracle.combine_mxfp4(payload, src, w)
    n4 = _unpack_e2m1(c4)
    for t in range(d["T"]):
        assert_bf16_expect(out[t], fx["expect"].get(t, []), d["H"], f"bf16 token {t}")
        assert list(s8[t]) == fx["mx8_scales"][t], f"mxfp8 scales token {t}"
        assert_codes_expect(c8[t], fx["mx8_codes"].get(t, []), d["H"], 8, f"e4m3 token {t}")
        assert list(s4[t]) == fx["mx4_scales"][t], f"mxfp4 scales token {t}"
        assert_codes_expect(n4[t], fx["mx4_codes"].get(t, []), d["H"], 4, f"e2m1 token {t}")


def test_golden_nonfinite_rmsnorm():
    """NaN and inf in the residual: IEEE propagation through the statistic
    (NaN row; inf -> rstd = +0, signed zeros, inf * 0 = NaN), and the MXFP8
    copy of the normalised row follows the NaN-block rule."""
    fx = load_nonfinite("nonfinite_rmsnorm_small.txt")
    d = fx["dims"]
    payload, src, w, res, gam = nonfinite_arrays(fx)
    assert [c["name"] for c in fx["cases"]] == ["wb0", "wb1"]
    for case in fx["cases"]:
        eps, wb = case["eps"], case["weight_bias"]
        ro, no = oracle.combine_residual_rmsnorm(payload, src, w, None, res, gam, eps, wb)
        ro2, no2, codes, scales = oracle.combine_residual_rmsnorm_mxfp8(
            payload, src, w, None, res, gam, eps, wb)
        for t in range(d["T"]):
            for got in (ro[t], ro2[t]):
                assert_bf16_expect(got, fx["expect_residual"][t], d["H"], f"residual_out {t}")
            for got in (no[t], no2[t]):
                assert_bf16_expect(got, case["expect_norm"][t], d["H"],
                                   f"norm_out {case['name']} token {t}")
            assert list(scales[t]) == case["mx8_scales"][t], f"scales {case['name']} {t}"
            assert_codes_expect(codes[t], case["mx8_codes"][t], d["H"], 8,
                                f"codes {case['name']} {t}")


def test_bf16_rounding_matches_torch_including_nonfinite():
    """oracle_bf16_rne against torch's CPU float -> bfloat16 cast (round to
    nearest even) on every bf16 value with the low half at the rounding
    boundaries, the fp32 extremes and random fp32 patterns: identical bits
    for every non-NaN input (inf, overflow to inf, subnormals, signed zeros);
    a quiet NaN for every NaN input."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    rng = np.random.default_rng(31)
    bits = np.concatenate([(hi[:, None] | lows[None, :]).reshape(-1),
                           rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32),
                           np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000,
                                     0x7F800000, 0xFF800000, 0x00000001, 0x80000001,
                                     0x00FF8000, 0x7FC00000, 0xFFC00000, 0x7F800001],
                                    np.uint32)])
    f = bits.view(np.float32)
    got = np.array([oracle.bf16_rne(float(v)) for v in f], dtype=np.uint16)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert ((got[nan] & 0x7FC0) == 0x7FC0).all(), "NaN must stay a quiet NaN"
    # the cases the fixtures work by hand, by value
    assert oracle.bf16_rne(float(np.uint32(0x7F7F8000).view(np.float32))) == 0x7F80
    assert oracle.bf16_rne(float(np.uint32(0x7F7F7FFF).view(np.float32))) == 0x7F7F
    assert oracle.bf16_rne(math.inf) == 0x7F80 and oracle.bf16_rne(-math.inf) == 0xFF80


def test_reduce_dense_nonfinite_equals_combine_with_identity_map():
    """NaN, +-inf and values near the bf16 limit in the inputs, the token
    input and the residual: the local reduce gives the bits of the pinned
    combine through the identity slot map."""
    x, sc, tok, res, gam, ident = _dense_case(3)
    rng = np.random.default_rng(4)
    special = to_bf16_bits([np.nan, np.inf, -np.inf, 3.3e38, -3.3e38])
    for arr in (x.reshape(-1), tok.reshape(-1), res.reshape(-1)):
        pos = rng.choice(arr.size, size=max(4, arr.size // 200), replace=False)
        arr[pos] = special[rng.integers(0, special.size, pos.size)]
    for s_, t_ in [(sc, tok), (None, None), (None, tok)]:
        np.testing.assert_array_equal(oracle.reduce_dense(x, s_, t_),
                                      oracle.combine(x, ident, s_, t_))
    for wb in (0.0, 1.0):
        ro, no = oracle.reduce_dense(x, sc, tok, res, gam, 1e-6, wb)
        ro2, no2 = oracle.combine_residual_rmsnorm(x, ident, sc, tok, res, gam, 1e-6, wb)
        np.testing.assert_array_equal(ro, ro2)
        np.testing.assert_array_equal(no, no2)
