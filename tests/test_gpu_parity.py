"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance, per output:
  * bf16 outputs (combine, residual_out, norm_out): at most one bf16 step
    apart on the monotone integer line, NaN only where the oracle has NaN.
    The combine and residual_out take the same fp32 operations in the same
    order as the oracle, and norm_out is evaluated in fp64 on both sides
    (only the summation order of the statistic differs), so all of them are
    also required to be identical on all but 0.1% of elements.
  * MXFP8 scales: bit-exact.
  * e4m3 codes: at most one code step apart, on at most 0.1% of elements.
Outputs are poisoned first, so every element the kernel should write is
checked, and rows past num_tokens must keep the poison.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import gen
import oracle
import moe_expert_combine_amd as mc
from tests.test_oracle_pins import (_unpack_e2m1, assert_bf16_expect, assert_codes_expect,
                                    load_fixture, load_nonfinite, nonfinite_arrays,
                                    to_bf16_bits, ulp_dist_bf16)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
POISON16 = 0xFFFF      # a NaN pattern the kernels never produce from finite data
POISON8 = 0xEE


def dev16(a):
    """uint16 numpy bits -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def host16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(inp):
    d = dict(payload=dev16(inp.payload),
             src_info=torch.from_numpy(inp.src_info).to(DEV),
             weights=None if inp.weights is None else torch.from_numpy(inp.weights).to(DEV),
             shared=None if inp.shared is None else dev16(inp.shared))
    if inp.residual is not None:
        d["residual"] = dev16(inp.residual)
        d["gamma"] = dev16(inp.gamma)
    return d


def poisoned16(T, H, extra=0):
    return torch.full((T + extra, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def check_bf16(got, ref, exact_frac, what):
    d = ulp_dist_bf16(got, ref)
    assert d.max() <= 1, f"{what}: max ulp distance {d.max()}"
    frac = (d != 0).mean() if d.size else 0.0
    assert frac <= exact_frac, f"{what}: {frac:.2e} of elements differ by one step"


def e4m3_step_dist(a, b):
    """Distance in e4m3 code steps on the monotone line (NaN codes excluded)."""
    def key(c):
        c = c.astype(np.int32)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return np.abs(key(a) - key(b))


def check_mxfp8(codes, scales, rc, rs, what):
    np.testing.assert_array_equal(scales, rs, err_msg=f"{what}: scales")
    nan_g = (codes & 0x7F) == 0x7F
    nan_r = (rc & 0x7F) == 0x7F
    np.testing.assert_array_equal(nan_g, nan_r, err_msg=f"{what}: NaN codes")
    d = e4m3_step_dist(codes[~nan_g], rc[~nan_g])
    assert d.max(initial=0) <= 1, f"{what}: code distance {d.max()}"
    assert (d != 0).mean() <= 1e-3 if d.size else True, f"{what}: too many off-by-one codes"


# ----------------------------------------------------------------- runners

def run_combine(inp, extra_rows=0, d=None):
    d = d or to_dev(inp)
    out = poisoned16(inp.T, inp.H, extra_rows)
    mc.moe_combine(d["payload"], d["src_info"], d["weights"], d["shared"], out=out)
    torch.cuda.synchronize()
    o = host16(out)
    if extra_rows:
        assert (o[inp.T:] == POISON16).all(), "rows past num_tokens were written"
    return o[:inp.T]


def run_rmsnorm(inp, wb, extra_rows=0, in_place=False, d=None):
    d = d or to_dev(inp)
    norm = poisoned16(inp.T, inp.H, extra_rows)
    if in_place:
        ro = torch.cat([d["residual"], poisoned16(0, inp.H, extra_rows)]) if extra_rows else d["residual"]
        res_in = ro
    else:
        ro = poisoned16(inp.T, inp.H, extra_rows)
        res_in = d["residual"]
    mc.moe_combine_residual_rmsnorm(d["payload"], d["src_info"], d["weights"], d["shared"],
                                    res_in, d["gamma"], inp.eps, wb,
                                    residual_out=ro, norm_out=norm)
    torch.cuda.synchronize()
    a, b = host16(ro), host16(norm)
    if extra_rows:
        assert (a[inp.T:] == POISON16).all() and (b[inp.T:] == POISON16).all()
    return a[:inp.T], b[:inp.T]


def run_mxfp8(inp, extra_rows=0, d=None):
    d = d or to_dev(inp)
    T, H = inp.T, inp.H
    codes = torch.full((T + extra_rows, H), POISON8, dtype=torch.uint8, device=DEV)
    scales = torch.full((T + extra_rows, H // 32), POISON8, dtype=torch.uint8, device=DEV)
    mc.moe_combine_mxfp8(d["payload"], d["src_info"], d["weights"], d["shared"],
                         out_fp8=codes.view(torch.float8_e4m3fn), out_scales=scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    if extra_rows:
        assert (c[T:] == POISON8).all() and (s[T:] == POISON8).all()
    return c[:T], s[:T]


def run_rmsnorm_mxfp8(inp, wb, extra_rows=0, want_norm=True, d=None):
    d = d or to_dev(inp)
    T, H = inp.T, inp.H
    ro = poisoned16(T, H, extra_rows)
    no = poisoned16(T, H, extra_rows) if want_norm else None
    codes = torch.full((T + extra_rows, H), POISON8, dtype=torch.uint8, device=DEV)
    scales = torch.full((T + extra_rows, H // 32), POISON8, dtype=torch.uint8, device=DEV)
    mc.moe_combine_residual_rmsnorm_mxfp8(d["payload"], d["src_info"], d["weights"], d["shared"],
                                          d["residual"], d["gamma"], inp.eps, wb,
                                          residual_out=ro, out_fp8=codes.view(torch.float8_e4m3fn),
                                          out_scales=scales, norm_out=no)
    torch.cuda.synchronize()
    a, c, sc = host16(ro), codes.cpu().numpy(), scales.cpu().numpy()
    b = host16(no) if want_norm else None
    if extra_rows:
        assert (a[T:] == POISON16).all() and (c[T:] == POISON8).all() and (sc[T:] == POISON8).all()
        if want_norm:
            assert (b[T:] == POISON16).all()
    return a[:T], (b[:T] if want_norm else None), c[:T], sc[:T]


def check_rmsnorm_mxfp8(inp, wb, extra_rows=0, want_norm=True, what="", ref=None, d=None):
    ro, no, c, sc = run_rmsnorm_mxfp8(inp, wb, extra_rows, want_norm, d)
    ref = inp if ref is None else ref
    rro, rno, rc, rs = oracle.combine_residual_rmsnorm_mxfp8(
        ref.payload, ref.src_info, ref.weights, ref.shared, ref.residual, ref.gamma, ref.eps, wb)
    check_bf16(ro, rro, 1e-3, f"{what} residual_out (rmsnorm+mxfp8) wb={wb}")
    if want_norm:
        check_bf16(no, rno, 1e-3, f"{what} norm_out (rmsnorm+mxfp8) wb={wb}")
    check_mxfp8(c, sc, rc, rs, f"{what} mxfp8 of norm wb={wb}")


def run_mxfp4(inp, extra_rows=0, d=None):
    d = d or to_dev(inp)
    T, H = inp.T, inp.H
    codes = torch.full((T + extra_rows, H // 2), POISON8, dtype=torch.uint8, device=DEV)
    scales = torch.full((T + extra_rows, H // 32), POISON8, dtype=torch.uint8, device=DEV)
    mc.moe_combine_mxfp4(d["payload"], d["src_info"], d["weights"], d["shared"],
                         out_fp4=codes, out_scales=scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    if extra_rows:
        assert (c[T:] == POISON8).all() and (s[T:] == POISON8).all()
    return c[:T], s[:T]


def check_mxfp4(codes, scales, rc, rs, what):
    """Scales bit-exact; e2m1 codes (unpacked) within one step on <= 0.1%."""
    np.testing.assert_array_equal(scales, rs, err_msg=f"{what}: scales")

    def unpack(b):
        b = b.astype(np.int32)
        c = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[0], -1)
        return np.where(c & 0x8, -(c & 0x7), c & 0x7)
    d = np.abs(unpack(codes) - unpack(rc))
    assert d.max(initial=0) <= 1, f"{what}: e2m1 code distance {d.max()}"
    assert (d != 0).mean() <= 1e-3, f"{what}: too many off-by-one e2m1 codes"


def oracle_all(inp, kind, wb=0.0):
    if kind == "bf16":
        return oracle.combine(inp.payload, inp.src_info, inp.weights, inp.shared)
    if kind == "rmsnorm":
        return oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                               inp.shared, inp.residual, inp.gamma,
                                               inp.eps, wb)
    return oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights, inp.shared)


def check_all_kinds(inp, wbs=(0.0, 1.0), extra_rows=3, what="", ref=None, d=None):
    """Every output kind of the HIP path on inp against the oracle on ref
    (default: the same inputs). d: device tensors for inp, if prebuilt."""
    ref = inp if ref is None else ref
    check_bf16(run_combine(inp, extra_rows, d), oracle_all(ref, "bf16"), 1e-3, f"{what} combine")
    if inp.residual is not None:
        for wb in wbs:
            ro, no = run_rmsnorm(inp, wb, extra_rows, d=d)
            rro, rno = oracle_all(ref, "rmsnorm", wb)
            check_bf16(ro, rro, 1e-3, f"{what} residual_out wb={wb}")
            check_bf16(no, rno, 1e-3, f"{what} norm_out wb={wb}")
    if inp.H % 32 == 0:
        c, s = run_mxfp8(inp, extra_rows, d)
        rc, rs = oracle_all(ref, "mxfp8")
        check_mxfp8(c, s, rc, rs, f"{what} mxfp8")
        c4, s4 = run_mxfp4(inp, extra_rows, d)
        rc4, rs4 = oracle.combine_mxfp4(ref.payload, ref.src_info, ref.weights, ref.shared)
        check_mxfp4(c4, s4, rc4, rs4, f"{what} mxfp4")
        if inp.residual is not None:
            for i, wb in enumerate(wbs):
                check_rmsnorm_mxfp8(inp, wb, extra_rows, want_norm=(i == 0), what=what, ref=ref, d=d)


def with_norm_inputs(c):
    c = dict(c)
    c.setdefault("residual_sd", 1.0)
    c.setdefault("gamma_sd", 0.1)
    return c


# --------------------------------------------------------------- fixtures

def test_golden_fixtures_on_gpu():
    """The hand-worked examples, through the HIP path."""
    fx = load_fixture("combine_small.txt")
    dd = fx["dims"]
    payload = np.zeros((dd["ep"], dd["mtpr"], dd["H"]), np.uint16)
    for (r, row), vals in fx["rows"].items():
        payload[r, row] = to_bf16_bits(vals)
    src = np.full((dd["T"], dd["k"], 2), -1, np.int32)
    w = np.zeros((dd["T"], dd["k"]), np.float32)
    for (t, j), (r, row, wj) in fx["slots"].items():
        src[t, j] = (r, row)
        w[t, j] = wj
    out = mc.moe_combine(dev16(payload), torch.from_numpy(src).to(DEV),
                         torch.from_numpy(w).to(DEV))
    o = host16(out)
    for t, vals in fx["expect"].items():
        np.testing.assert_array_equal(o[t], to_bf16_bits(vals))

    fx = load_fixture("rmsnorm_small.txt")
    payload = np.zeros((1, 1, 8), np.uint16)
    payload[0, 0] = to_bf16_bits(fx["rows"][(0, 0)])
    src = torch.zeros((1, 1, 2), dtype=torch.int32, device=DEV)
    w = torch.ones((1, 1), dtype=torch.float32, device=DEV)
    res = dev16(to_bf16_bits(fx["residual"][0])[None])
    g = dev16(to_bf16_bits(fx["gamma"]))
    for case in fx["cases"]:
        ro, no = mc.moe_combine_residual_rmsnorm(dev16(payload), src, w, None, res, g,
                                                 case["eps"], case["weight_bias"])
        np.testing.assert_array_equal(host16(ro)[0], to_bf16_bits(fx["expect_residual"][0]))
        np.testing.assert_array_equal(host16(no)[0], to_bf16_bits(case["norm"][0]),
                                      err_msg=case["name"])

    fx = load_fixture("mxfp8_small.txt")
    x0 = np.array(fx["x"][0], dtype=np.float32)
    payload = np.stack([to_bf16_bits(x0), to_bf16_bits(-x0)])[None]
    src = torch.tensor([[[0, 0]], [[0, 1]]], dtype=torch.int32, device=DEV)
    w = torch.ones((2, 1), dtype=torch.float32, device=DEV)
    codes, scales = mc.moe_combine_mxfp8(dev16(payload), src, w)
    codes = codes.view(torch.uint8).cpu().numpy()
    scales = scales.cpu().numpy()
    for t in range(2):
        assert list(scales[t]) == fx["scales"][t]
        assert list(codes[t]) == fx["codes"][t]


def test_golden_mxfp4_on_gpu():
    fx = load_fixture("mxfp4_small.txt")
    x0 = np.array(fx["x"][0], dtype=np.float32)
    src = torch.zeros((1, 1, 2), dtype=torch.int32, device=DEV)
    w = torch.ones((1, 1), dtype=torch.float32, device=DEV)
    codes, scales = mc.moe_combine_mxfp4(dev16(to_bf16_bits(x0)[None, None]), src, w)
    assert list(scales.cpu().numpy()[0]) == fx["scales"][0]
    assert list(codes.cpu().numpy()[0]) == fx["codes"][0]


def test_golden_rmsnorm_mxfp8_on_gpu():
    fx = load_fixture("rmsnorm_mxfp8_small.txt")
    payload = np.zeros((1, 1, 32), np.uint16)
    payload[0, 0] = to_bf16_bits(fx["rows"][(0, 0)])
    src = torch.zeros((1, 1, 2), dtype=torch.int32, device=DEV)
    w = torch.ones((1, 1), dtype=torch.float32, device=DEV)
    res = dev16(to_bf16_bits(fx["residual"][0])[None])
    g = dev16(to_bf16_bits(fx["gamma"]))
    for case in fx["cases"]:
        ro, codes, scales, _ = mc.moe_combine_residual_rmsnorm_mxfp8(
            dev16(payload), src, w, None, res, g, case["eps"], case["weight_bias"])
        np.testing.assert_array_equal(host16(ro)[0], to_bf16_bits([2, -2] * 16))
        assert list(scales.cpu().numpy()[0]) == case["scale"][0], case["name"]
        assert list(codes.view(torch.uint8).cpu().numpy()[0]) == case["codes"][0], case["name"]


def test_golden_nonfinite_on_gpu():
    """The hand-worked non-finite fixtures through the HIP path: NaN / +-inf
    blocks (byte 0xFF, codes at e = 0), bf16 overflow at the halfway point,
    NaN and inf in the residual through both RMSNorm epilogues."""
    fx = load_nonfinite("nonfinite_combine_small.txt")
    d = fx["dims"]
    payload, src, w, _, _ = nonfinite_arrays(fx)
    p, s, wt = dev16(payload), torch.from_numpy(src).to(DEV), torch.from_numpy(w).to(DEV)
    out = host16(mc.moe_combine(p, s, wt))
    c8, s8 = mc.moe_combine_mxfp8(p, s, wt)
    c8, s8 = c8.view(torch.uint8).cpu().numpy(), s8.cpu().numpy()
    c4, s4 = mc.moe_combine_mxfp4(p, s, wt)
    n4, s4 = _unpack_e2m1(c4.cpu().numpy()), s4.cpu().numpy()
    for t in range(d["T"]):
        assert_bf16_expect(out[t], fx["expect"].get(t, []), d["H"], f"bf16 token {t}")
        assert list(s8[t]) == fx["mx8_scales"][t], f"mxfp8 scales token {t}"
        assert_codes_expect(c8[t], fx["mx8_codes"].get(t, []), d["H"], 8, f"e4m3 token {t}")
        assert list(s4[t]) == fx["mx4_scales"][t], f"mxfp4 scales token {t}"
        assert_codes_expect(n4[t], fx["mx4_codes"].get(t, []), d["H"], 4, f"e2m1 token {t}")

    fx = load_nonfinite("nonfinite_rmsnorm_small.txt")
    d = fx["dims"]
    payload, src, w, res, gam = nonfinite_arrays(fx)
    p, s, wt = dev16(payload), torch.from_numpy(src).to(DEV), torch.from_numpy(w).to(DEV)
    r, g = dev16(res), dev16(gam)
    for case in fx["cases"]:
        eps, wb = case["eps"], case["weight_bias"]
        ro, no = mc.moe_combine_residual_rmsnorm(p, s, wt, None, r, g, eps, wb)
        ro2, codes, scales, no2 = mc.moe_combine_residual_rmsnorm_mxfp8(
            p, s, wt, None, r, g, eps, wb, want_norm_out=True)
        ro, no, ro2, no2 = host16(ro), host16(no), host16(ro2), host16(no2)
        codes, scales = codes.view(torch.uint8).cpu().numpy(), scales.cpu().numpy()
        for t in range(d["T"]):
            for got in (ro[t], ro2[t]):
                assert_bf16_expect(got, fx["expect_residual"][t], d["H"], f"residual_out {t}")
            for got in (no[t], no2[t]):
                assert_bf16_expect(got, case["expect_norm"][t], d["H"],
                                   f"norm_out {case['name']} token {t}")
            assert list(scales[t]) == case["mx8_scales"][t], f"scales {case['name']} {t}"
            assert_codes_expect(codes[t], case["mx8_codes"][t], d["H"], 8,
                                f"codes {case['name']} {t}")


def _plant_nonfinite(arr, rows, rng, frac):
    """Write NaN, +-inf and near-limit finite values (bf16 0x7F7F = 3.39e38,
    and its negative) over about frac of the elements of the given rows."""
    special = np.array([0x7FC0, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x7F70], np.uint16)
    flat = arr.reshape(-1, arr.shape[-1])
    n = max(1, int(frac * rows.size * arr.shape[-1]))
    rr = rng.choice(rows, size=n)
    hh = rng.integers(0, arr.shape[-1], size=n)
    flat[rr, hh] = special[rng.integers(0, special.size, size=n)]


def check_mxfp4_nan_aware(codes, scales, rc, rs, nan_elems, what):
    """check_mxfp4, except that elements whose value is NaN may carry either
    sign on the saturated code (e2m1 has no NaN)."""
    np.testing.assert_array_equal(scales, rs, err_msg=f"{what}: scales")
    g, r = _unpack_e2m1(codes), _unpack_e2m1(rc)
    np.testing.assert_array_equal(g[nan_elems] & 7, 7, err_msg=f"{what}: NaN elements")
    np.testing.assert_array_equal(r[nan_elems] & 7, 7)
    key = lambda c: np.where(c & 0x8, -(c.astype(np.int32) & 0x7), c.astype(np.int32) & 0x7)
    dd = np.abs(key(g) - key(r))[~nan_elems]
    assert dd.max(initial=0) <= 1 and (dd != 0).mean() <= 1e-3, f"{what}: e2m1 codes"


@pytest.mark.parametrize("seed", [0, 1])
def test_nonfinite_values_in_occupied_rows(seed):
    """NaN, +-inf and values at the bf16 limit in payload rows that are read,
    in the shared-expert rows and in the residual: every combine epilogue
    (bf16, residual + RMSNorm with weight_bias 0 and 1, MXFP8, RMSNorm +
    MXFP8, MXFP4) against the oracle, NaN matching NaN."""
    c = with_norm_inputs(dict(T=96, H=1024, E=32, ep=4, k=8, shared_sd=0.5, drop_frac=0.1))
    inp = gen.make_inputs(c, seed=seed)
    rng = np.random.default_rng(100 + seed)
    kept = inp.src_info[..., 0] >= 0
    occ = (inp.src_info[..., 0] * inp.mtpr + inp.src_info[..., 1])[kept]
    _plant_nonfinite(inp.payload, np.unique(occ), rng, 2e-4)
    _plant_nonfinite(inp.shared, np.arange(inp.T), rng, 1e-4)
    _plant_nonfinite(inp.residual, rng.choice(inp.T, inp.T // 8, replace=False), rng, 2e-4)
    acc = oracle.routed_sum_f32(inp.payload, inp.src_info, inp.weights, inp.shared)
    assert np.isnan(acc).any() and np.isinf(acc).any()
    check_bf16(run_combine(inp, 2), oracle_all(inp, "bf16"), 1e-3, "nonfinite combine")
    for wb in (0.0, 1.0):
        ro, no = run_rmsnorm(inp, wb, 2)
        rro, rno = oracle_all(inp, "rmsnorm", wb)
        check_bf16(ro, rro, 1e-3, f"nonfinite residual_out wb={wb}")
        check_bf16(no, rno, 1e-3, f"nonfinite norm_out wb={wb}")
        check_rmsnorm_mxfp8(inp, wb, 2, want_norm=True, what="nonfinite")
    cc, ss = run_mxfp8(inp, 2)
    rc, rs = oracle_all(inp, "mxfp8")
    check_mxfp8(cc, ss, rc, rs, "nonfinite mxfp8")
    assert (ss == 0xFF).any()
    c4, s4 = run_mxfp4(inp, 2)
    rc4, rs4 = oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared)
    check_mxfp4_nan_aware(c4, s4, rc4, rs4, np.isnan(acc), "nonfinite mxfp4")


def test_nonfinite_values_in_local_reduce():
    """The dense local reduce and its residual + RMSNorm form with NaN, +-inf
    and limit values in the inputs, the token input and the residual."""
    d = gen.make_dense_inputs(dict(n_in=8, T=64, H=2048, scales=True, token_sd=0.5,
                                   residual_sd=1.0), seed=3)
    rng = np.random.default_rng(7)
    _plant_nonfinite(d.x, np.arange(d.x.shape[0] * d.x.shape[1]), rng, 1e-4)
    _plant_nonfinite(d.tok, np.arange(d.T), rng, 1e-4)
    _plant_nonfinite(d.residual, rng.choice(d.T, 8, replace=False), rng, 3e-4)
    x, sc, tk = dev16(d.x), torch.from_numpy(d.scales).to(DEV), dev16(d.tok)
    ref = oracle.reduce_dense(d.x, d.scales, d.tok)
    assert ((ref & 0x7FFF) > 0x7F80).any()
    check_bf16(host16(mc.moe_reduce_dense(x, sc, tk)), ref, 1e-3, "nonfinite reduce_dense")
    for wb in (0.0, 1.0):
        ro, no = mc.moe_reduce_dense_residual_rmsnorm(x, sc, tk, dev16(d.residual),
                                                      dev16(d.gamma), d.eps, wb)
        rro, rno = oracle.reduce_dense(d.x, d.scales, d.tok, d.residual, d.gamma, d.eps, wb)
        check_bf16(host16(ro), rro, 1e-3, f"nonfinite reduce residual_out wb={wb}")
        check_bf16(host16(no), rno, 1e-3, f"nonfinite reduce norm_out wb={wb}")


# ------------------------------------------------------------ small shapes

def test_tiny_config_all_outputs():
    check_all_kinds(gen.make_inputs(with_norm_inputs(gen.CONFIGS["tiny"]), 0), what="tiny")


@pytest.mark.parametrize("T,H,k,ep,extra", [
    (1, 8, 1, 1, {}),                       # one vector, one slot
    (7, 264, 3, 2, {}),                     # ragged hidden (33 vectors), odd top_k
    (33, 1032, 5, 3, dict(drop_frac=0.3)),  # ragged tail past one chunk, drops
    (65, 4096, 8, 8, dict(shared_sd=0.5)),  # shared expert, exact tiles
    (17, 7168, 8, 8, dict(drop_frac=0.5, shared_sd=0.5)),
    (9, 2048, 13, 4, {}),                   # top_k > 8: two slot groups
    (5, 512, 32, 8, dict(drop_frac=0.2)),   # maximum top_k
    (40, 96, 2, 1, dict(weights=False)),    # unit weights (no router weights)
    (3, 30000, 8, 8, {}),                   # wide row: RMSNorm with 8 vectors/lane
    (2, 32768, 4, 2, dict(shared_sd=0.5)),  # widest RMSNorm row supported
])
def test_ragged_and_edge_shapes(T, H, k, ep, extra):
    c = with_norm_inputs(dict(T=T, H=H, E=max(k, 8) * ep, ep=ep, k=k, **extra))
    check_all_kinds(gen.make_inputs(c, seed=T), what=f"T={T} H={H} k={k}")


def _random_combine_case(i):
    """Seeded random shape: top_k, ranks, experts, hidden (multiples of 8,
    ragged or not), drops, routing law, shared expert and unit weights."""
    rng = np.random.default_rng(7000 + i)
    k = int(rng.choice([1, 2, 3, 4, 6, 8, 13, 16, 32]))
    ep = int(rng.choice([1, 2, 3, 4, 8]))
    E = ep * max(-(-k // ep), int(rng.integers(1, 9)))
    c = dict(T=int(rng.integers(1, 80)), k=k, ep=ep, E=E,
             H=int(rng.choice([8, 32, 96, 264, 520, 1000, 1024, 2056, 4096, 7168])),
             drop_frac=float(rng.choice([0.0, 0.0, 0.1, 0.5])),
             weights=bool(rng.random() < 0.8),
             routing="zipf" if rng.random() < 0.3 else "uniform")
    if rng.random() < 0.4:
        c["shared_sd"] = 0.5
    return with_norm_inputs(c)


@pytest.mark.parametrize("i", range(24))
def test_random_shapes_every_output(i):
    c = _random_combine_case(i)
    check_all_kinds(gen.make_inputs(c, seed=i), what=f"random case {i}: {c}")


def test_mx_outputs_at_minimum_alignment():
    """Code and scale arrays only as aligned as the entry points require
    (e4m3 8 bytes, e2m1 4 bytes, scales 1 byte): the wider paired stores
    must not be taken, and every byte must still match the oracle."""
    inp = gen.make_inputs(with_norm_inputs(dict(T=40, H=2048, E=64, ep=8, k=8, shared_sd=0.5)), 3)
    d = to_dev(inp)
    T, H = inp.T, inp.H
    big = torch.full((T * H + 64,), POISON8, dtype=torch.uint8, device=DEV)
    sbig = torch.full((T * (H // 32) + 64,), POISON8, dtype=torch.uint8, device=DEV)
    codes = big[8:8 + T * H].view(T, H)                       # 8-byte aligned only
    scales = sbig[1:1 + T * (H // 32)].view(T, H // 32)       # 1-byte aligned
    mc.moe_combine_mxfp8(d["payload"], d["src_info"], d["weights"], d["shared"],
                         out_fp8=codes.view(torch.float8_e4m3fn), out_scales=scales)
    rc, rs = oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights, inp.shared)
    check_mxfp8(codes.cpu().numpy(), scales.cpu().numpy(), rc, rs, "mxfp8 at minimum alignment")
    assert (big[:8].cpu().numpy() == POISON8).all() and (sbig[:1].cpu().numpy() == POISON8).all()

    ro = poisoned16(T, H)
    c2 = big[8:8 + T * H].view(T, H)
    mc.moe_combine_residual_rmsnorm_mxfp8(d["payload"], d["src_info"], d["weights"], d["shared"],
                                          d["residual"], d["gamma"], inp.eps, 1.0, residual_out=ro,
                                          out_fp8=c2.view(torch.float8_e4m3fn), out_scales=scales)
    rro, rno, rc2, rs2 = oracle.combine_residual_rmsnorm_mxfp8(
        inp.payload, inp.src_info, inp.weights, inp.shared, inp.residual, inp.gamma, inp.eps, 1.0)
    check_mxfp8(c2.cpu().numpy(), scales.cpu().numpy(), rc2, rs2, "rmsnorm+mxfp8 at minimum alignment")

    c4 = big[4:4 + T * (H // 2)].view(T, H // 2)              # 4-byte aligned only
    mc.moe_combine_mxfp4(d["payload"], d["src_info"], d["weights"], d["shared"],
                         out_fp4=c4, out_scales=scales)
    rc4, rs4 = oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared)
    check_mxfp4(c4.cpu().numpy(), scales.cpu().numpy(), rc4, rs4, "mxfp4 at minimum alignment")


def test_unoccupied_nan_rows_and_all_dropped_tokens():
    c = with_norm_inputs(dict(T=48, H=1024, E=32, ep=4, k=8, unoccupied="nan",
                              drop_frac=0.4, shared_sd=0.5))
    inp = gen.make_inputs(c, seed=4, mtpr=1024)
    inp.src_info[5] = -1                     # token 5: every slot dropped
    inp.src_info[6] = -1
    inp.shared[6] = 0                        # token 6: dropped, zero shared
    check_all_kinds(inp, what="nan rows")
    out = run_combine(inp)
    assert not ((out & 0x7FFF) > 0x7F80).any()


def test_all_slots_dropped_without_shared_gives_plus_zero():
    inp = gen.make_inputs(dict(T=12, H=256, E=8, ep=2, k=4), seed=1)
    inp.src_info[:] = -1
    assert (run_combine(inp) == 0).all()
    c, s = run_mxfp8(inp)
    assert (c == 0).all() and (s == 0).all()


# ------------------------------------------------ slots outside the payload

def _padded_dev(inp, pad):
    """Device tensors for inp whose payload sits between `pad` ranks of NaN
    rows on each side, in one allocation. A slot outside the payload that the
    kernel failed to drop would read those rows (NaN in the output) or another
    real row (a wrong sum), never memory outside the allocation."""
    d = to_dev(inp)
    ep, mtpr, H = inp.payload.shape
    host = np.full((ep + 2 * pad, mtpr, H), 0x7FC0, np.uint16)
    host[pad:pad + ep] = inp.payload
    d["payload_alloc"] = dev16(host)
    d["payload"] = d["payload_alloc"][pad:pad + ep]
    return d


def _with_slots(inp, pairs, frac, seed):
    """(inputs whose slot map names the (rank, row) pairs on a fraction of the
    kept slots, the same inputs with exactly those slots dropped)."""
    rng = np.random.default_rng(seed)
    bad, clean = inp.src_info.copy(), inp.src_info.copy()
    kept = np.argwhere(inp.src_info[..., 0] >= 0)
    pick = kept[rng.random(len(kept)) < frac]
    assert len(pick) >= len(pairs)
    for n, (t, j) in enumerate(pick):
        bad[t, j] = pairs[n % len(pairs)]
        clean[t, j] = (-1, -1)
    return dataclasses.replace(inp, src_info=bad), dataclasses.replace(inp, src_info=clean)


def test_slots_just_outside_the_payload_are_dropped():
    """A slot whose rank is outside [0, ep_size) or whose row is outside
    [0, max_tokens_per_rank) reads nothing and counts as dropped, on every
    output kind. Here the bad pairs stay within four ranks of the payload, and
    the payload is padded by four NaN ranks on each side."""
    inp = gen.make_inputs(with_norm_inputs(dict(T=41, H=1056, E=32, ep=4, k=8, shared_sd=0.5)), seed=11)
    ep, m = inp.ep, inp.mtpr
    pairs = [(ep, 0), (ep + 1, m - 1), (ep + 3, 7), (0, m), (ep - 1, m + 17), (1, 2 * m + 1),
             (0, -1), (2, -1), (ep - 1, -m), (3, -3 * m), (-5, 3)]
    for r, w in pairs:   # where an unchecked read would land, in rows of the padded allocation
        assert r < 0 or -4 * m <= r * m + w < (ep + 4) * m
    bad, clean = _with_slots(inp, pairs, 0.3, seed=11)
    check_all_kinds(bad, ref=clean, d=_padded_dev(bad, pad=4), what="slots just outside the payload")


def test_slots_far_outside_the_payload_are_dropped():
    """Extreme ranks and rows (2^30, the int32 limits) are dropped too."""
    inp = gen.make_inputs(with_norm_inputs(dict(T=29, H=2048, E=64, ep=8, k=6, shared_sd=0.5)), seed=12)
    i32max, i32min = 2**31 - 1, -2**31
    pairs = [(1 << 30, 0), (i32max, i32max), (0, i32max), (inp.ep - 1, i32min), (3, 1 << 30),
             (i32max, -1), (i32min, 0)]
    bad, clean = _with_slots(inp, pairs, 0.3, seed=12)
    check_all_kinds(bad, ref=clean, what="slots far outside the payload")


def test_zero_tokens_leaves_outputs_untouched():
    inp = gen.make_inputs(dict(T=4, H=64, E=8, ep=1, k=2), seed=0)
    d = to_dev(inp)
    out = poisoned16(0, 64, 3)
    mc.moe_combine(d["payload"], d["src_info"][:0], d["weights"][:0], out=out)
    torch.cuda.synchronize()
    assert (host16(out) == POISON16).all()


def test_in_place_residual_update():
    inp = gen.make_inputs(with_norm_inputs(dict(T=20, H=7168, E=64, ep=8, k=8)), seed=9)
    ro, no = run_rmsnorm(inp, 1.0, in_place=True)
    rro, rno = oracle_all(inp, "rmsnorm", 1.0)
    check_bf16(ro, rro, 1e-3, "in-place residual_out")
    check_bf16(no, rno, 1e-3, "in-place norm_out")


def test_layout_invariance_on_gpu():
    """Same (token, slot) rows under another ep_size / row order: identical."""
    rng = np.random.default_rng(3)
    T, H, E, k = 64, 2048, 32, 8
    rows = to_bf16_bits(rng.standard_normal((T, k, H)).astype(np.float32))
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = torch.from_numpy(rng.random((T, k)).astype(np.float32)).to(DEV)
    outs = []
    for ep in (1, 4, 8):
        src, loads = gen.dispatch_slots(topk, np.zeros((T, k), bool), E, ep, None)
        payload = gen.scatter_rows(src, rows, ep, int(loads.max()) + 3)
        outs.append(host16(mc.moe_combine(dev16(payload), torch.from_numpy(src).to(DEV), w)))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_e4m3_conversion_every_bf16_pattern():
    """All 65536 bf16 patterns as single-slot sums (so acc is exactly each
    pattern), blocks of 32 consecutive patterns: the kernel's integer e4m3 and
    UE8M0 route against the oracle, NaN/inf blocks included."""
    H = 1024
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(64, H)
    rng = np.random.default_rng(0)
    shuffled = rng.permutation(allp.reshape(-1)).reshape(64, H)
    payload = np.concatenate([allp, shuffled])[None]
    T = payload.shape[1]
    src = np.stack([np.zeros(T, np.int32), np.arange(T, dtype=np.int32)], axis=-1)[:, None, :]
    src = np.ascontiguousarray(src)
    w = np.ones((T, 1), np.float32)
    codes, scales = mc.moe_combine_mxfp8(dev16(payload), torch.from_numpy(src).to(DEV),
                                         torch.from_numpy(w).to(DEV))
    codes = codes.view(torch.uint8).cpu().numpy()
    rc, rs = oracle.combine_mxfp8(payload, src, w)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes, rc)


def test_mxfp8_codes_identical_on_fp32_sums():
    """Weighted sums of eight rows have full 24-bit mantissas, so they hit
    e4m3 rounding boundaries the bf16 patterns above cannot; the codes of
    both MXFP8 epilogues must still equal the oracle's exactly."""
    inp = gen.make_inputs(with_norm_inputs(dict(T=512, H=7168, E=256, ep=8, k=8, shared_sd=0.5,
                                                hot_row_frac=0.01, hot_scale=64.0)), 5)
    c, s = run_mxfp8(inp)
    rc, rs = oracle_all(inp, "mxfp8")
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
    _, _, c2, s2 = run_rmsnorm_mxfp8(inp, 1.0, want_norm=False)
    _, _, rc2, rs2 = oracle.combine_residual_rmsnorm_mxfp8(
        inp.payload, inp.src_info, inp.weights, inp.shared, inp.residual, inp.gamma, inp.eps, 1.0)
    np.testing.assert_array_equal(s2, rs2)
    np.testing.assert_array_equal(c2, rc2)


def test_e2m1_conversion_every_bf16_pattern():
    """All 65536 bf16 patterns as single-slot sums through the MXFP4 path."""
    H = 1024
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(64, H)
    rng = np.random.default_rng(1)
    payload = np.concatenate([allp, rng.permutation(allp.reshape(-1)).reshape(64, H)])[None]
    T = payload.shape[1]
    src = np.ascontiguousarray(np.stack([np.zeros(T, np.int32), np.arange(T, dtype=np.int32)],
                                        axis=-1)[:, None, :])
    w = np.ones((T, 1), np.float32)
    codes, scales = mc.moe_combine_mxfp4(dev16(payload), torch.from_numpy(src).to(DEV),
                                         torch.from_numpy(w).to(DEV))
    rc, rs = oracle.combine_mxfp4(payload, src, w)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("tile", ["64x1", "64x2", "64x4", "128x2", "128x4", "256x1", "256x4",
                                  "512x8", "512x4", "1024x1", "448x2", "896x1", "192x8", "1024x2",
                                  "448x2x4", "448x2x2", "64x2x4", "256x4x2"])
def test_every_tile_shape(monkeypatch, tile):
    """Each launch shape the tile override can pick computes the same result."""
    monkeypatch.setenv("MOE_COMBINE_TILE", tile)
    c = with_norm_inputs(dict(T=19, H=7168, E=64, ep=8, k=6, drop_frac=0.1, shared_sd=0.5))
    inp = gen.make_inputs(c, seed=2)
    nt, v = (int(x) for x in tile.split("x")[:2])
    check_bf16(run_combine(inp, 2), oracle_all(inp, "bf16"), 1e-3, tile)
    c_, s_ = run_mxfp8(inp, 2)
    check_mxfp8(c_, s_, *oracle_all(inp, "mxfp8"), tile)
    c4, s4 = run_mxfp4(inp, 2)
    check_mxfp4(c4, s4, *oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared), tile)
    if nt * v * 8 >= inp.H:
        ro, no = run_rmsnorm(inp, 0.0, 2)
        rro, rno = oracle_all(inp, "rmsnorm", 0.0)
        check_bf16(ro, rro, 1e-3, tile)
        check_bf16(no, rno, 1e-3, tile)
        check_rmsnorm_mxfp8(inp, 1.0, 2, want_norm=True, what=tile)


# ----------------------------------------------- full workload sizes

@pytest.mark.slow
def test_full_size_mxfp4():
    """MXFP4 output on the MXFP8 workload's inputs (T=16384, H=7168)."""
    inp = gen.make_inputs("mxfp8", 0)
    c, s = run_mxfp4(inp)
    check_mxfp4(c, s, *oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared),
                "mxfp4 workload")


@pytest.mark.slow
@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_full_size_rmsnorm_mxfp8(wb):
    """The RMSNorm workload with the normalised row quantised to MXFP8."""
    inp = gen.make_inputs("rmsnorm", 0)
    check_rmsnorm_mxfp8(inp, wb, want_norm=(wb == 0.0), what="rmsnorm workload")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dsv3", "skewed", "rmsnorm", "mxfp8"])
def test_full_size_workloads(name):
    """The full synthetic workloads in the launch configuration the benchmark
    times, compared element by element with the oracle."""
    inp = gen.make_inputs(name, 0)
    if name == "rmsnorm":
        for wb in (0.0, 1.0):
            ro, no = run_rmsnorm(inp, wb)
            rro, rno = oracle_all(inp, "rmsnorm", wb)
            check_bf16(ro, rro, 1e-3, f"{name} residual_out wb={wb}")
            check_bf16(no, rno, 1e-3, f"{name} norm_out wb={wb}")
    elif name == "mxfp8":
        c, s = run_mxfp8(inp)
        check_mxfp8(c, s, *oracle_all(inp, "mxfp8"), name)
    else:
        check_bf16(run_combine(inp), oracle_all(inp, "bf16"), 1e-3, name)


# ------------------------------------------------- dense / local reduce

@pytest.mark.parametrize("n_in,T,H,scales,tok", [
    (1, 5, 8, False, False), (2, 33, 264, True, True), (8, 64, 7168, False, False),
    (13, 9, 1032, True, False), (32, 3, 512, True, True), (4, 17, 4096, False, True)])
def test_reduce_dense(n_in, T, H, scales, tok):
    d = gen.make_dense_inputs(dict(n_in=n_in, T=T, H=H, scales=scales,
                                   token_sd=0.5 if tok else None, residual_sd=1.0), seed=n_in)
    x = dev16(d.x)
    sc = None if d.scales is None else torch.from_numpy(d.scales).to(DEV)
    tk = None if d.tok is None else dev16(d.tok)
    out = poisoned16(T, H, 2)
    mc.moe_reduce_dense(x, sc, tk, out=out)
    torch.cuda.synchronize()
    o = host16(out)
    assert (o[T:] == POISON16).all()
    check_bf16(o[:T], oracle.reduce_dense(d.x, d.scales, d.tok), 1e-3, "reduce_dense")
    if H % 8 == 0 and H <= 32768:
        ro, no = mc.moe_reduce_dense_residual_rmsnorm(x, sc, tk, dev16(d.residual), dev16(d.gamma),
                                                      d.eps, 1.0)
        rro, rno = oracle.reduce_dense(d.x, d.scales, d.tok, d.residual, d.gamma, d.eps, 1.0)
        check_bf16(host16(ro), rro, 1e-3, "reduce_dense residual_out")
        check_bf16(host16(no), rno, 1e-3, "reduce_dense norm_out")


def test_skip_a2a_partials_then_local_reduce():
    """Each simulated rank combines only the slots it hosts (other slots
    dropped), writing a bf16 partial; the local reduce sums the partials.
    The same pipeline in the oracle gives the same bits."""
    inp = gen.make_inputs(dict(T=256, H=2048, E=64, ep=8, k=8), seed=5)
    d = to_dev(inp)
    parts, ref_parts = [], []
    for r in range(inp.ep):
        src = inp.src_info.copy()
        src[src[..., 0] != r] = -1
        parts.append(mc.moe_combine(d["payload"], torch.from_numpy(src).to(DEV), d["weights"]))
        ref_parts.append(oracle.combine(inp.payload, src, inp.weights))
    out = mc.moe_reduce_dense(torch.stack(parts).contiguous())
    ref = oracle.reduce_dense(np.stack(ref_parts))
    np.testing.assert_array_equal(host16(out), ref)
    # and it differs from the direct combine only by the roundings of the
    # partials (<= half a bf16 step of each) and of the two results
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    direct = f(oracle.combine(inp.payload, inp.src_info, inp.weights))
    bound = sum(np.abs(f(p_)) for p_ in ref_parts) * 2.0 ** -8 \
        + (np.abs(direct) + np.abs(f(ref))) * 2.0 ** -8 + 1e-30
    assert (np.abs(f(ref) - direct) <= bound).all()


@pytest.mark.slow
def test_full_size_dense8():
    d = gen.make_dense_inputs("dense8", 0)
    out = mc.moe_reduce_dense(dev16(d.x))
    check_bf16(host16(out), oracle.reduce_dense(d.x), 1e-3, "dense8")


# ------------------------------------------------------------- dispatch

def _dispatch_case(T, H, k, E, ep, cap, drop, seed, bad_ids=False):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[rng.random((T, k)) < drop] = -1
    if bad_ids:
        ids[rng.random((T, k)) < 0.05] = E + 3          # out of range -> dropped
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    clean = np.where((ids >= 0) & (ids < E), ids, -1).astype(np.int32)
    if cap is None:
        kept = clean[clean >= 0]
        cap = max(1, int(np.bincount(kept // (E // ep), minlength=ep).max()) if kept.size else 1)
    return x, ids, clean, cap


@pytest.mark.parametrize("T,H,k,E,ep,cap,drop,bad", [
    (1, 8, 1, 1, 1, None, 0.0, False),
    (37, 264, 3, 12, 3, None, 0.1, False),
    (300, 1024, 8, 64, 8, 40, 0.0, False),         # capacity drops
    (1500, 512, 4, 256, 4, None, 0.2, True),       # > one chunk, bad ids
    (2048, 2048, 8, 4096, 8, None, 0.0, False),    # maximum expert count
    (513, 96, 32, 32, 1, 200, 0.0, False),         # top_k = 32, tight capacity
    (2000, 64, 8, 1024, 1, None, 0.0, False),      # 1024 experts on one rank: 63 chunks per column
    (700, 64, 6, 4096, 2, None, 0.05, True),       # 2048 experts per rank
    (4100, 64, 8, 4096, 1, 3000, 0.0, False),      # 4096 experts on one rank, capacity drops
    (64, 64, 4, 16, 4, 1, 0.0, False),             # capacity 1: one row per rank
    (100, 64, 2, 8, 2, None, 1.0, False),          # every slot dropped: nothing placed
])
@pytest.mark.parametrize("path", ["place", "count_scan"])
def test_dispatch_matches_oracle(T, H, k, E, ep, cap, drop, bad, path, monkeypatch):
    monkeypatch.setenv("MOE_DISPATCH_PATH", path)
    x, ids, clean, cap = _dispatch_case(T, H, k, E, ep, cap, drop, seed=T + k, bad_ids=bad)
    poison = np.full((ep, cap, H), 0xFFFF, np.uint16)
    counts0 = np.arange(E, dtype=np.int32) % 7                 # accumulates onto this
    rp, rs, rc = oracle.dispatch(x, clean, E, ep, cap, payload=poison.copy(), recv_counts=counts0.copy())
    pay = dev16(poison)
    cnt = torch.from_numpy(counts0.copy()).to(DEV)
    pay, src = mc.moe_dispatch(dev16(x), torch.from_numpy(ids).to(DEV), E, ep, cap,
                               payload=pay, recv_counts=cnt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(src.cpu().numpy(), rs)
    np.testing.assert_array_equal(host16(pay), rp)               # placed rows and untouched ones
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)


@pytest.mark.parametrize("i", range(12))
@pytest.mark.parametrize("path", ["place", "count_scan"])
def test_dispatch_random_shapes(i, path, monkeypatch):
    monkeypatch.setenv("MOE_DISPATCH_PATH", path)
    rng = np.random.default_rng(9000 + i)
    k = int(rng.choice([1, 2, 4, 8, 32]))
    ep = int(rng.choice([1, 2, 4, 8]))
    E = ep * max(-(-k // ep), int(rng.choice([1, 3, 16, 64, 512])))
    T = int(rng.integers(1, 3000))
    H = int(rng.choice([8, 64, 264, 1024]))
    cap = None if rng.random() < 0.5 else int(rng.integers(1, max(2, T * k // ep)))
    drop = float(rng.choice([0.0, 0.2]))
    x, ids, clean, cap = _dispatch_case(T, H, k, E, ep, cap, drop, seed=i, bad_ids=bool(rng.random() < 0.3))
    counts0 = np.zeros(E, dtype=np.int32)
    rp, rs, rc = oracle.dispatch(x, clean, E, ep, cap, recv_counts=counts0.copy())
    cnt = torch.from_numpy(counts0).to(DEV)
    pay, src = mc.moe_dispatch(dev16(x), torch.from_numpy(ids).to(DEV), E, ep, cap, recv_counts=cnt)
    torch.cuda.synchronize()
    what = f"T={T} H={H} k={k} E={E} ep={ep} cap={cap}"
    np.testing.assert_array_equal(src.cpu().numpy(), rs, err_msg=what)
    np.testing.assert_array_equal(host16(pay), rp, err_msg=what)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc, err_msg=what)


def test_dispatch_identity_combine_round_trip_on_gpu():
    """GPU dispatch -> identity experts -> GPU combine gives the oracle's bits
    for the same pipeline, and bf16(x * sum of kept weights) within 1 step."""
    inp = gen.make_inputs(dict(T=512, H=2048, E=64, ep=8, k=8, drop_frac=0.1), seed=3)
    rng = np.random.default_rng(0)
    x = to_bf16_bits(rng.standard_normal((inp.T, inp.H)).astype(np.float32))
    ids = inp.topk_ids.copy()
    ids[inp.src_info[..., 0] < 0] = -1
    cap = inp.mtpr
    pay, src = mc.moe_dispatch(dev16(x), torch.from_numpy(ids).to(DEV), 64, 8, cap)
    w = torch.from_numpy(inp.weights).to(DEV)
    out = host16(mc.moe_combine(pay, src, w))
    rp, rs, _ = oracle.dispatch(x, ids, 64, 8, cap)
    np.testing.assert_array_equal(out, oracle.combine(rp, rs, inp.weights))
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wsum = np.where(rs[..., 0] >= 0, inp.weights, 0).astype(np.float64).sum(axis=1)
    assert ulp_dist_bf16(out, to_bf16_bits(f * wsum[:, None])).max() <= 1


@pytest.mark.slow
@pytest.mark.parametrize("name,path", [("dsv3", "place"), ("dsv3", "count_scan"),
                                       ("mxfp8", "place"), ("mxfp8", "count_scan")])
def test_full_size_dispatch(name, path, monkeypatch):
    monkeypatch.setenv("MOE_DISPATCH_PATH", path)
    inp = gen.make_inputs(dict(gen.CONFIGS[name], H=8), seed=0)   # routing only
    T, H, E = inp.T, gen.CONFIGS[name]["H"], inp.meta["E"]
    rng = np.random.default_rng(1)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    rp, rs, rc = oracle.dispatch(x, inp.topk_ids, E, inp.ep, inp.mtpr)
    cnt = torch.zeros(E, dtype=torch.int32, device=DEV)
    pay, src = mc.moe_dispatch(dev16(x), torch.from_numpy(inp.topk_ids).to(DEV), E, inp.ep,
                               inp.mtpr, recv_counts=cnt)
    np.testing.assert_array_equal(src.cpu().numpy(), rs)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(src.cpu().numpy(), inp.src_info)   # generator's map too
    v = rs[..., 0] >= 0
    np.testing.assert_array_equal(host16(pay)[rs[..., 0][v], rs[..., 1][v]],
                                  rp[rs[..., 0][v], rs[..., 1][v]])


# ------------------------------------------------------------ HIP graphs

@pytest.mark.parametrize("path", ["place", "count_scan"])
def test_hip_graph_capture_and_replay(path, monkeypatch):
    """The entry points allocate nothing and never synchronise, so they can
    be captured in a graph: dispatch (either placement path) followed by the
    combine, replayed three times with new input contents written eagerly
    between replays; every replay matches the oracle."""
    monkeypatch.setenv("MOE_DISPATCH_PATH", path)
    inp = gen.make_inputs(dict(T=200, H=1024, E=32, ep=4, k=4, drop_frac=0.1), seed=2)
    T, H, E = inp.T, inp.H, 32
    ids = inp.topk_ids.copy()
    ids[inp.src_info[..., 0] < 0] = -1
    ids_d = torch.from_numpy(ids).to(DEV)
    w_d = torch.from_numpy(inp.weights).to(DEV)
    x_d = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    pay = torch.zeros((inp.ep, inp.mtpr, H), dtype=torch.bfloat16, device=DEV)
    src = torch.empty((T, inp.k, 2), dtype=torch.int32, device=DEV)
    ws = torch.empty(mc.dispatch_workspace_size(T, inp.k, E, inp.ep, inp.mtpr),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        mc.moe_dispatch(x_d, ids_d, E, inp.ep, inp.mtpr, payload=pay, src_info=src, workspace=ws)
        mc.moe_combine(pay, src, w_d, None, out=out)

    rng = np.random.default_rng(0)
    x0 = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x_d.copy_(dev16(x0))
    step()                                   # eager warm-up
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * (rep + 1))
        x_d.copy_(dev16(x))                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rp, rs, _ = oracle.dispatch(x, ids, E, inp.ep, inp.mtpr)
        np.testing.assert_array_equal(src.cpu().numpy(), rs)
        np.testing.assert_array_equal(host16(out), oracle.combine(rp, rs, inp.weights),
                                      err_msg=f"replay {rep}")
