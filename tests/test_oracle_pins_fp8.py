"""Pins of the oracle's fp8 and MX functions against something other than
themselves.

* oracle.brute re-derives every step element by element: scalar encoders
  written from the formats' definitions (frexp / round, not the code-table
  searches of oracle.formats), fp32 roundings through struct, math.fsum sums.
* Inputs are built so that the rounding points the path fixes are the ones
  that decide the result: each test checks that a plausible single mistake
  (amax taken before the bf16 store, an fp64 reciprocal scale, a scale left
  out, a transposed operand) would change the answer, and a planted-mistake
  test confirms the comparison catches it.
* Exact-integer inputs where every rounding point is exact, so the fp8
  backward's GEMMs must equal plain integer arithmetic.

Sources: "Collective GEMMs in Tensor Sequence Parallelism", section
"Supported quantization recipes" (FP8 current scaling, MXFP8); "Tensor
parallelism", section "Code" (ReLU' = 1 only where z > 0)."""
import math

import numpy as np
import pytest

from oracle import brute, formats, ops


def lists(a):
    return [[float(v) for v in row] for row in np.asarray(a)]


def q4(a):
    return formats.e4m3_to_f64(formats.e4m3_encode(a))


def gelu_scalar(z):
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def gelu_grad_scalar(z):
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0))) + z * math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


# ----------------------------------------------------------------- encoders
def test_scalar_encoders_agree_with_code_table_encoders():
    g = np.random.default_rng(301)
    v = np.concatenate([g.standard_normal(20000) * np.exp(g.uniform(-30, 14, 20000)),
                        formats.E4M3_TABLE[:0x7F], (formats.E4M3_TABLE[1:0x7F] + formats.E4M3_TABLE[:0x7E]) / 2,
                        formats.E5M2_TABLE[:0x7C], (formats.E5M2_TABLE[1:0x7C] + formats.E5M2_TABLE[:0x7B]) / 2,
                        [448.0, 464.0, 479.0, 500.0, 57344.0, 61440.0, 1e6, 2.0 ** -10, 2.0 ** -17, 0.0]])
    v = np.concatenate([v, -v]).astype(np.float32).astype(np.float64)
    e4 = formats.e4m3_to_f64(formats.e4m3_encode(v))
    e5 = formats.e5m2_to_f64(formats.e5m2_encode(v))
    bf = formats.round_bf16(v)
    for i, x in enumerate(v):
        assert brute.e4m3(x) == e4[i] and math.copysign(1, brute.e4m3(x)) == math.copysign(1, e4[i]), x
        assert brute.e5m2(x) == e5[i], x
        assert brute.bf16(x) == bf[i], x


# ------------------------------------------------------- fp8 forward (current)
def _fwd_inputs(seed, M, D, F):
    g = np.random.default_rng(seed)
    xq = q4(g.standard_normal((M, D)) * 4)
    wu = q4(g.standard_normal((D, F)) * 4)
    wd = q4(g.standard_normal((F, D)) * 4)
    return xq, wu, wd


@pytest.mark.parametrize("seed,M,D,F", [(311, 4, 8, 12), (312, 3, 16, 7), (313, 5, 5, 9)])
def test_fp8_forward_equals_brute_force(seed, M, D, F):
    xq, wu, wd = _fwd_inputs(seed, M, D, F)
    sx, su, sd = 0.25, 0.015625, 0.0078125
    r = ops.tp_mlp_fwd_fp8(xq, sx, wu, su, wd, sd, ops.ACT_GELU_ERF)
    b = brute.mlp_fwd_fp8(lists(xq), sx, lists(wu), su, lists(wd), sd, gelu_scalar)
    assert np.allclose(r["Z"], b["Z"], rtol=1e-14, atol=0)
    assert np.array_equal(r["Hb"], np.array(b["Hb"]))
    assert r["amax"] == b["amax"] and r["inv"] == b["inv"] and r["sH"] == b["sH"]
    assert np.array_equal(formats.e4m3_to_f64(r["Hq_codes"]), np.array(b["Hq"]))
    assert np.allclose(r["P"], b["P"], rtol=1e-13, atol=0)


def test_fp8_forward_amax_is_taken_on_the_stored_bf16_values():
    """An H whose largest element moves when rounded to bf16, and whose
    codes then depend on which amax is used: the oracle's equality with the
    brute force pins the rounding point (amax over the stored bf16 H)."""
    for seed in range(340, 400):
        xq, wu, wd = _fwd_inputs(seed, 6, 16, 40)
        r = ops.tp_mlp_fwd_fp8(xq, 0.25, wu, 0.015625, wd, 0.0078125, ops.ACT_GELU_ERF)
        amax_raw = float(np.max(np.abs(r["H"])))
        inv_raw = brute.fp32(448.0 / brute.fp32(amax_raw))
        wrong = [[brute.e4m3(brute.fp32(v * inv_raw)) for v in row] for row in r["Hb"]]
        if amax_raw != r["amax"] and np.array(wrong).tolist() != formats.e4m3_to_f64(r["Hq_codes"]).tolist():
            break
    else:
        raise AssertionError("no discriminating input found")
    b = brute.mlp_fwd_fp8(lists(xq), 0.25, lists(wu), 0.015625, lists(wd), 0.0078125, gelu_scalar)
    assert np.array_equal(formats.e4m3_to_f64(r["Hq_codes"]), np.array(b["Hq"]))
    assert r["amax"] == b["amax"] and np.allclose(r["P"], b["P"], rtol=1e-13, atol=0)


def _find_fp32_inv_witness():
    """(amax, v) with amax >= |v| both bf16 values, such that
    e4m3(fp32(v * fp32(448 / amax))) differs from e4m3(v * 448 / amax)."""
    g = np.random.default_rng(315)
    for _ in range(4000):
        amax = float(formats.round_bf16(np.array([g.uniform(1.0, 1000.0)]))[0])
        inv32 = brute.fp32(448.0 / amax)
        inv64 = 448.0 / amax
        if inv32 == inv64:
            continue
        v = formats.round_bf16(g.uniform(-amax, amax, 4096))
        c32 = formats.e4m3_encode((v.astype(np.float32) * np.float32(inv32)).astype(np.float64))
        c64 = formats.e4m3_encode(v * inv64)
        bad = np.flatnonzero(c32 != c64)
        if bad.size:
            return amax, float(v[bad[0]])
    raise AssertionError("no witness found")


def test_current_scaling_reciprocal_is_an_fp32_quotient():
    amax, v = _find_fp32_inv_witness()
    q = ops.quantize_current(np.array([amax, v]), "e4m3")
    want = [brute.e4m3(brute.fp32(t * brute.fp32(448.0 / amax))) for t in (amax, v)]
    assert formats.e4m3_to_f64(q["codes"]).tolist() == want
    assert q["inv"] == brute.fp32(448.0 / amax) and q["s"] == brute.fp32(amax / 448.0)
    assert brute.e4m3(v * (448.0 / amax)) != want[1]          # the fp64 reading gives another code


def test_current_scaling_special_cases():
    q = ops.quantize_current(np.zeros((3, 4)), "e4m3")
    assert q["inv"] == 1.0 and q["s"] == 1.0 and not q["codes"].any()
    q = ops.quantize_current(np.array([-3.5, 0.5, 1.75]), "e5m2")
    assert q["inv"] == 16384.0 and q["s"] == 2.0 ** -14
    assert formats.e5m2_to_f64(q["codes"]).tolist() == [-57344.0, 8192.0, 28672.0]
    q = ops.quantize_current(np.array([7.0, -7.0, 1.0]), "e4m3")
    assert formats.e4m3_to_f64(q["codes"]).tolist() == [448.0, -448.0, 64.0]    # amax maps to the top code


# ------------------------------------------------------------- fp8 backward
def _bwd_inputs(seed, M, D, F):
    g = np.random.default_rng(seed)
    x8, wu8, wd8 = q4(g.standard_normal((M, D)) * 8), q4(g.standard_normal((D, F)) * 8), q4(g.standard_normal((F, D)) * 8)
    h8 = q4(np.abs(g.standard_normal((M, F))) * 8)
    z = formats.round_bf16(g.standard_normal((M, F)))
    dy = formats.round_bf16(g.standard_normal((M, D)))
    return x8, wu8, wd8, h8, z, dy


@pytest.mark.parametrize("seed,M,D,F", [(321, 4, 6, 5), (322, 3, 8, 4)])
def test_fp8_backward_equals_brute_force(seed, M, D, F):
    x8, wu8, wd8, h8, z, dy = _bwd_inputs(seed, M, D, F)
    sx, su, sd, sh = 0.125, 0.0078125, 0.0078125, 0.03125
    r = ops.tp_mlp_bwd_fp8(x8, sx, wu8, su, wd8, sd, z, h8, sh, dy, ops.ACT_GELU_ERF)
    b = brute.mlp_bwd_fp8(lists(x8), sx, lists(wu8), su, lists(wd8), sd, lists(z), lists(h8), sh, lists(dy),
                          gelu_grad_scalar)
    assert np.array_equal(r["dYq"], np.array(b["dYq"])) and r["s_dY"] == b["s_dY"]
    assert np.allclose(r["dH"], b["dH"], rtol=1e-13, atol=0)
    assert np.array_equal(r["dZ"], np.array(b["dZ"]))
    assert np.array_equal(r["dZq"], np.array(b["dZq"])) and r["s_dZ"] == b["s_dZ"]
    for k in ("dW_down", "dW_up", "dX"):
        assert np.allclose(r[k], b[k], rtol=1e-13, atol=0), k


def test_fp8_backward_exact_integer_inputs():
    """Every rounding point exact: e4m3 integers with unit scales, dY on the
    e5m2 grid scaled by a power of two (amax 3.5, so 57344 / amax = 2^14),
    ReLU with exact zeros in Z.  dYq s_dY = dY, dH = dY W_down^T, dZ =
    dH * [Z > 0] and dW_down = Hq^T dY are then plain integer / half-integer
    arithmetic."""
    g = np.random.default_rng(323)
    M, D, F = 6, 8, 5
    x8 = g.integers(-3, 4, (M, D)).astype(np.float64)
    wu8 = g.integers(-3, 4, (D, F)).astype(np.float64)
    wd8 = g.integers(-3, 4, (F, D)).astype(np.float64)
    h8 = g.integers(0, 4, (M, F)).astype(np.float64)
    z = g.integers(-2, 3, (M, F)).astype(np.float64)
    z[0, :] = 0.0                                                        # the kink itself
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, -0.5, -1.0, -1.5, -2.0, -2.5, -3.0])
    dy = g.choice(grid, (M, D))
    dy[2, 3] = -3.5
    r = ops.tp_mlp_bwd_fp8(x8, 1.0, wu8, 1.0, wd8, 1.0, z, h8, 1.0, dy, ops.ACT_RELU)
    assert r["s_dY"] == 2.0 ** -14 and np.array_equal(r["dYq"] * r["s_dY"], dy)
    dh = dy @ wd8.T
    assert np.array_equal(r["dH"], dh)
    assert np.array_equal(r["dZ"], dh * (z > 0))
    assert not r["dZ"][0].any()                                          # ReLU'(0) = 0
    assert np.array_equal(r["dW_down"], h8.T @ dy)
    b = brute.mlp_bwd_fp8(lists(x8), 1.0, lists(wu8), 1.0, lists(wd8), 1.0, lists(z), lists(h8), 1.0, lists(dy),
                          lambda t: 1.0 if t > 0 else 0.0)
    for k in ("dW_up", "dX"):
        assert np.allclose(r[k], b[k], rtol=1e-13, atol=0), k


# ----------------------------------------------------------------- MXFP8
@pytest.mark.parametrize("seed", [331, 332])
def test_mx_forward_equals_brute_force(seed):
    g = np.random.default_rng(seed)
    M, D, F = 3, 64, 96
    x = g.standard_normal((M, D)) * np.exp(g.uniform(-4, 4, (M, 1)))
    x[1, 32:] = 0.0                                                      # an all-zero block
    xc, xs = formats.mx_e4m3_quantize(x)
    uc, us = formats.mx_e4m3_quantize(g.standard_normal((F, D)) * 0.1)
    dc, ds = formats.mx_e4m3_quantize(g.standard_normal((D, F)) * 0.1)
    r = ops.tp_mlp_fwd_mx(xc, xs, uc, us, dc, ds, ops.ACT_GELU_ERF)
    xd, ud, dd = (formats.mx_e4m3_decode(c, s) for c, s in ((xc, xs), (uc, us), (dc, ds)))
    # the brute-force quantiser reproduces the input codes' values
    for row, got in zip(x, xd):
        assert brute.mx_quantize_row([float(t) for t in row])[0] == got.tolist()
    b = brute.mlp_fwd_mx(lists(xd), lists(ud), lists(dd), gelu_scalar)
    assert np.allclose(r["Z"], b["Z"], rtol=1e-13, atol=1e-300)
    assert np.array_equal(formats.mx_e4m3_decode(r["Hq_codes"], r["Hq_scales"]), np.array(b["Hq"]))
    assert np.array_equal(r["Hq_scales"], np.array(b["Hexp"]))
    assert np.allclose(r["P"], b["P"], rtol=1e-13, atol=1e-300)


# ------------------------------------------------------- GeLU (tanh form)
def test_gelu_tanh_at_closed_form_points():
    """0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) evaluated with math.tanh
    at points, and its derivative against the product rule written out."""
    c = math.sqrt(2.0 / math.pi)
    for z in (-6.0, -3.0, -1.0, -0.5, -1e-3, 0.0, 1e-3, 0.25, 1.0, 2.0, 3.7, 8.0):
        u = c * (z + 0.044715 * z ** 3)
        want = 0.5 * z * (1.0 + math.tanh(u))
        assert abs(ops.gelu_tanh(np.array([z]))[0] - want) <= 1e-15 * max(1.0, abs(want))
        t = math.tanh(u)
        dwant = 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * z * z)
        assert abs(ops.gelu_tanh_grad(np.array([z]))[0] - dwant) <= 1e-15 * max(1.0, abs(dwant))
    # known value: at z = 1, u = sqrt(2/pi) * 1.044715
    assert abs(ops.gelu_tanh(np.array([1.0]))[0] - 0.8411919906082768) < 1e-15


# ------------------------------------------------------- planted mistakes
def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible single mistake, planted in the oracle, makes one of the
    comparisons above fail."""
    xq, wu, wd = _fwd_inputs(311, 4, 8, 12)
    b = brute.mlp_fwd_fp8(lists(xq), 0.25, lists(wu), 0.015625, lists(wd), 0.0078125, gelu_scalar)

    def fwd_agrees():
        try:
            r = ops.tp_mlp_fwd_fp8(xq, 0.25, wu, 0.015625, wd, 0.0078125, ops.ACT_GELU_ERF)
        except AssertionError:          # the oracle's own guard caught it
            return False
        return (np.array_equal(formats.e4m3_to_f64(r["Hq_codes"]), np.array(b["Hq"]))
                and np.allclose(r["P"], b["P"], rtol=1e-13, atol=0))
    assert fwd_agrees()
    real_round = formats.round_bf16
    # 1. H not rounded to bf16 before its amax and quantisation (kept in
    # fp32, or not rounded at all)
    monkeypatch.setattr(formats, "round_bf16", lambda v: np.asarray(v, dtype=np.float32).astype(np.float64))
    assert not fwd_agrees()
    monkeypatch.setattr(formats, "round_bf16", lambda v: np.asarray(v, dtype=np.float64))
    assert not fwd_agrees()
    monkeypatch.setattr(formats, "round_bf16", real_round)
    # 2. the second GEMM's scale without s_H
    real_q = ops.quantize_current
    monkeypatch.setattr(ops, "quantize_current", lambda v, f: {**real_q(v, f), "s": 1.0})
    assert not fwd_agrees()
    monkeypatch.setattr(ops, "quantize_current", real_q)
    # 3. backward: dW_down from dY before quantisation (dYq left out)
    x8, wu8, wd8, h8, z, dy = _bwd_inputs(321, 4, 6, 5)
    bb = brute.mlp_bwd_fp8(lists(x8), 0.125, lists(wu8), 0.0078125, lists(wd8), 0.0078125, lists(z), lists(h8),
                           0.03125, lists(dy), gelu_grad_scalar)

    def bwd_agrees():
        r = ops.tp_mlp_bwd_fp8(x8, 0.125, wu8, 0.0078125, wd8, 0.0078125, z, h8, 0.03125, dy, ops.ACT_GELU_ERF)
        return all(np.allclose(r[k], bb[k], rtol=1e-13, atol=0) for k in ("dW_down", "dW_up", "dX"))
    assert bwd_agrees()
    monkeypatch.setattr(ops, "quantize_current", lambda v, f: {**real_q(v, f), "dec": np.asarray(v) / real_q(v, f)["s"]})
    assert not bwd_agrees()
    monkeypatch.setattr(ops, "quantize_current", real_q)
    # 4. a transposed operand in the backward (W_down read as [D, F/T])
    real_gemm = ops.gemm
    calls = []

    def gemm_t(a, b_):
        calls.append(1)
        if len(calls) == 1:                       # dH = dYq . W_down^T -> uses W_down un-transposed
            return real_gemm(a, np.asarray(b_)[::-1])
        return real_gemm(a, b_)
    monkeypatch.setattr(ops, "gemm", gemm_t)
    assert not bwd_agrees()
