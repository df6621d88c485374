"""Pins of the fp64 oracle against facts that do not come from the oracle:
bit definitions, library casts, brute force, closed forms, finite
differences, the pages' own invariants and printed numbers."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, formats, ops, schedule, shapes
import synthetic_inputs as si

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


# ------------------------------------------------------------------ formats
def test_e4m3_table_from_definition():
    t = formats.E4M3_TABLE
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x44] == 3.0 and t[0x48] == 4.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.isfinite(t).sum() == 254


def test_e4m3_matches_torch_cast():
    # independent implementation: PyTorch's float8_e4m3fn cast
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 300)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = formats.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_roundtrip_ties_and_saturation():
    codes = np.array([c for c in range(256) if not math.isnan(formats.E4M3_TABLE[c])], dtype=np.uint8)
    vals = formats.e4m3_to_f64(codes)
    assert np.array_equal(formats.e4m3_encode(vals), codes)
    pos = formats.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    enc = formats.e4m3_encode(mids).astype(int)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)     # tie -> even code
    assert np.array_equal(enc, expect)
    assert formats.e4m3_encode(np.array([1000.0, 449.0, -1e9]))[0] == 0x7E
    assert formats.e4m3_encode(np.array([-1e9]))[0] == 0xFE
    assert formats.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_bf16_matches_torch_and_ties():
    g = np.random.default_rng(7)
    bits = g.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # structured mantissa tails around the rounding point, every exponent
    exps = np.arange(0, 255, dtype=np.uint32) << np.uint32(23)
    tails = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x18000, 0x10000, 0x7F8000], dtype=np.uint32)
    hi = np.array([0, 0x10000, 0x7E0000, 0x7F0000], dtype=np.uint32)
    struct = (exps[:, None, None] | hi[None, :, None] | tails[None, None, :]).ravel()
    bits = np.concatenate([bits, struct, struct | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = formats.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # explicit ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert formats.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert formats.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


# -------------------------------------------------------------- activations
@pytest.mark.parametrize("act", [ops.ACT_RELU, ops.ACT_GELU_ERF, ops.ACT_GELU_TANH, ops.ACT_NONE, ops.ACT_SILU])
def test_activation_derivatives_by_central_differences(act):
    z = np.linspace(-6, 6, 2401) + 1e-3      # avoid the ReLU kink
    h = 1e-6
    fd = (ops.act_fwd(z + h, act) - ops.act_fwd(z - h, act)) / (2 * h)
    assert np.max(np.abs(fd - ops.act_grad(z, act))) < 1e-7


def test_activation_closed_forms():
    assert ops.gelu_erf(np.array([0.0]))[0] == 0.0
    assert ops.gelu_erf_grad(np.array([0.0]))[0] == 0.5
    assert ops.gelu_tanh_grad(np.array([0.0]))[0] == 0.5
    assert ops.relu_grad(np.array([0.0]))[0] == 0.0            # page: 1 only where z > 0
    big = np.array([10.0, -10.0])
    assert np.allclose(ops.gelu_erf(big), [10.0, 0.0], atol=1e-12)
    z = np.linspace(-8, 8, 100001)
    diff = np.max(np.abs(ops.gelu_erf(z) - ops.gelu_tanh(z)))
    assert 1e-4 < diff < 5e-4
    # Phi(1) from the standard normal table
    assert abs(ops.gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15


def test_silu_closed_forms():
    from scipy.special import expit
    z = np.linspace(-30, 30, 6001)
    assert np.allclose(ops.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)      # z * logistic(z)
    assert np.allclose(ops.silu(-z), ops.silu(z) - z, rtol=0, atol=1e-12)       # sigma(-z) = 1 - sigma(z)
    assert ops.silu(np.array([0.0]))[0] == 0.0
    assert ops.silu_grad(np.array([0.0]))[0] == 0.5
    # logistic(1) = 1 / (1 + 1/e) = 0.7310585786300049
    assert abs(ops.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    assert abs(ops.silu(np.array([40.0]))[0] - 40.0) < 1e-12 and abs(ops.silu(np.array([-40.0]))[0]) < 1e-15
    assert np.allclose(ops.silu_grad(np.array([40.0, -40.0])), [1.0, 0.0], atol=1e-12)


# --------------------------------------------------------------- e5m2
def test_e5m2_table_from_definition():
    t = formats.E5M2_TABLE
    assert t[0x7B] == 57344.0 and t[0x01] == 2.0 ** -16 and t[0x04] == 2.0 ** -14
    assert np.isinf(t[0x7C]) and np.isnan(t[0x7D]) and t[0x3C] == 1.0
    assert np.all(np.diff(t[:0x7C]) > 0)                  # ascending magnitudes
    assert np.array_equal(t[0x80:0xFC], -t[:0x7C])


def test_e5m2_encoder_against_torch_and_saturation():
    g = np.random.default_rng(86)
    v = np.concatenate([g.standard_normal(200000) * np.exp(g.uniform(-20, 11, 200000)),
                        formats.E5M2_TABLE[:0x7C], (formats.E5M2_TABLE[1:0x7C] + formats.E5M2_TABLE[:0x7B]) / 2])
    v = v[np.abs(v) < 57344].astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(formats.e5m2_encode(v.astype(np.float64)), want)   # includes every tie
    assert np.array_equal(formats.e5m2_encode(np.array([60000.0, -1e9, 57344.0])), [0x7B, 0xFB, 0x7B])


def test_fp8_backward_mirror_composes_and_bounds():
    g = np.random.default_rng(87)
    M, D, Ft = 32, 64, 48
    q4 = lambda a: formats.e4m3_to_f64(formats.e4m3_encode(a))
    x8, wu8, wd8, h8 = q4(g.standard_normal((M, D)) * 8), q4(g.standard_normal((D, Ft)) * 8), \
        q4(g.standard_normal((Ft, D)) * 8), q4(np.abs(g.standard_normal((M, Ft))) * 8)
    sx, su, sd, sh = 0.125, 0.0078125, 0.0078125, 0.03125
    z = formats.round_bf16(g.standard_normal((M, Ft)))
    dy = formats.round_bf16(g.standard_normal((M, D)))
    r = ops.tp_mlp_bwd_fp8(x8, sx, wu8, su, wd8, sd, z, h8, sh, dy, ops.ACT_GELU_ERF)
    # quantised gradients: within half an e5m2 step (2^-3 relative in the normal range)
    for q, v, s in ((r["dYq"], dy, r["s_dY"]), (r["dZq"], r["dZ"], r["s_dZ"])):
        normal = np.abs(v) >= 2.0 ** -14 * s
        assert np.all(np.abs(q * s - v)[normal] <= 2.0 ** -3 * np.abs(v)[normal] * (1 + 1e-6))
        assert np.max(np.abs(q)) == 57344.0                 # current scaling maps amax to the top code
    # the chain, step by step
    assert np.allclose(r["dH"], r["dYq"] @ wd8.T * r["s_dY"] * sd, rtol=1e-12)
    assert np.array_equal(r["dZ"], formats.round_bf16(r["dH"] * ops.gelu_erf_grad(z)))
    assert np.allclose(r["dW_down"], h8.T @ r["dYq"] * sh * r["s_dY"], rtol=1e-12)
    assert np.allclose(r["dW_up"], x8.T @ r["dZq"] * sx * r["s_dZ"], rtol=1e-12)
    assert np.allclose(r["dX"], r["dZq"] @ wu8.T * r["s_dZ"] * su, rtol=1e-12)
    # and close to the unquantised backward
    ref = ops.tp_mlp_bwd(x8 * sx, wu8 * su, wd8 * sd, z, h8 * sh, dy, ops.ACT_GELU_ERF)
    for k in ("dW_down", "dW_up", "dX"):
        assert ops.normalized_error(r[k], ref[k]) < 0.25 * np.max(np.abs(ref[k]))


# ---------------------------------------------------------- delayed scaling
def test_delayed_scale_from_history():
    assert ops.fp8_delayed_scale([0.0, 0.0]) == 1.0
    assert ops.fp8_delayed_scale([1.0, 448.0, 3.0]) == 1.0
    assert ops.fp8_delayed_scale([2.0, 896.0]) == 2.0
    assert ops.fp8_delayed_scale([7.0]) == float(np.float32(np.float32(7.0) / np.float32(448.0)))


def test_fp8_delayed_forward_rounding_and_saturation():
    g = np.random.default_rng(85)
    M, D, Ft = 16, 64, 48
    xq = formats.e4m3_to_f64(formats.e4m3_encode(g.standard_normal((M, D))))
    wu = formats.e4m3_to_f64(formats.e4m3_encode(g.standard_normal((D, Ft)) * 4))
    wd = formats.e4m3_to_f64(formats.e4m3_encode(g.standard_normal((Ft, D)) * 4))
    sx, su, sd = 0.5, 0.03125, 0.0625
    h = ops.act_fwd(ops.gemm(xq, wu) * sx * su, ops.ACT_GELU_ERF)
    amax = float(np.max(np.abs(h)))
    # a fresh scale (amax of this very H): no element saturates, each within
    # half an e4m3 step of its value; P is the GEMM of the decoded codes
    s_h = ops.fp8_delayed_scale([amax])
    r = ops.tp_mlp_fwd_fp8_delayed(xq, sx, wu, su, wd, sd, s_h, ops.ACT_GELU_ERF)
    assert r["amax"] == amax
    dec = formats.e4m3_to_f64(r["Hq_codes"]) * s_h
    normal = np.abs(h) >= 2.0 ** -6 * s_h
    assert np.all(np.abs(dec - h)[normal] <= 2.0 ** -4 * np.abs(h)[normal] * (1 + 1e-6))
    assert np.allclose(r["P"], ops.gemm(formats.e4m3_to_f64(r["Hq_codes"]), wd) * s_h * sd, rtol=0, atol=1e-12)
    # a stale scale half as large: the largest elements saturate at +-448 s_h
    r2 = ops.tp_mlp_fwd_fp8_delayed(xq, sx, wu, su, wd, sd, s_h / 2, ops.ACT_GELU_ERF)
    big = np.abs(h) >= 448 * s_h / 2 * (1 + 2.0 ** -4)
    assert big.any()
    assert np.all(np.abs(formats.e4m3_to_f64(r2["Hq_codes"]))[big] == 448.0)


# ------------------------------------------------------------------ MXFP8
def test_mx_quantizer_against_definition_brute_force():
    # OCP MX: per 32-block a power-of-two scale X with max|V| / X in [256, 512)
    # (e4m3's largest normal exponent is 8), each element the nearest e4m3
    # value of V / X (ties to the even code), saturated at 448
    g = np.random.default_rng(81)
    v = g.standard_normal((6, 128)) * np.exp(g.uniform(-12, 12, size=(6, 1)))
    v[2, 32:64] = 0.0                                   # an all-zero block
    v[3, :32] = g.choice([-1.0, 1.0], 32) * 2.0 ** 5    # amax exactly a power of two
    v[4, 64:96] *= 1e-38                                # tiny block: scale exponent clamps at 0
    codes, e = formats.mx_e4m3_quantize(v)
    x = formats.e8m0_to_f64(e)
    grid = formats.E4M3_TABLE[:0x7F]                    # non-negative finite e4m3 values
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, 32 * b:32 * (b + 1)]
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert e[r, b] == 0
            elif e[r, b] > 0:
                assert 256 <= amax / x[r, b] < 512
            for i, val in enumerate(blk):
                t = abs(val) / x[r, b]
                d = np.abs(grid - t)
                best = np.flatnonzero(d == d.min())
                want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                if t >= 448:
                    want = 0x7E
                got = int(codes[r, 32 * b + i]) & 0x7F
                assert got == want, (r, b, i)
    assert e[3, 0] == 5 - 8 + 127
    dec = formats.mx_e4m3_decode(codes, e)
    assert np.array_equal(dec[2, 32:64], np.zeros(32))


def test_mx_roundtrip_and_relation_to_scaling():
    g = np.random.default_rng(82)
    # values already on an MX grid come back unchanged
    c0 = g.integers(0, 0x7F, size=(4, 64)).astype(np.uint8) | (g.integers(0, 2, size=(4, 64)) << 7).astype(np.uint8)
    c0[:, ::32] = 0x78                                    # 256 (2^8): the block maximum sets the scale
    e0 = g.integers(100, 150, size=(4, 2)).astype(np.uint8)
    v = formats.mx_e4m3_decode(c0, e0)
    c, e = formats.mx_e4m3_quantize(v)
    assert np.array_equal(e, e0) and np.array_equal(formats.mx_e4m3_decode(c, e), v)
    # scaling a block by a power of two moves only its exponent
    w = g.standard_normal((3, 96))
    c1, e1 = formats.mx_e4m3_quantize(w)
    c2, e2 = formats.mx_e4m3_quantize(w * 2.0 ** 7)
    assert np.array_equal(c1, c2) and np.array_equal(e2.astype(int), e1.astype(int) + 7)


def test_mx_input_quantizer_agrees_with_oracle():
    # the seeded-input MXFP8 cast (torch frexp / ldexp / float8 cast) and the
    # oracle's quantiser are written independently and must agree
    x = si.normal_f32((96, 512), 83) * np.float32(3.0)
    x[5, 64:96] = 0
    c, e = si.to_mxfp8(x)
    c2, e2 = formats.mx_e4m3_quantize(x.astype(np.float64))
    assert np.array_equal(c.numpy(), c2) and np.array_equal(e.numpy(), e2)


def test_mx_mlp_forward_composes_the_steps():
    g = np.random.default_rng(84)
    M, D, Ft = 8, 64, 96
    xq, xs = formats.mx_e4m3_quantize(g.standard_normal((M, D)))
    wu_q, wu_s = formats.mx_e4m3_quantize(g.standard_normal((Ft, D)) * 0.1)
    wd_q, wd_s = formats.mx_e4m3_quantize(g.standard_normal((D, Ft)) * 0.1)
    r = ops.tp_mlp_fwd_mx(xq, xs, wu_q, wu_s, wd_q, wd_s, ops.ACT_GELU_ERF)
    z = formats.mx_e4m3_decode(xq, xs) @ formats.mx_e4m3_decode(wu_q, wu_s).T
    assert np.allclose(r["Z"], z, rtol=0, atol=1e-12)
    assert np.array_equal(r["Hq_codes"], formats.mx_e4m3_quantize(ops.gelu_erf(z))[0])
    h_dec = formats.mx_e4m3_decode(r["Hq_codes"], r["Hq_scales"])
    # within e4m3's normal range (2^-6 .. 448 times the block scale) the
    # rounding error is at most half a step, 2^-4 of the value; above 448
    # the element saturates
    X = formats.e8m0_to_f64(np.repeat(r["Hq_scales"], 32, axis=1))
    t = np.abs(r["H"]) / X
    normal = (t >= 2.0 ** -6) & (t <= 448)
    assert np.all(np.abs(h_dec - r["H"])[normal] <= 2.0 ** -4 * np.abs(r["H"])[normal])
    assert np.all(np.abs(h_dec)[t > 448] == 448 * X[t > 448])
    assert np.allclose(r["P"], h_dec @ formats.mx_e4m3_decode(wd_q, wd_s).T, rtol=0, atol=1e-12)


# --------------------------------------------------------------- gated MLP
def _gated_brute(x, wg, wu, wd, act):
    """Pure-Python gated MLP share: correctly rounded sums (math.fsum) and
    the math module's erf / exp."""
    M, D = len(x), len(x[0])
    F = len(wg[0])
    def a(z):
        if act == ops.ACT_SILU:
            return z / (1.0 + math.exp(-z))
        if act == ops.ACT_GELU_ERF:
            return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
        assert act == ops.ACT_NONE
        return z
    h = [[a(math.fsum(x[i][k] * wg[k][j] for k in range(D))) * math.fsum(x[i][k] * wu[k][j] for k in range(D))
          for j in range(F)] for i in range(M)]
    return [[math.fsum(h[i][j] * wd[j][c] for j in range(F)) for c in range(D)] for i in range(M)]


@pytest.mark.parametrize("act", [ops.ACT_SILU, ops.ACT_GELU_ERF, ops.ACT_NONE])
def test_gated_mlp_fwd_vs_brute(act):
    g = np.random.default_rng(71 + act)
    M, D, F = 3, 5, 4
    x, wg, wu, wd = g.standard_normal((M, D)), g.standard_normal((D, F)), g.standard_normal((D, F)), \
        g.standard_normal((F, D))
    ref = np.array(_gated_brute(x.tolist(), wg.tolist(), wu.tolist(), wd.tolist(), act))
    got = ops.gated_mlp_fwd(x, wg, wu, wd, act)["P"]
    assert np.max(np.abs(got - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


def test_gated_mlp_special_cases():
    g = np.random.default_rng(73)
    M, D, F = 6, 7, 5
    x, wg, wd = g.standard_normal((M, D)), g.standard_normal((D, F)), g.standard_normal((F, D))
    # U == 1 (X's column 0 is all ones, W_up selects it): the gated MLP is the
    # plain MLP with the gate weight as its expansion, forward and backward
    x[:, 0] = 1.0
    wu = np.zeros((D, F))
    wu[0, :] = 1.0
    dy = g.standard_normal((M, D))
    for act in (ops.ACT_SILU, ops.ACT_GELU_ERF, ops.ACT_RELU):
        gf = ops.gated_mlp_fwd(x, wg, wu, wd, act)
        pf = ops.tp_mlp_fwd(x, wg, wd, act)
        assert np.array_equal(gf["U"], np.ones((M, F)))
        assert np.allclose(gf["P"], pf["P"], rtol=0, atol=1e-13)
        gb = ops.gated_mlp_bwd(x, wg, wu, wd, gf["G"], gf["U"], gf["H"], dy, act)
        pb = ops.tp_mlp_bwd(x, wg, wd, pf["Z"], pf["H"], dy, act)
        assert np.allclose(gb["dG"], pb["dZ"], rtol=0, atol=1e-13)
        assert np.allclose(gb["dW_gate"], pb["dW_up"], rtol=0, atol=1e-12)
        assert np.allclose(gb["dW_down"], pb["dW_down"], rtol=0, atol=1e-12)
    # no activation and W_gate == W_up: H = G^2 exactly
    f = ops.gated_mlp_fwd(x, wg, wg, wd, ops.ACT_NONE)
    assert np.array_equal(f["H"], f["G"] * f["G"])


def test_gated_sharded_equals_unsharded():
    # [WE]: gate and expansion column-partitioned, contraction row-partitioned;
    # the partials sum to the unsharded output, the shard gradients are the
    # blocks of the unsharded ones and the dX partials sum to the unsharded dX
    g = np.random.default_rng(75)
    M, D, F, T = 8, 12, 16, 4
    x, wg, wu, wd, dy = (g.standard_normal((M, D)), g.standard_normal((D, F)), g.standard_normal((D, F)),
                         g.standard_normal((F, D)), g.standard_normal((M, D)))
    full = ops.gated_mlp_fwd(x, wg, wu, wd, ops.ACT_SILU)
    fullb = ops.gated_mlp_bwd(x, wg, wu, wd, full["G"], full["U"], full["H"], dy, ops.ACT_SILU)
    P = np.zeros((M, D))
    dX = np.zeros((M, D))
    for t in range(T):
        wgt, wut, wdt = ops.col_block(wg, T, t), ops.col_block(wu, T, t), ops.row_block(wd, T, t)
        f = ops.gated_mlp_fwd(x, wgt, wut, wdt, ops.ACT_SILU)
        b = ops.gated_mlp_bwd(x, wgt, wut, wdt, f["G"], f["U"], f["H"], dy, ops.ACT_SILU)
        assert f["H"].shape == (M, F // T) and f["P"].shape == (M, D)
        P += f["P"]
        dX += b["dX"]
        assert np.allclose(b["dW_gate"], ops.col_block(fullb["dW_gate"], T, t), rtol=0, atol=1e-12)
        assert np.allclose(b["dW_up"], ops.col_block(fullb["dW_up"], T, t), rtol=0, atol=1e-12)
        assert np.allclose(b["dW_down"], ops.row_block(fullb["dW_down"], T, t), rtol=0, atol=1e-12)
    assert np.allclose(P, full["P"], rtol=0, atol=1e-12)
    assert np.allclose(dX, fullb["dX"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("act", [ops.ACT_SILU, ops.ACT_GELU_ERF])
def test_gated_gradients_by_finite_differences(act):
    # L = <Gm, P>, dP = Gm
    M, D, F = 4, 5, 3
    g = np.random.default_rng(77 + act)
    x, wg, wu, wd, Gm = (g.standard_normal((M, D)), g.standard_normal((D, F)) * 0.5,
                         g.standard_normal((D, F)) * 0.5, g.standard_normal((F, D)) * 0.5,
                         g.standard_normal((M, D)))
    f = ops.gated_mlp_fwd(x, wg, wu, wd, act)
    b = ops.gated_mlp_bwd(x, wg, wu, wd, f["G"], f["U"], f["H"], Gm, act)
    args = [x, wg, wu, wd]

    def loss(a):
        return float(np.sum(Gm * ops.gated_mlp_fwd(*a, act)["P"]))

    eps = 1e-6
    for k, grad in enumerate((b["dX"], b["dW_gate"], b["dW_up"], b["dW_down"])):
        fd = np.zeros_like(args[k])
        for idx in np.ndindex(args[k].shape):
            ap, am = list(args), list(args)
            ap[k], am[k] = args[k].copy(), args[k].copy()
            ap[k][idx] += eps
            am[k][idx] -= eps
            fd[idx] = (loss(ap) - loss(am)) / (2 * eps)
        assert np.max(np.abs(fd - grad)) <= 1e-7 * (1 + np.max(np.abs(grad))), k


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize("m,k,n", [(8, 32, 32), (37, 19, 23), (1, 1, 1), (5, 64, 3)])
def test_gemm_vs_brute(m, k, n):
    g = np.random.default_rng(m * 1000 + k)
    a = g.standard_normal((m, k))
    b = g.standard_normal((k, n))
    ref = np.array(brute.matmul(brute.to_lists(a), brute.to_lists(b)))
    assert np.max(np.abs(ops.gemm(a, b) - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))
    # transposed operands by index
    y, _ = ops.seq_chunk_gemm(np.ascontiguousarray(a.T), np.ascontiguousarray(b.T), trans_a=True, trans_b=True)
    assert np.max(np.abs(y - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_mlp_fwd_bwd_vs_brute(act):
    g = np.random.default_rng(11)
    M, D, Ft = 6, 10, 7
    x, wu, wd = g.standard_normal((M, D)), g.standard_normal((D, Ft)) * 0.3, g.standard_normal((Ft, D)) * 0.3
    dy = g.standard_normal((M, D))
    a = ops.ACT_RELU if act == "relu" else ops.ACT_GELU_ERF
    f = ops.tp_mlp_fwd(x, wu, wd, a)
    z, h, p = brute.mlp_fwd(brute.to_lists(x), brute.to_lists(wu), brute.to_lists(wd), act)
    assert np.allclose(f["P"], p, rtol=0, atol=1e-12)
    b = ops.tp_mlp_bwd(x, wu, wd, f["Z"], f["H"], dy, a)
    bb = brute.mlp_bwd(brute.to_lists(x), brute.to_lists(wu), brute.to_lists(wd), z, h, brute.to_lists(dy), act)
    for key in ("dW_down", "dW_up", "dX", "dZ"):
        assert np.allclose(b[key], bb[key], rtol=0, atol=1e-12), key


# ------------------------------------------------------ sharding invariants
def _rand_or_int(kind, shape, seed):
    g = np.random.default_rng(seed)
    return g.integers(-3, 4, size=shape).astype(np.float64) if kind == "int" else g.standard_normal(shape)


@pytest.mark.parametrize("kind", ["int", "float"])
def test_column_and_row_parallel_invariants(kind):
    M, K, N, T = 16, 24, 32, 4
    x = _rand_or_int(kind, (M, K), 1)
    w = _rand_or_int(kind, (K, N), 2)
    full = ops.gemm(x, w)
    tol = 0 if kind == "int" else 1e-12
    # I1 concat_t X W_t = X W
    cat = np.concatenate([ops.gemm(x, ops.col_block(w, T, t)) for t in range(T)], axis=1)
    assert np.max(np.abs(cat - full)) <= tol * (1 + np.max(np.abs(full)))
    # I2 sum_t X_t W_t = X W
    s = sum(ops.gemm(ops.col_block(x, T, t), ops.row_block(w, T, t)) for t in range(T))
    assert np.max(np.abs(s - full)) <= tol * (1 + np.max(np.abs(full)))
    # I8 concat_r reduce(r) = sum_t P_t (all-reduce = reduce-scatter + all-gather)
    parts = np.stack([_rand_or_int(kind, (M, N), 10 + t) for t in range(T)])
    cat = np.concatenate([ops.partial_reduce_seqshard(parts, r) for r in range(T)], axis=0)
    assert np.max(np.abs(cat - parts.sum(axis=0))) <= tol * (1 + np.max(np.abs(parts)))
    for r in range(T):
        assert ops.partial_reduce_seqshard(parts, r).shape == (M // T, N)


@pytest.mark.parametrize("act", [ops.ACT_RELU, ops.ACT_GELU_ERF])
def test_sharded_mlp_equals_unsharded(act):
    # I3-I7 on the page's own Megatron MLP shapes (8, 32, 128, 4)
    m, d, f, T = 8, 32, 128, 4
    g = np.random.default_rng(3)
    x, a, b = g.standard_normal((m, d)), g.standard_normal((d, f)) * 0.2, g.standard_normal((f, d)) * 0.2
    dy = g.standard_normal((m, d))
    un = ops.mlp_unsharded(x, a, b, act)
    unb = ops.mlp_unsharded_bwd(x, a, b, un["pre"], dy, act)
    P = []
    dX = np.zeros((m, d))
    for t in range(T):
        wu, wd = ops.col_block(a, T, t), ops.row_block(b, T, t)
        fw = ops.tp_mlp_fwd(x, wu, wd, act)
        P.append(fw["P"])
        bw = ops.tp_mlp_bwd(x, wu, wd, fw["Z"], fw["H"], dy, act)
        assert bw["dW_up"].shape == wu.shape and bw["dW_down"].shape == wd.shape      # I7
        assert bw["dX"].shape == (m, d)                                              # full partial
        assert np.allclose(bw["dW_up"], ops.col_block(unb["dA"], T, t), atol=1e-12)  # I4
        assert np.allclose(bw["dW_down"], ops.row_block(unb["dB"], T, t), atol=1e-12)  # I6
        dX += bw["dX"]
    assert np.allclose(sum(P), un["Y"], atol=1e-12)                                  # I3
    assert np.allclose(dX, unb["dX"], atol=1e-12)                                    # I5


@pytest.mark.parametrize("act", [ops.ACT_GELU_ERF, ops.ACT_GELU_TANH, ops.ACT_RELU])
def test_gradients_by_finite_differences(act):
    # I10: L = <G, P>; dP = G; gradients must be derivatives of L
    M, D, Ft = 5, 6, 4
    g = np.random.default_rng(21)
    x, wu, wd, G = (g.standard_normal((M, D)), g.standard_normal((D, Ft)) * 0.5,
                    g.standard_normal((Ft, D)) * 0.5, g.standard_normal((M, D)))
    if act == ops.ACT_RELU:  # stay away from the kink
        z = x @ wu
        assert np.min(np.abs(z)) > 1e-3
    fw = ops.tp_mlp_fwd(x, wu, wd, act)
    bw = ops.tp_mlp_bwd(x, wu, wd, fw["Z"], fw["H"], G, act)

    def loss(x_, wu_, wd_):
        return float(np.sum(G * ops.tp_mlp_fwd(x_, wu_, wd_, act)["P"]))

    eps = 1e-6
    for name, arr, grad in (("X", x, bw["dX"]), ("Wup", wu, bw["dW_up"]), ("Wdown", wd, bw["dW_down"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            args_p = [x, wu, wd]
            args_m = [x, wu, wd]
            k = {"X": 0, "Wup": 1, "Wdown": 2}[name]
            args_p[k], args_m[k] = ap, am
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(fd - grad)) <= 1e-7 * (1 + np.max(np.abs(grad))), name


def test_page3_checker_reproduced():
    # P1: the page's generator with seeds 1,2,3 and its three asserts
    c = si.c1_tiny_mlp("page3")
    m, d, f, T = c["m"], c["d"], c["f"], c["t"]
    gold = GOLDEN["megatron_mlp_checker"]
    assert (m, d, f, T) == (gold["m"], gold["d"], gold["f"], gold["t"])
    x, a, b = (c[k].astype(np.float64) for k in ("x", "a", "b"))
    assert x[0, 0] == np.float32(0.001) - np.float32(0.5)    # (0*2654435761 + 1) % 1000 = 1
    un = ops.mlp_unsharded(x, a, b, ops.ACT_RELU)
    parts, pre, dx_parts = [], [], []
    for t in range(T):
        fw = ops.tp_mlp_fwd(x, ops.col_block(a, T, t), ops.row_block(b, T, t), ops.ACT_RELU)
        parts.append(fw["P"])
        pre.append(fw["Z"])
    y = sum(parts)
    close = lambda u, v: np.all(np.abs(u - v) < gold["rtol"] * (1 + np.abs(v)))
    assert close(y, un["Y"])
    dy = y.copy()                              # loss 1/2 ||Y||^2
    unb = ops.mlp_unsharded_bwd(x, a, b, un["pre"], dy, ops.ACT_RELU)
    for t in range(T):
        bw = ops.tp_mlp_bwd(x, ops.col_block(a, T, t), ops.row_block(b, T, t), pre[t],
                            ops.relu(pre[t]), dy, ops.ACT_RELU)
        assert close(bw["dW_up"], ops.col_block(unb["dA"], T, t))
        dx_parts.append(bw["dX"])
    assert close(sum(dx_parts), unb["dX"])


def test_special_cases():
    g = np.random.default_rng(2)
    x = g.standard_normal((8, 8))
    w = g.standard_normal((8, 8))
    eye = np.eye(8)
    assert np.array_equal(ops.gemm(eye, w), w)                       # X = I -> Y = W
    f = ops.tp_mlp_fwd(x, w, eye, ops.ACT_NONE)                      # W_down = I -> P = H
    assert np.allclose(f["P"], f["H"], atol=1e-14)
    parts = g.standard_normal((1, 8, 8))
    assert np.array_equal(ops.partial_reduce_seqshard(parts, 0), parts[0])   # T = 1
    y, _ = ops.seq_chunk_gemm(x, w, chunk_rows=2, chunk_order=[3, 0, 2, 1])
    assert np.array_equal(y, ops.gemm(x, w))                         # order-free


def test_fp8_mirror_error_bound_and_scale_direction():
    g = np.random.default_rng(4)
    M, D, Ft = 16, 64, 32
    xq, sx = si.to_e4m3_current(g.standard_normal((M, D)).astype(np.float32))
    wuq, su = si.to_e4m3_current((g.standard_normal((D, Ft)) * 0.02).astype(np.float32))
    wdq, sd = si.to_e4m3_current((g.standard_normal((Ft, D)) * 0.02).astype(np.float32))
    X, WU, WD = (formats.e4m3_to_f64(q.numpy()) for q in (xq, wuq, wdq))
    r = ops.tp_mlp_fwd_fp8(X, sx, WU, su, WD, sd, ops.ACT_GELU_ERF)
    # the largest |H_b| maps to the largest finite code
    assert np.max(np.abs(formats.e4m3_to_f64(r["Hq_codes"]))) == 448.0
    deq = formats.e4m3_to_f64(r["Hq_codes"]) * r["sH"]
    # e4m3 nearest rounding: half an ulp (2^-4 relative) in the normal range,
    # half the subnormal spacing (2^-10 * sH) below it
    assert np.all(np.abs(deq - r["Hb"]) <= 2.0 ** -4 * np.abs(r["Hb"]) * (1 + 1e-6) + 2.0 ** -10 * r["sH"] * 1.001)
    exact = ops.tp_mlp_fwd(X * sx, WU * su, WD * sd, ops.ACT_GELU_ERF)
    # the quantised path stays close to the exact layer in the normalised measure
    assert ops.normalized_error(r["P"], exact["P"]) < 0.06
    # amax does not depend on order
    assert r["amax"] == float(np.max(np.abs(r["Hb"][::-1])))


# --------------------------------------------- pages' printed numbers (golden)
def test_fig3_schedule_numbers():
    gold = GOLDEN["fig3_boundary_units"]
    n = gold["chunks"]
    assert schedule.serial(n) == gold["serial"]
    assert schedule.allgather_gemm(n) == gold["allgather_overlapped"]
    assert schedule.gemm_reducescatter(n) == gold["reducescatter_overlapped"]
    # the target is max(compute, comm) per boundary ("Choosing the chunk count")
    assert schedule.allgather_gemm(16, c=1.0, m=0.5) == 16.0


def test_shapes_and_payloads_from_pages():
    o = GOLDEN["column_parallel_opening_example"]
    cp = shapes.column_parallel(o["M"], o["K"], o["N"], o["T"])
    assert list(cp["W_t"]) == o["W_t"] and list(cp["Y_t"]) == o["Y_t"]
    w = GOLDEN["mlp_pair_worked_example"]
    up = shapes.column_parallel(w["M"], w["D"], w["F"], w["T"])
    down = shapes.row_parallel(w["M"], w["F"], w["D"], w["T"])
    assert list(up["W_t"]) == w["expansion_shard"] and list(up["Y_t"]) == w["intermediate"]
    assert list(down["W_t"]) == w["contraction_shard"] and list(down["Y_t"]) == w["partial"]
    pb = shapes.partial_payload_bytes(w["M"], w["D"])
    assert pb == w["payload_bytes"] and round(pb / 1e6, 1) == w["payload_MB_printed"]
    assert w["F"] // 8 == w["F_shard_at_T8"]
    c = GOLDEN["allreduce_cost_example"]
    ar = 2 * c["b"] * c["s"] * c["h"]
    assert ar == c["bytes"] and round(ar / 1e6) == c["MB_printed"]


def test_chunk_and_range_orders():
    assert si.ring_chunk_order(4, 4, 0) == [0, 3, 2, 1]
    assert si.ring_chunk_order(8, 8, 0) == [0, 7, 6, 5, 4, 3, 2, 1]
    o = si.ring_chunk_order(8, 16, 0)
    assert o[:4] == [0, 1, 14, 15] and o[-2:] == [2, 3] and sorted(o) == list(range(16))
    assert si.dest_range_order(8, 0) == [1, 2, 3, 4, 5, 6, 7, 0]


def test_store_bf16_rounds_only_the_consumed_intermediate():
    g = np.random.default_rng(8)
    M, D, Ft = 16, 32, 24
    # integer-valued activations are exact in bf16: rounding them changes nothing
    x = g.integers(-3, 4, size=(M, D)).astype(np.float64)
    wu = g.integers(-2, 3, size=(D, Ft)).astype(np.float64)
    wd = g.integers(-2, 3, size=(Ft, D)).astype(np.float64)
    a = ops.tp_mlp_fwd(x, wu, wd, ops.ACT_RELU, store="bf16")
    b = ops.tp_mlp_fwd(x, wu, wd, ops.ACT_RELU)
    assert np.array_equal(a["P"], b["P"]) and np.array_equal(a["H"], b["H"])
    # general values: P is the product of the rounded H, and Z/H are unrounded
    x = g.standard_normal((M, D))
    a = ops.tp_mlp_fwd(x, wu * 0.1, wd * 0.1, ops.ACT_GELU_ERF, store="bf16")
    assert np.array_equal(a["P"], formats.round_bf16(a["H"]) @ (wd * 0.1))
    assert np.array_equal(a["Z"], x @ (wu * 0.1))
    dy = g.standard_normal((M, D))
    r = ops.tp_mlp_bwd(x, wu, wd, a["Z"], a["H"], dy, ops.ACT_GELU_ERF, store="bf16")
    assert np.array_equal(r["dW_up"], x.T @ formats.round_bf16(r["dZ"]))
    assert np.array_equal(r["dW_down"], a["H"].T @ dy)


def test_linear_bwd_by_finite_differences_and_brute_force():
    # O8 pinned: the gradients of L = <G, X.W> (forward by correctly rounded
    # brute force) in X and W, and the two products against brute force
    M, K, N = 5, 7, 3
    g = np.random.default_rng(31)
    x, w, G = g.standard_normal((M, K)), g.standard_normal((K, N)), g.standard_normal((M, N))
    bw = ops.linear_bwd(x, w, G)
    assert bw["dW"].shape == w.shape and bw["dX"].shape == x.shape                   # I7

    def loss(x_, w_):
        y = np.array(brute.matmul(brute.to_lists(x_), brute.to_lists(w_)))
        return float(np.sum(G * y))

    eps = 1e-6
    for name, arr, grad in (("X", x, bw["dX"]), ("W", w, bw["dW"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            fd[idx] = ((loss(ap, w) - loss(am, w)) if name == "X" else (loss(x, ap) - loss(x, am))) / (2 * eps)
        assert np.max(np.abs(fd - grad)) <= 1e-7 * (1 + np.max(np.abs(grad))), name
    tl = brute.to_lists
    assert np.allclose(bw["dW"], brute.matmul(brute.transpose(tl(x)), tl(G)), rtol=1e-13, atol=1e-13)
    assert np.allclose(bw["dX"], brute.matmul(tl(G), brute.transpose(tl(w))), rtol=1e-13, atol=1e-13)


def test_linear_bwd_shard_invariants():
    # I4/I5 for a column-parallel layer (W split by columns, dY_t its columns):
    # dW_t is column block t of the unsharded dW, and the dX_t sum to the
    # unsharded dX; I6 for a row-parallel layer (W split by rows, X_t the
    # matching columns of X, dY whole): dW_t is row block t and dX_t is
    # column block t of the unsharded gradients.  Integer inputs: exact.
    M, K, N, T = 6, 8, 12, 4
    g = np.random.default_rng(32)
    x = g.integers(-3, 4, (M, K)).astype(np.float64)
    w = g.integers(-3, 4, (K, N)).astype(np.float64)
    dy = g.integers(-3, 4, (M, N)).astype(np.float64)
    un = ops.linear_bwd(x, w, dy)
    dx_sum = np.zeros_like(x)
    for t in range(T):
        b = ops.linear_bwd(x, ops.col_block(w, T, t), ops.col_block(dy, T, t))
        assert np.array_equal(b["dW"], ops.col_block(un["dW"], T, t))
        dx_sum += b["dX"]
    assert np.array_equal(dx_sum, un["dX"])
    for t in range(T):
        b = ops.linear_bwd(ops.col_block(x, T, t), ops.row_block(w, T, t), dy)
        assert np.array_equal(b["dW"], ops.row_block(un["dW"], T, t))
        assert np.array_equal(b["dX"], ops.col_block(un["dX"], T, t))
