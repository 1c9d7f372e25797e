"""Pins of the oracle's SwiGLU with fused casts (CPU only).

The pages ("scratch: the backward pass, unrolled", section "What is asserted,
and from where") fix: the SwiGLU input is saved as E4M3, the forward emits the
next GEMM's E4M3 operand, the backward emits both tile orientations and computes
in BF16 from the dequantized E4M3 input.  Readings pinned here: H is the exact
silu(G)*U rounded once to BF16; the backward dequantizes G~ = bf16(fl32(dec*s)),
and dG = bf16(dH*U~*silu'(G~)), dU = bf16(dH*silu(G~)) with one rounding each.

The pins use torch's float64 silu and its float64 autograd derivative (library
routines), an exact double-to-bf16 rounding built from torch's float32 cast
(round-to-odd to float32 first), and torch's float8/float32 arithmetic for the
dequantization -- none of them the oracle's code.  Exhaustive over every finite
BF16 gate value.
"""
import numpy as np
import pytest
import torch

from fine_grained_block_amd import workloads as wl

T = 128


def round_to_odd_f32(x):
    t = x.astype(np.float32)
    back = t.astype(np.float64)
    inexact = back != x
    over = np.abs(back) > np.abs(x)
    t = np.where(inexact & over, np.nextafter(t, np.float32(0)), t)
    return (t.view(np.uint32) | inexact.astype(np.uint32)).view(np.float32)


def bf16_exact(x64):
    """float64 -> bf16 bits, one RNE rounding (round-to-odd float32 + torch's RNE cast)."""
    return torch.from_numpy(round_to_odd_f32(np.asarray(x64, np.float64))).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


def torch_silu(g64):
    return torch.nn.functional.silu(torch.from_numpy(g64)).numpy()


def torch_dsilu(g64):
    t = torch.from_numpy(g64.copy()).requires_grad_(True)
    torch.nn.functional.silu(t).sum().backward()
    return t.grad.numpy()


# Where a float64 value sits within float64 error of a bf16 rounding midpoint, the
# rounding is decided in decimal arithmetic (Python's decimal module) with enough
# digits to resolve 1 - sigma(g) ~ e^-g.
import decimal


def _ctx(g):
    digits = 60 + (int(abs(float(g)) / 2.302585) + 10 if g > 0 else 0)
    return decimal.Context(prec=digits, Emin=-10 ** 7, Emax=10 ** 7, traps=[])


def _sigma_dec(C, g):
    gd = C.create_decimal(float(g))
    if gd >= 0:
        return C.divide(1, C.add(1, C.exp(-gd)))
    e = C.exp(gd)
    return C.divide(e, C.add(1, e))


def _dec_value(C, kind, g, factor):
    gd = C.create_decimal(float(g))
    sig = _sigma_dec(C, g)
    if kind == "silu":
        f = C.multiply(gd, sig)
    else:
        f = C.multiply(sig, C.add(1, C.multiply(gd, C.subtract(1, sig))))
    return C.multiply(f, C.create_decimal(float(factor)))


def _bf16_of_decimal(C, v):
    """RNE of a decimal to bf16 bits (finite, within the bf16 range)."""
    if v == 0:
        return 0x8000 if v.is_signed() else 0
    sign = 0x8000 if v < 0 else 0
    a = v.copy_abs()                                      # exact (abs() would round to 28 digits)
    two = C.create_decimal(2)
    e = int(C.divide(a.ln(C), two.ln(C)).to_integral_value(decimal.ROUND_FLOOR))
    while C.power(two, e) > a:
        e -= 1
    while C.power(two, e + 1) <= a:
        e += 1
    e = max(e, -126)
    m = int(C.divide(a, C.power(two, e - 7)).to_integral_value(decimal.ROUND_HALF_EVEN))
    val = np.float32(np.ldexp(np.float64(m), e - 7))
    return sign | (int(val.view(np.uint32)) >> 16)


def bf16_of_product(kind, g64, factor64):
    """bf16 bits of silu(g)*factor (kind "silu") or silu'(g)*factor ("dsilu"), one RNE
    rounding of the exact value."""
    base = torch_silu(g64) if kind == "silu" else torch_dsilu(g64)
    x = base * factor64
    out = bf16_exact(x)
    ax = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        e = np.maximum(e, -126)
        ulp = np.exp2(e - 7)
        frac = ax / ulp - np.floor(ax / ulp)
    near = (ax > 0) & (np.abs(frac - 0.5) < 1e-9)
    for i in np.nonzero(near)[0]:
        g, f = float(g64[i]), float(factor64[i])
        if g <= 5000.0:
            C = _ctx(g)
            out[i] = _bf16_of_decimal(C, _dec_value(C, kind, g, f))
        else:
            # g > 5000: silu(g) and silu'(g) differ from g and 1 by less than e^-4000
            # relative; sigma(g) < 1 puts silu(g)*f strictly inside |g f| and
            # g (1 - sigma) > 1 - sigma puts silu'(g)*f strictly outside |f|, which
            # decides a tie of the exact product
            C = decimal.Context(prec=60, traps=[])
            base = C.create_decimal(g * f if kind == "silu" else f)
            nudge = C.create_decimal("-1e-40" if kind == "silu" else "1e-40")
            out[i] = _bf16_of_decimal(C, C.multiply(base, C.add(1, nudge)))
    return out


def test_forward_every_finite_gate_unit_up(orc):
    g = all_finite_bf16()
    gu = np.concatenate([g[None, :], np.full((1, g.size), 0x3F80, np.uint16)], axis=1)    # U = 1
    h = orc.swiglu_h(gu)[0]
    want = bf16_of_product("silu", bf16_f64(g), np.ones(g.size))
    assert np.array_equal(h, want), int((h != want).sum())


def test_forward_every_finite_gate_random_up(orc):
    g = all_finite_bf16()
    rng = np.random.default_rng(3)
    u = wl.bf16_bits((rng.standard_normal(g.size) * np.exp(rng.uniform(-20, 20, g.size))).astype(np.float32))
    h = orc.swiglu_h(np.concatenate([g[None, :], u[None, :]], axis=1))[0]
    exact = torch_silu(bf16_f64(g)) * bf16_f64(u)
    fin = np.abs(exact) < 3.0e38                          # beyond, bf16 overflows (not an input domain)
    assert fin.mean() > 0.9
    want = bf16_of_product("silu", bf16_f64(g)[fin], bf16_f64(u)[fin])
    assert np.array_equal(h[fin], want), int((h[fin] != want).sum())


def test_forward_layout_gate_then_up(orc):
    """G is the first F columns, U the last F, row by row."""
    rng = np.random.default_rng(4)
    R, F = 3, 256
    gu = wl.bf16_bits(rng.standard_normal((R, 2 * F)).astype(np.float32))
    h = orc.swiglu_h(gu)
    want = bf16_of_product("silu", bf16_f64(gu[:, :F]).ravel(), bf16_f64(gu[:, F:]).ravel()).reshape(R, F)
    assert np.array_equal(h, want)


def dequant_bf16(q, s, F):
    """G~, U~ by torch: float8 decode times the fp32 scale in float32, then bf16."""
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    R = q.shape[0]
    sc = torch.from_numpy(np.repeat(s.T, T, axis=1)[:, :2 * F].copy())
    v = (dec * sc).to(torch.bfloat16).to(torch.float64).numpy()
    return v[:, :F], v[:, F:]


def test_backward_quantized_random_stash(orc):
    """Every finite bf16 value as a dequantized gate: the stash is built so that
    dequantization is exact (unit scales, codes on the grid) for a sweep of
    gates, plus quantized random data for the general rule."""
    rng = np.random.default_rng(5)
    R, F = 512, 256
    gu = wl.bf16_bits((rng.standard_normal((R, 2 * F)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32))
    q, s = orc.quantize_1x128(gu)
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    dgu = orc.swiglu_dgu(q, s, dh)
    g, u = dequant_bf16(q, s, F)
    d = bf16_f64(dh)
    assert np.array_equal(dgu[:, :F], bf16_of_product("dsilu", g.ravel(), (d * u).ravel()).reshape(R, F))
    assert np.array_equal(dgu[:, F:], bf16_of_product("silu", g.ravel(), d.ravel()).reshape(R, F))


def test_backward_derivative_all_gates(orc):
    """silu' at every finite bf16 gate against torch's float64 autograd: scales 1 and
    U~ = 1 make G~ any bf16 value that E4M3 holds; the rest come through dU/dG with
    a scale that carries them (each 1x128 tile holds one gate and a 448 for scale 1)."""
    g_all = all_finite_bf16()
    gf = bf16_f64(g_all)
    # the dequantized gate is fl32(dec * s): choose per-row scales s = g / dec(code) exactly
    # representable: take code 0x38 (1.0) and s = g (fp32 holds every bf16 value)
    R = g_all.size
    F = 128
    q = np.zeros((R, 2 * F), np.uint8)
    q[:, 0] = 0x38                                        # gate = 1.0 * s_g
    q[:, F] = 0x38                                        # up = 1.0 * s_u
    s = np.zeros((2, R), np.float32)
    s[0] = gf.astype(np.float32)
    s[1] = 1.0
    dh = np.full((R, F), 0x3F80, np.uint16)               # dH = 1
    dgu = orc.swiglu_dgu(q, s, dh)
    assert np.array_equal(dgu[:, 0], bf16_of_product("dsilu", gf, np.ones(R)))
    assert np.array_equal(dgu[:, F], bf16_of_product("silu", gf, np.ones(R)))
    # columns whose stash codes are 0 give (signed) zero gates: silu(+-0) = +-0, and
    # U~ = 0 there, so dG = dH * 0 * 1/2; both come out as zeros of either sign
    assert np.all((dgu[:, F + 1:] & 0x7FFF) == 0)
    assert np.all((dgu[:, 1:F] & 0x7FFF) == 0)


def test_fused_forms_are_the_quantizers_of_the_bf16_tensors(orc):
    rng = np.random.default_rng(6)
    R, F = 130, 384
    gu = wl.bf16_bits(rng.standard_normal((R, 2 * F)).astype(np.float32))
    q_gu, s_gu, q_h, s_h, h = orc.swiglu_fwd_quant(gu)
    assert np.array_equal(q_gu, orc.quantize_1x128(gu)[0])
    assert np.array_equal(q_h, orc.quantize_1x128(h)[0])
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    dgu, q, s, qT, sT = orc.swiglu_bwd_quant(q_gu, s_gu, dh)
    assert np.array_equal(qT, orc.quantize_128x1(dgu)[0])


def test_zero_gate_keeps_ties_to_even(orc):
    """silu'(0) = 1/2 exactly, so dG = bf16(dH * U~ / 2) rounds an exact tie to even:
    dH = 9, U~ = 29 gives 130.5 -> 130 and dH = 3, U~ = 89 gives 133.5 -> 134;
    dU = dH * silu(0) = 0."""
    R, F = 2, 128
    q = np.zeros((R, 2 * F), np.uint8)
    q[:, F] = 0x38                                        # up = 1.0 * 29
    s = np.zeros((2, R), np.float32)
    s[0] = 1.0
    s[1] = [29.0, 89.0]
    dh = np.zeros((R, F), np.uint16)
    dh[:, 0] = [0x4110, 0x4040]                           # 9.0, 3.0
    dgu = orc.swiglu_dgu(q, s, dh)
    assert list(dgu[:, 0]) == [0x4302, 0x4306]            # 130.0, 134.0
    assert np.all((dgu[:, F] & 0x7FFF) == 0)


@pytest.mark.parametrize("zero", [0x0000, 0x8000])
def test_zero_products_take_the_ieee_sign(orc, zero):
    """A product with a zero factor is a zero whose sign is the product's, as
    float64 arithmetic in torch gives it: H = silu(g) * (+-0) at every finite
    gate; in the backward dU = dH * silu(G~) and dG = dH * U~ * silu'(G~) with
    dH = +-0 (torch's float64 silu and autograd derivative)."""
    z = -0.0 if zero == 0x8000 else 0.0
    g_all = all_finite_bf16()
    gf = bf16_f64(g_all)
    F = 128
    n = g_all.size - g_all.size % F
    gu = np.concatenate([g_all[:n].reshape(-1, F), np.full((n // F, F), zero, np.uint16)], axis=1)
    h = orc.swiglu_h(gu).reshape(-1)
    assert np.array_equal(h, bf16_exact(torch_silu(gf[:n]) * z))
    R = g_all.size
    q = np.zeros((R, 2 * F), np.uint8)
    q[:, 0] = 0x38
    q[:, F] = 0x38
    s = np.zeros((2, R), np.float32)
    s[0] = gf.astype(np.float32)
    s[1] = 1.0
    dh = np.full((R, F), zero, np.uint16)
    dgu = orc.swiglu_dgu(q, s, dh)
    assert np.array_equal(dgu[:, 0], bf16_exact(torch_dsilu(gf) * 1.0 * z))
    assert np.array_equal(dgu[:, F], bf16_exact(torch_silu(gf) * z))
