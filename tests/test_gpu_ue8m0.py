"""Power-of-two (UE8M0) scales on the GPU against the CPU oracle.

Quantizers: codes bit-exact and every fp32 scale exactly 2^(byte - 127) of the
oracle's E8M0 byte.  GEMMs: the matrix core applies the scales and chains the
fp32 accumulator through its C input, so the acceptance bound is the in-block
truncation bound plus fp32 rounding of 16 sub-group additions per block, plus
half a bf16 ulp for BF16 outputs."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import (model_dgrad, model_fprop, model_grouped_rows, model_grouped_wgrad, model_wgrad)
from parity import (assert_codes_equal, assert_scales_equal, bf16_dev, bf16_host_f64, check_gemm, f32_dev,
                    host, hw_bound_dgrad, hw_bound_fprop, hw_bound_wgrad, sample_idx, u8_dev)
from test_gpu_quant import SMALL, stress

pytestmark = pytest.mark.gpu
T = 128
SUBGROUPS = 16     # fp32 additions per 128-block when the accumulator is chained through C


def dec_scales(orc, e):
    return orc.e8m0_decode(e).astype(np.float32)


@pytest.mark.parametrize("R,C", SMALL)
def test_quantizers_small(orc, R, C):
    x = stress(R, C, 7000 + R * 7 + C)
    xd = bf16_dev(x)
    oq, oe = orc.quantize_1x128_ue8m0(x)
    oqT, oeT = orc.quantize_128x1_ue8m0(x)
    q, s = fgb.quantize_1x128(xd, ue8m0=True)
    assert_codes_equal(q, oq, f"ue8m0 q[{R}x{C}]")
    assert_scales_equal(s, dec_scales(orc, oe), f"ue8m0 s[{R}x{C}]")
    qT, sT = fgb.quantize_128x1(xd, ue8m0=True)
    assert_codes_equal(qT, oqT, f"ue8m0 qT[{R}x{C}]")
    assert_scales_equal(sT, dec_scales(orc, oeT), f"ue8m0 sT[{R}x{C}]")
    dq, ds, dqT, dsT = fgb.quantize_dual(xd, ue8m0=True)
    assert_codes_equal(dq, oq, "ue8m0 dual q")
    assert_scales_equal(ds, dec_scales(orc, oe), "ue8m0 dual s")
    assert_codes_equal(dqT, oqT, "ue8m0 dual qT")
    assert_scales_equal(dsT, dec_scales(orc, oeT), "ue8m0 dual sT")
    rq, rs = fgb.requant_128x1(q, s, ue8m0=True)
    orq, ore = orc.requant_128x1_ue8m0(oq, oe)
    assert_codes_equal(rq, orq, "ue8m0 requant qT")
    assert_scales_equal(rs, dec_scales(orc, ore), "ue8m0 requant sT")


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384)])
def test_quantize_128x128_small(orc, K, N):
    w = stress(K, N, 8000 + K + N)
    q, qT, s = fgb.quantize_128x128(bf16_dev(w), ue8m0=True)
    oq, oqT, oe = orc.quantize_128x128_ue8m0(w)
    assert_codes_equal(q, oq, "ue8m0 w q")
    assert_codes_equal(qT, oqT, "ue8m0 w qT")
    assert_scales_equal(s, dec_scales(orc, oe), "ue8m0 w s")


def test_amax_floor(orc):
    x = stress(130, 256, 5)
    for fl in (1e-4, 3.0):
        q, s = fgb.quantize_1x128(bf16_dev(x), amax_floor=fl, ue8m0=True)
        oq, oe = orc.quantize_1x128_ue8m0(x, amax_floor=fl)
        assert_codes_equal(q, oq, f"ue8m0 q floor {fl}")
        assert_scales_equal(s, dec_scales(orc, oe), f"ue8m0 s floor {fl}")


def test_quant_stress_full(orc):
    """Quant-stress workload [16384, 7168]: every tiling with power-of-two scales."""
    d = wl.quant_stress()
    x = d["x"]
    xd = bf16_dev(x)
    q, s, qT, sT = fgb.quantize_dual(xd, ue8m0=True)
    oq, oe = orc.quantize_1x128_ue8m0(x)
    assert_codes_equal(q, oq, "stress ue8m0 q")
    assert_scales_equal(s, dec_scales(orc, oe), "stress ue8m0 s")
    oqT, oeT = orc.quantize_128x1_ue8m0(x)
    assert_codes_equal(qT, oqT, "stress ue8m0 qT")
    assert_scales_equal(sT, dec_scales(orc, oeT), "stress ue8m0 sT")
    del qT, sT, oqT, oeT
    rq, rs = fgb.requant_128x1(q, s, ue8m0=True)
    orq, ore = orc.requant_128x1_ue8m0(oq, oe)
    assert_codes_equal(rq, orq, "stress ue8m0 requant")
    assert_scales_equal(rs, dec_scales(orc, ore), "stress ue8m0 requant s")
    del rq, rs, orq, ore
    w, wT, ws = fgb.quantize_128x128(xd, ue8m0=True)
    ow, owT, oe = orc.quantize_128x128_ue8m0(x)
    assert_codes_equal(w, ow, "stress ue8m0 w")
    assert_codes_equal(wT, owT, "stress ue8m0 wT")
    assert_scales_equal(ws, dec_scales(orc, oe), "stress ue8m0 ws")


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def rand_codes(g, shape):
    c = g.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C
    return c


def po2_scales(g, shape):
    return np.exp2(g.integers(-12, 4, shape)).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 384, 640), (1, 128, 128), (300, 896, 256),
                                   (700, 1792, 384)])
def test_fprop_small(orc, M, N, K):
    g = np.random.default_rng(M * 31 + N * 7 + K + 1)
    qx, qwT = rand_codes(g, (M, K)), rand_codes(g, (N, K))
    sx, sw = po2_scales(g, (K // T, M)), po2_scales(g, (K // T, N // T))
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw), ue8m0=True)
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw)
    check_gemm(bf16_host_f64(y), r, aabs, True, f"ue8m0 fprop {M}x{N}x{K}", hw_bound_fprop(qx, sx, qwT, sw),
               SUBGROUPS * (K // T), stated=False)


@pytest.mark.parametrize("M,K,N", [(300, 384, 640), (200, 256, 1152), (333, 896, 384)])
def test_dgrad_small(orc, M, K, N):
    g = np.random.default_rng(M * 13 + N * 5 + K + 1)
    qdy, qw = rand_codes(g, (M, N)), rand_codes(g, (K, N))
    sdy, sw = po2_scales(g, (N // T, M)), po2_scales(g, (K // T, N // T))
    dx = fgb.gemm_dgrad(u8_dev(qdy), f32_dev(sdy), u8_dev(qw), f32_dev(sw), ue8m0=True)
    r, aabs = orc.gemm_dgrad(qdy, sdy, qw, sw)
    check_gemm(bf16_host_f64(dx), r, aabs, True, f"ue8m0 dgrad {M}x{K}x{N}", hw_bound_dgrad(qdy, sdy, qw, sw),
               SUBGROUPS * (N // T), stated=False)


@pytest.mark.parametrize("K,N,M", [(256, 384, 300), (128, 128, 1), (384, 256, 1024), (256, 896, 300),
                                   (896, 896, 200)])
def test_wgrad_small(orc, K, N, M):
    g = np.random.default_rng(K * 3 + N * 11 + M + 1)
    Mp = -(-M // T) * T
    qxT, qdyT = rand_codes(g, (K, Mp)), rand_codes(g, (N, Mp))
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    nb = Mp // T
    sxT, sdyT = po2_scales(g, (nb, K)), po2_scales(g, (nb, N))
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M, ue8m0=True)
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M)
    hw = hw_bound_wgrad(qxT, sxT, qdyT, sdyT, M)
    check_gemm(host(dw), r, aabs, False, f"ue8m0 wgrad {K}x{N}x{M}", hw, SUBGROUPS * nb, stated=False)
    prev = g.standard_normal((K, N)).astype(np.float32)
    dw2 = f32_dev(prev)
    fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M, dw=dw2, accumulate=True, ue8m0=True)
    check_gemm(host(dw2), r + prev, aabs + np.abs(prev), False, "ue8m0 wgrad accumulate", hw, SUBGROUPS * nb + 1, stated=False)


SMALL_INT_CODES = np.array([0x00, 0x80, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8, 0x4C, 0xCC, 0x50, 0xD0],
                           np.uint8)   # 0, -0, +-1, +-2, +-3, +-4, +-6, +-8


def test_exact_small_integers_all_kinds(orc):
    """Products that are small integers times powers of two lose nothing in the
    matrix core, and every partial sum here is exact in fp32: the outputs must
    equal the exact result (rounded once to bf16 for Fprop/Dgrad)."""
    g = np.random.default_rng(11)
    M, N, K = 300, 384, 512
    qx, qwT = g.choice(SMALL_INT_CODES, (M, K)), g.choice(SMALL_INT_CODES, (N, K))
    sx, sw = np.exp2(g.integers(-3, 3, (K // T, M))).astype(np.float32), np.exp2(g.integers(-3, 3, (K // T, N // T))).astype(np.float32)
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw), ue8m0=True)
    r, _ = orc.gemm_fprop(qx, sx, qwT, sw)
    assert np.all(np.abs(r) < 2.0 ** 24)
    assert np.array_equal(host(y.view(torch.int16)).view(np.uint16), orc.bf16_round(r))
    qxT, qdyT = g.choice(SMALL_INT_CODES, (K, M + 84)), g.choice(SMALL_INT_CODES, (N, M + 84))
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    sxT, sdyT = np.exp2(g.integers(-3, 3, (3, K))).astype(np.float32), np.exp2(g.integers(-3, 3, (3, N))).astype(np.float32)
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M, ue8m0=True)
    r, _ = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M)
    assert np.array_equal(host(dw).astype(np.float64), r)


def test_accumulator_chain_is_fp32():
    """Wgrad over two 128-blocks: block 0 contributes 2^16 (one product 256 * 256),
    block 1 small terms.  Chained through the matrix core's C input, the small
    terms survive exactly as in an fp32 add (2^16 + 1 is exact), and beyond fp32
    precision they round to nearest even, not truncate (2^24 + 3 -> 2^24 + 4)."""
    K, N, M = 128, 128, 256
    qxT = np.zeros((K, M), np.uint8)
    qdyT = np.zeros((N, M), np.uint8)
    qxT[:, 0] = 0x78           # 256
    qdyT[:, 0] = 0x78          # 256 -> product 2^16 in block 0
    qxT[:, 128] = 0x38         # 1
    qdyT[:, 128] = 0x38        # 1 -> product 1 in block 1
    s1 = np.ones((2, K), np.float32)
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(s1), u8_dev(qdyT), f32_dev(np.ones((2, N), np.float32)), M, ue8m0=True)
    assert np.all(host(dw) == 65537.0)
    # block 0 = 2^24 (scale 2^8 on 2^16), block 1 = 3: fp32 round-to-nearest-even gives 2^24 + 4
    sxT = np.ones((2, K), np.float32)
    sxT[0] = 256.0
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(np.where(qdyT == 0x38, 0x44, qdyT).astype(np.uint8)),
                        f32_dev(np.ones((2, N), np.float32)), M, ue8m0=True)
    assert np.all(host(dw) == 2.0 ** 24 + 4.0)


def test_grouped_small(orc):
    from test_gpu_grouped import grouped_inputs, offsets_dev
    loads = np.array([130, 0, 1, 256, 70])
    K, N = 256, 384
    offsets, x, dy, ws = grouped_inputs(loads, K, N, 77)
    od = offsets_dev(offsets)
    qx, sx = fgb.quantize_1x128(bf16_dev(x), ue8m0=True)
    qs = [fgb.quantize_128x128(bf16_dev(w), ue8m0=True) for w in ws]
    qw, qwT, sw = (torch.stack([q[k] for q in qs]) for k in range(3))
    y = fgb.gemm_fprop_grouped(od, qx, sx, qwT, sw, ue8m0=True)
    qdy, sdy, qdyT, sdyT = fgb.quantize_dual(bf16_dev(dy), ue8m0=True)
    dx = fgb.gemm_dgrad_grouped(od, qdy, sdy, qw, sw, ue8m0=True)
    qxT, sxT = fgb.requant_128x1(qx, sx, ue8m0=True)
    dw = fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT, ue8m0=True)
    torch.cuda.synchronize()
    oqx, oex = orc.quantize_1x128_ue8m0(x)
    assert_codes_equal(qx, oqx, "grouped ue8m0 qx")
    osx = dec_scales(orc, oex)
    owq = [orc.quantize_128x128_ue8m0(w) for w in ws]
    oqw = np.stack([o[0] for o in owq]); oqwT = np.stack([o[1] for o in owq])
    osw = np.stack([dec_scales(orc, o[2]) for o in owq])
    oqdy, oedy = orc.quantize_1x128_ue8m0(dy)
    osdy = dec_scales(orc, oedy)
    oqxT, oexT = orc.requant_128x1_ue8m0(oqx, oex)
    oqdyT, oedyT = orc.quantize_128x1_ue8m0(dy)
    osxT, osdyT = dec_scales(orc, oexT), dec_scales(orc, oedyT)
    R = int(offsets[-1])
    hwf, hwd = np.zeros((R, N)), np.zeros((R, K))
    hww = np.zeros((len(loads), K, N))
    for e in range(len(loads)):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            hwf[a:b] = hw_bound_fprop(oqx[a:b], osx[:, a:b], oqwT[e], osw[e])
            hwd[a:b] = hw_bound_dgrad(oqdy[a:b], osdy[:, a:b], oqw[e], osw[e])
            hww[e] = hw_bound_wgrad(oqxT[:, a:b], osxT[a // T:b // T], oqdyT[:, a:b], osdyT[a // T:b // T], b - a)
    r, aabs = orc.gemm_fprop_grouped(offsets, oqx, osx, oqwT, osw)
    check_gemm(bf16_host_f64(y), r, aabs, True, "ue8m0 fprop grouped", hwf, SUBGROUPS * (K // T),
               model=model_grouped_rows(offsets, model_fprop, oqx, osx, oqwT, osw), po2=True)
    r, aabs = orc.gemm_dgrad_grouped(offsets, oqdy, osdy, oqw, osw)
    check_gemm(bf16_host_f64(dx), r, aabs, True, "ue8m0 dgrad grouped", hwd, SUBGROUPS * (N // T),
               model=model_grouped_rows(offsets, model_dgrad, oqdy, osdy, oqw, osw), po2=True)
    r, aabs = orc.gemm_wgrad_grouped(offsets, oqxT, osxT, oqdyT, osdyT)
    check_gemm(host(dw).reshape(r.shape), r, aabs, False, "ue8m0 wgrad grouped", hww, SUBGROUPS * 2,
               model=model_grouped_wgrad(offsets, oqxT, osxT, oqdyT, osdyT), po2=True)


def test_linear_dsv3_attn_sampled(orc):
    """The DeepSeek-V3 attention-projection linear with power-of-two scales:
    quantizers bit-exact on the full tensors, GEMMs on sampled outputs."""
    d = wl.linear_dsv3_attn()
    M, K, N = d["M"], d["K"], d["N"]
    qx, sx = fgb.quantize_1x128(bf16_dev(d["x"]), ue8m0=True)
    qw, qwT, sw = fgb.quantize_128x128(bf16_dev(d["w"]), ue8m0=True)
    qdy, sdy, qdyT, sdyT = fgb.quantize_dual(bf16_dev(d["dy"]), ue8m0=True)
    qxT, sxT = fgb.requant_128x1(qx, sx, ue8m0=True)
    y = fgb.gemm_fprop(qx, sx, qwT, sw, ue8m0=True)
    dx = fgb.gemm_dgrad(qdy, sdy, qw, sw, ue8m0=True)
    dw = fgb.gemm_wgrad(qxT, sxT, qdyT, sdyT, M, ue8m0=True)
    torch.cuda.synchronize()
    oqx, oex = orc.quantize_1x128_ue8m0(d["x"])
    oqw, oqwT, oew = orc.quantize_128x128_ue8m0(d["w"])
    oqdy, oedy = orc.quantize_1x128_ue8m0(d["dy"])
    oqdyT, oedyT = orc.quantize_128x1_ue8m0(d["dy"])
    oqxT, oexT = orc.requant_128x1_ue8m0(oqx, oex)
    for got, want, name in [(qx, oqx, "qx"), (qwT, oqwT, "qwT"), (qdy, oqdy, "qdy"), (qdyT, oqdyT, "qdyT"),
                            (qxT, oqxT, "qxT")]:
        assert_codes_equal(got, want, f"dsv3 ue8m0 {name}")
    osx, osw, osdy = dec_scales(orc, oex), dec_scales(orc, oew), dec_scales(orc, oedy)
    osxT, osdyT = dec_scales(orc, oexT), dec_scales(orc, oedyT)
    for got, want, name in [(sx, osx, "sx"), (sw, osw, "sw"), (sdy, osdy, "sdy"), (sxT, osxT, "sxT"),
                            (sdyT, osdyT, "sdyT")]:
        assert_scales_equal(got, want, f"dsv3 ue8m0 {name}")
    rows, cols = sample_idx(M, 40, 1), sample_idx(N, 40, 2)
    r, aabs = orc.gemm_fprop(oqx, osx, oqwT, osw, rows, cols)
    check_gemm(bf16_host_f64(y)[np.ix_(rows, cols)], r, aabs, True, "dsv3 ue8m0 fprop",
               hw_bound_fprop(oqx, osx, oqwT, osw, rows, cols), SUBGROUPS * (K // T),
               model=model_fprop(oqx, osx, oqwT, osw, rows, cols), po2=True)
    colsK = sample_idx(K, 40, 3)
    r, aabs = orc.gemm_dgrad(oqdy, osdy, oqw, osw, rows, colsK)
    check_gemm(bf16_host_f64(dx)[np.ix_(rows, colsK)], r, aabs, True, "dsv3 ue8m0 dgrad",
               hw_bound_dgrad(oqdy, osdy, oqw, osw, rows, colsK), SUBGROUPS * (N // T),
               model=model_dgrad(oqdy, osdy, oqw, osw, rows, colsK), po2=True)
    wr, wc = sample_idx(K, 40, 4), sample_idx(N, 40, 5)
    r, aabs = orc.gemm_wgrad(oqxT, osxT, oqdyT, osdyT, M, wr, wc)
    check_gemm(host(dw)[np.ix_(wr, wc)], r, aabs, False, "dsv3 ue8m0 wgrad",
               hw_bound_wgrad(oqxT, osxT, oqdyT, osdyT, M, wr, wc), SUBGROUPS * (M // T),
               model=model_wgrad(oqxT, osxT, oqdyT, osdyT, M, wr, wc), po2=True)
