"""Non-finite inputs through every quantizer, GPU against the oracle.

NaN: a tile holding a NaN gets a NaN scale (the quiet NaN; E8M0 byte 0xFF for
power-of-two scales) and the code 0x7F for every element, so the NaN reaches
every GEMM output the tile feeds; all other tiles are quantized as usual.
Codes and scale bit patterns must equal the oracle's everywhere.

Inf: the tile's absmax is Inf, so its scale is Inf and its multiplier 448/Inf
= 0: finite elements become +-0 and the infinite element itself becomes
Inf * 0, a NaN (whose sign IEEE arithmetic leaves open) encoded as 0x7F.
Codes and scales must equal the oracle's everywhere.

Padding: the 128x1 outputs' padding rows stay 0x00 inside a NaN tile."""
import numpy as np
import pytest

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import assert_codes_equal, assert_scales_equal, bf16_dev, host

pytestmark = pytest.mark.gpu

R, C = 300, 384


def base(seed):
    g = np.random.default_rng(seed)
    return wl.bf16_bits(g.standard_normal((R, C)).astype(np.float32))


def with_nans():
    x = base(1)
    x[5, 130] = 0x7FC0          # quiet NaN
    x[200, 7] = 0xFFC1          # negative NaN with a payload
    x[299, 383] = 0x7F81        # signalling-pattern NaN, last (ragged) row tile
    x[140, 256:384] = 0x7FC0    # a whole 1x128 tile of NaN
    return x


def with_infs():
    x = base(2)
    x[6, 131] = 0x7F80          # +Inf
    x[201, 8] = 0xFF80          # -Inf
    x[298, 380] = 0x7F80
    return x


def inf_positions(x):
    return np.argwhere((x & 0x7FFF) == 0x7F80)


def check_inf_codes(got, want, pos_codes, name):
    """Codes equal everywhere; the infinite elements (given as (row, col) of the
    code array) hold the NaN code 0x7F on both sides."""
    g = host(got)
    for r, c in pos_codes:
        assert want[r, c] == 0x7F, f"{name}: oracle code {want[r, c]:#04x} at ({r},{c})"
    assert_codes_equal(got, want, name)


def test_nan_tiles_round_to_nearest(orc):
    x = with_nans()
    xd = bf16_dev(x)
    q, s = fgb.quantize_1x128(xd)
    oq, os_ = orc.quantize_1x128(x)
    assert np.isnan(os_[1, 5]) and np.all(oq[5, 128:256] == 0x7F)
    assert_codes_equal(q, oq, "nan q")
    assert_scales_equal(s, os_, "nan s")
    qT, sT = fgb.quantize_128x1(xd)
    oqT, osT = orc.quantize_128x1(x)
    assert np.all(oqT[383, 300:] == 0) and np.all(oqT[383, 256:300] == 0x7F)     # NaN tile, zero padding
    assert_codes_equal(qT, oqT, "nan qT")
    assert_scales_equal(sT, osT, "nan sT")
    q2, s2, qT2, sT2 = fgb.quantize_dual(xd)
    assert_codes_equal(q2, oq, "nan dual q")
    assert_scales_equal(s2, os_, "nan dual s")
    assert_codes_equal(qT2, oqT, "nan dual qT")
    assert_scales_equal(sT2, osT, "nan dual sT")
    w = x[:256, :384].copy()
    qw, qwT, sw = fgb.quantize_128x128(bf16_dev(w))
    oqw, oqwT, osw = orc.quantize_128x128(w)
    assert_codes_equal(qw, oqw, "nan qw")
    assert_codes_equal(qwT, oqwT, "nan qwT")
    assert_scales_equal(sw, osw, "nan sw")
    rq, rs = fgb.requant_128x1(q, s)
    orq, ors = orc.requant_128x1(oq, os_)
    assert_codes_equal(rq, orq, "nan requant qT")
    assert_scales_equal(rs, ors, "nan requant sT")


def test_nan_tiles_power_of_two_and_sr(orc):
    x = with_nans()
    xd = bf16_dev(x)
    q, s = fgb.quantize_1x128(xd, ue8m0=True)
    oq, oe = orc.quantize_1x128_ue8m0(x)
    assert_codes_equal(q, oq, "nan ue8m0 q")
    assert_scales_equal(s, orc.e8m0_decode(oe).astype(np.float32), "nan ue8m0 s")
    qT, sT = fgb.quantize_128x1(xd, ue8m0=True)
    oqT, oeT = orc.quantize_128x1_ue8m0(x)
    assert_codes_equal(qT, oqT, "nan ue8m0 qT")
    assert_scales_equal(sT, orc.e8m0_decode(oeT).astype(np.float32), "nan ue8m0 sT")
    qs, ss = fgb.quantize_1x128(xd, sr=(11, 3))
    oqs, oss = orc.quantize_1x128_sr(x, 11, 3)
    assert_codes_equal(qs, oqs, "nan sr q")
    assert_scales_equal(ss, oss, "nan sr s")
    qsT, ssT = fgb.quantize_128x1(xd, sr=(11, 3))
    oqsT, ossT = orc.quantize_128x1_sr(x, 11, 3)
    assert_codes_equal(qsT, oqsT, "nan sr qT")
    assert_scales_equal(ssT, ossT, "nan sr sT")


def test_nan_reaches_gemm(orc):
    """A NaN tile of X makes exactly the Fprop outputs of its row NaN."""
    x = with_nans()[:256, :256].copy()
    g = np.random.default_rng(5)
    w = wl.bf16_bits(g.standard_normal((256, 128)).astype(np.float32) * 0.02)
    qx, sx = fgb.quantize_1x128(bf16_dev(x))
    _, qwT, sw = fgb.quantize_128x128(bf16_dev(w))
    y = host(fgb.gemm_fprop(qx, sx, qwT, sw).float())
    nan_rows = {5, 200}
    for r in range(256):
        if r in nan_rows:
            assert np.all(np.isnan(y[r])), r
        else:
            assert not np.any(np.isnan(y[r])), r


def test_inf_tiles(orc):
    x = with_infs()
    xd = bf16_dev(x)
    pos = inf_positions(x)
    q, s = fgb.quantize_1x128(xd)
    oq, os_ = orc.quantize_1x128(x)
    assert np.isinf(os_[1, 6])
    check_inf_codes(q, oq, pos, "inf q")
    assert_scales_equal(s, os_, "inf s")
    qT, sT = fgb.quantize_128x1(xd)
    oqT, osT = orc.quantize_128x1(x)
    check_inf_codes(qT, oqT, pos[:, ::-1], "inf qT")
    assert_scales_equal(sT, osT, "inf sT")
    q2, s2, qT2, sT2 = fgb.quantize_dual(xd)
    check_inf_codes(q2, oq, pos, "inf dual q")
    check_inf_codes(qT2, oqT, pos[:, ::-1], "inf dual qT")
    assert_scales_equal(s2, os_, "inf dual s")
    assert_scales_equal(sT2, osT, "inf dual sT")
    w = x[:256, :384].copy()
    pw = inf_positions(w)
    qw, qwT, sw = fgb.quantize_128x128(bf16_dev(w))
    oqw, oqwT, osw = orc.quantize_128x128(w)
    check_inf_codes(qw, oqw, pw, "inf qw")
    check_inf_codes(qwT, oqwT, pw[:, ::-1], "inf qwT")
    assert_scales_equal(sw, osw, "inf sw")
    qs, ss = fgb.quantize_1x128(xd, sr=(7, 1))
    oqs, oss = orc.quantize_1x128_sr(x, 7, 1)
    check_inf_codes(qs, oqs, pos, "inf sr q")
    assert_scales_equal(ss, oss, "inf sr s")
    qe, se = fgb.quantize_1x128(xd, ue8m0=True)
    oqe, oe = orc.quantize_1x128_ue8m0(x)
    assert_codes_equal(qe, oqe, "inf ue8m0 q")       # power of two: Inf * 2^-127 saturates, no NaN
    assert_scales_equal(se, orc.e8m0_decode(oe).astype(np.float32), "inf ue8m0 s")
