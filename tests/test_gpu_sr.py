"""GPU stochastic-rounding quantizers against the CPU oracle: the same seed and
salt must give identical codes and scale bit patterns (padding included).
Small ragged shapes with every value class (signed zeros, zero tiles, tiny
negatives, bf16 subnormals -- the E4M3-subnormal branch of the cast), then the
full quant-stress and linear workloads."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import assert_codes_equal, assert_scales_equal, bf16_dev, host
from test_gpu_quant import stress

pytestmark = pytest.mark.gpu

SMALL = [(1, 128), (3, 8), (130, 200), (64, 384), (257, 136), (128, 128), (5, 1024)]
KEYS = [(0, 0), (0x0123456789ABCDEF, 7), (2 ** 64 - 1, 2 ** 32 - 1)]


@pytest.mark.parametrize("R,C", SMALL)
@pytest.mark.parametrize("seed,salt", KEYS)
def test_sr_1x128_128x1_dual_small(orc, R, C, seed, salt):
    x = stress(R, C, 4000 + R * 7 + C)
    xd = bf16_dev(x)
    q, s = fgb.quantize_1x128(xd, sr=(seed, salt))
    oq, os_ = orc.quantize_1x128_sr(x, seed, salt)
    assert_codes_equal(q, oq, f"sr q[{R}x{C}]")
    assert_scales_equal(s, os_, f"sr s[{R}x{C}]")
    qT, sT = fgb.quantize_128x1(xd, sr=(seed, salt))
    oqT, osT = orc.quantize_128x1_sr(x, seed, salt)
    assert_codes_equal(qT, oqT, f"sr qT[{R}x{C}]")
    assert_scales_equal(sT, osT, f"sr sT[{R}x{C}]")
    dq, ds, dqT, dsT = fgb.quantize_dual(xd, sr=(seed, salt))
    assert_codes_equal(dq, oq, f"sr dual q[{R}x{C}]")
    assert_scales_equal(ds, os_, f"sr dual s[{R}x{C}]")
    assert_codes_equal(dqT, oqT, f"sr dual qT[{R}x{C}]")
    assert_scales_equal(dsT, osT, f"sr dual sT[{R}x{C}]")


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384), (384, 128)])
@pytest.mark.parametrize("seed,salt", KEYS)
def test_sr_128x128_small(orc, K, N, seed, salt):
    w = stress(K, N, 5000 + K + N)
    q, qT, s = fgb.quantize_128x128(bf16_dev(w), sr=(seed, salt))
    oq, oqT, os_ = orc.quantize_128x128_sr(w, seed, salt)
    assert_codes_equal(q, oq, f"sr w q[{K}x{N}]")
    assert_codes_equal(qT, oqT, f"sr w qT[{K}x{N}]")
    assert_scales_equal(s, os_, f"sr w s[{K}x{N}]")
    q2, qT2, _ = fgb.quantize_128x128(bf16_dev(w), want_q=False, sr=(seed, salt))
    assert q2 is None
    assert_codes_equal(qT2, oqT, "sr w qT only")


def test_sr_amax_floor(orc):
    x = stress(200, 256, 77)
    q, s = fgb.quantize_1x128(bf16_dev(x), amax_floor=1e-3, sr=(5, 6))
    oq, os_ = orc.quantize_1x128_sr(x, 5, 6, amax_floor=1e-3)
    assert_codes_equal(q, oq, "sr floor q")
    assert_scales_equal(s, os_, "sr floor s")


def test_sr_deterministic_and_keyed():
    x = bf16_dev(stress(256, 512, 9))
    a = host(fgb.quantize_1x128(x, sr=(11, 3))[0])
    b = host(fgb.quantize_1x128(x, sr=(11, 3))[0])
    assert np.array_equal(a, b)
    assert not np.array_equal(a, host(fgb.quantize_1x128(x, sr=(12, 3))[0]))
    assert not np.array_equal(a, host(fgb.quantize_1x128(x, sr=(11, 4))[0]))
    assert not np.array_equal(a, host(fgb.quantize_1x128(x, sr=(11 + 2 ** 32, 3))[0]))


def test_sr_quant_stress_full(orc):
    """Workload 5 ([16384, 7168], values from 1e-6 to 1e3, zeros, tiny negatives,
    bf16 subnormals): all four SR quantizers, bit-exact."""
    d = wl.quant_stress()
    x = d["x"]
    xd = bf16_dev(x)
    seed, salt = 0x9E3779B97F4A7C15, 0xA5A5
    q, s = fgb.quantize_1x128(xd, sr=(seed, salt))
    oq, os_ = orc.quantize_1x128_sr(x, seed, salt)
    assert_codes_equal(q, oq, "stress sr 1x128 q")
    assert_scales_equal(s, os_, "stress sr 1x128 s")
    qT, sT = fgb.quantize_128x1(xd, sr=(seed, salt))
    oqT, osT = orc.quantize_128x1_sr(x, seed, salt)
    assert_codes_equal(qT, oqT, "stress sr 128x1 qT")
    assert_scales_equal(sT, osT, "stress sr 128x1 sT")
    dq, ds, dqT, dsT = fgb.quantize_dual(xd, sr=(seed, salt))
    assert_codes_equal(dq, oq, "stress sr dual q")
    assert_codes_equal(dqT, oqT, "stress sr dual qT")
    del q, s, qT, sT, dq, ds, dqT, dsT, oqT, osT
    qw, qwT, sw = fgb.quantize_128x128(xd, sr=(seed, salt))
    oqw, oqwT, osw = orc.quantize_128x128_sr(x, seed, salt)
    assert_codes_equal(qw, oqw, "stress sr 128x128 q")
    assert_codes_equal(qwT, oqwT, "stress sr 128x128 qT")
    assert_scales_equal(sw, osw, "stress sr 128x128 s")


def test_sr_linear_workload_full(orc):
    """Workload 2 operands with SR: X 1x128, dY dual, W 128x128; and every SR code
    is one of the two grid neighbours of the round-to-nearest code's value."""
    d = wl.linear_dsv3_attn()
    seed = 20260101
    q, s = fgb.quantize_1x128(bf16_dev(d["x"]), sr=(seed, 1))
    oq, os_ = orc.quantize_1x128_sr(d["x"], seed, 1)
    assert_codes_equal(q, oq, "x sr 1x128")
    assert_scales_equal(s, os_, "x sr 1x128 s")
    rq = host(fgb.quantize_1x128(bf16_dev(d["x"]))[0])
    step = np.abs((host(q).astype(np.int16) & 0x7F) - (rq.astype(np.int16) & 0x7F))
    assert int(step.max()) <= 1
    dq, ds, dqT, dsT = fgb.quantize_dual(bf16_dev(d["dy"]), sr=(seed, 2))
    oq, os_ = orc.quantize_1x128_sr(d["dy"], seed, 2)
    oqT, osT = orc.quantize_128x1_sr(d["dy"], seed, 2)
    assert_codes_equal(dq, oq, "dy sr dual 1x128")
    assert_codes_equal(dqT, oqT, "dy sr dual 128x1")
    assert_scales_equal(dsT, osT, "dy sr dual 128x1 s")
    q, qT, s = fgb.quantize_128x128(bf16_dev(d["w"]), sr=(seed, 3))
    oq, oqT, os_ = orc.quantize_128x128_sr(d["w"], seed, 3)
    assert_codes_equal(q, oq, "w sr q")
    assert_codes_equal(qT, oqT, "w sr qT")
    assert_scales_equal(s, os_, "w sr s")
