"""Second stage of the two-stage weight cast on the GPU against the CPU oracle:
a 128x128 E4M3 weight with fp32 tile scales (made by the oracle's first stage)
requantized to power-of-two tiles.  Codes bit-exact in both layouts, every
scale exactly 2^(byte - 127) of the oracle's E8M0 byte."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import assert_codes_equal, assert_scales_equal, f32_dev, u8_dev
from test_gpu_quant import stress

pytestmark = pytest.mark.gpu
T = 128


def first_stage(orc, K, N, seed, amax_floor=0.0):
    w = stress(K, N, seed)
    q, _, s = orc.quantize_128x128(w, amax_floor)
    return q, s


def check(orc, q, s, amax_floor, name, want_q=True, want_qT=True):
    oq2, oq2T, oe = orc.requant_128x128_ue8m0(q, s, amax_floor)
    q2, q2T, s2 = fgb.requant_128x128_ue8m0(u8_dev(q), f32_dev(s), amax_floor, want_q=want_q, want_qT=want_qT)
    if want_q:
        assert_codes_equal(q2, oq2, name + " q2")
    else:
        assert q2 is None
    if want_qT:
        assert_codes_equal(q2T, oq2T, name + " q2T")
    else:
        assert q2T is None
    assert_scales_equal(s2, orc.e8m0_decode(oe).astype(np.float32), name + " s2")


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384), (640, 128), (128, 1152)])
def test_two_stage_small(orc, K, N):
    q, s = first_stage(orc, K, N, 9100 + K + N)
    check(orc, q, s, 0.0, f"two-stage {K}x{N}")


def test_two_stage_one_layout_only(orc):
    q, s = first_stage(orc, 256, 256, 9200)
    check(orc, q, s, 0.0, "q2 only", want_qT=False)
    check(orc, q, s, 0.0, "q2T only", want_q=False)


def test_two_stage_floors_and_zero_tiles(orc):
    """Zero tiles and tiles far below the floors: the pages' minimum power-of-two
    scales 2^-42 (amax floor 1e-10) and 2^-33 (floor 448 * 2^-33)."""
    q, s = first_stage(orc, 256, 384, 9300)
    q[:128, :128] = 0                                   # an all-zero tile
    q[128:, 128:256] = np.where(q[128:, 128:256] & 0x7F, 0x01, 0)   # tiny codes ...
    s[1, 1] = np.float32(2.0 ** -40)                    # ... at a tiny scale
    for floor in (0.0, 1e-10, 448.0 * 2.0 ** -33):
        check(orc, q, s, floor, f"floor {floor}")


def test_two_stage_strided(orc):
    """Operands inside wider allocations (ld > width)."""
    K, N = 256, 256
    q, s = first_stage(orc, K, N, 9400)
    dev = torch.device("cuda:0")
    qbig = torch.zeros((K, N + 64), dtype=torch.uint8, device=dev)
    qbig[:, :N] = u8_dev(q)
    q2big = torch.full((K, N + 32), 0x55, dtype=torch.uint8, device=dev)
    q2Tbig = torch.full((N, K + 48), 0x55, dtype=torch.uint8, device=dev)
    s2 = torch.empty((K // T, N // T), dtype=torch.float32, device=dev)
    fgb.requant_128x128_ue8m0(qbig[:, :N], f32_dev(s), q2=q2big[:, :N], q2T=q2Tbig[:, :K], s2=s2)
    oq2, oq2T, oe = orc.requant_128x128_ue8m0(q, s)
    assert_codes_equal(q2big[:, :N], oq2, "strided q2")
    assert_codes_equal(q2Tbig[:, :K], oq2T, "strided q2T")
    assert bool((q2big[:, N:] == 0x55).all()) and bool((q2Tbig[:, K:] == 0x55).all())
    assert_scales_equal(s2, orc.e8m0_decode(oe).astype(np.float32), "strided s2")


def test_two_stage_dsv3_weight(orc):
    """The DeepSeek-V3 attention projection's weight [7168, 7168], first stage
    with the weight amax floor 1e-4 of the pages' conventions."""
    w = wl.normal_bf16((7168, 7168), 0.02, 9500, 0)
    q, _, s = orc.quantize_128x128(w, 1e-4)
    check(orc, q, s, 0.0, "dsv3 W")
