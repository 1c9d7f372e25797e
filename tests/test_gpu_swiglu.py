"""GPU SwiGLU with fused casts against the CPU oracle: H, [dG | dU], every code
and every scale bit pattern identical (padding included).  Every finite bf16
gate value is covered in both directions (which exercises the fp32 fast path,
the fp64 fallback near bf16 rounding midpoints, tiny gates whose g*u/2 ties are
broken by the tanh correction, and gates beyond |g| = 80), then ragged shapes
and one GPU's share of the MoE expert tensors."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import assert_codes_equal, assert_scales_equal, bf16_dev, f32_dev, host, u8_dev

pytestmark = pytest.mark.gpu
T = 128


def finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


def bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def check_fwd(orc, gu, name, floor=0.0):
    q_gu, s_gu, q_h, s_h, h = fgb.swiglu_fwd_quant(bf16_dev(gu), amax_floor=floor, want_h=True)
    oq_gu, os_gu, oq_h, os_h, oh = orc.swiglu_fwd_quant(gu, amax_floor=floor)
    hb = bits(h)
    if not np.array_equal(hb, oh):
        bad = np.argwhere(hb != oh)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} H values differ; first at {i}: gpu {hb[i]:#06x} oracle {oh[i]:#06x}")
    assert_codes_equal(q_h, oq_h, f"{name} q_h")
    assert_scales_equal(s_h, os_h, f"{name} s_h")
    assert_codes_equal(q_gu, oq_gu, f"{name} q_gu")
    assert_scales_equal(s_gu, os_gu, f"{name} s_gu")
    return oq_gu, os_gu                                  # the backward's inputs come from the oracle


def check_bwd(orc, q_gu, s_gu, dh, name, floor=0.0):
    q, s, qT, sT, dgu = fgb.swiglu_bwd_quant(u8_dev(q_gu), f32_dev(s_gu), bf16_dev(dh), amax_floor=floor,
                                             want_dgu=True)
    odgu, oq, os_, oqT, osT = orc.swiglu_bwd_quant(q_gu, s_gu, dh, amax_floor=floor)
    db = bits(dgu)
    if not np.array_equal(db, odgu):
        bad = np.argwhere(db != odgu)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} dG/dU values differ; first at {i}: "
                             f"gpu {db[i]:#06x} oracle {odgu[i]:#06x}")
    assert_codes_equal(q, oq, f"{name} q")
    assert_scales_equal(s, os_, f"{name} s")
    assert_codes_equal(qT, oqT, f"{name} qT")
    assert_scales_equal(sT, osT, f"{name} sT")


def test_forward_every_finite_gate(orc):
    g = finite_bf16()                                   # 65280 values = 255 rows of 256
    F = 256
    G = g.reshape(-1, F)
    rng = np.random.default_rng(1)
    for name, U in [("u=1", np.full_like(G, 0x3F80)),
                    ("u random", wl.bf16_bits((rng.standard_normal(G.shape) *
                                               np.exp(rng.uniform(-8, 8, G.shape))).astype(np.float32))),
                    ("u=+0", np.zeros_like(G)), ("u=-0", np.full_like(G, 0x8000))]:
        gu = np.concatenate([G, U], axis=1)
        # keep H finite: drop rows whose |g*u| could overflow bf16
        gf = torch.from_numpy(G.view(np.int16)).view(torch.bfloat16).float().numpy()
        uf = torch.from_numpy(U.view(np.int16)).view(torch.bfloat16).float().numpy()
        ok = np.all(np.abs(gf.astype(np.float64) * uf) < 1e38, axis=1)
        check_fwd(orc, np.ascontiguousarray(gu[ok]), f"fwd every gate {name}")


def test_backward_every_finite_gate(orc):
    """Stash codes 1.0 with per-row scales equal to every finite bf16 value make G~
    take each of them; U~ = 1 or 37, dH = 1, random, +0 or -0."""
    g = finite_bf16()
    gf = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).float().numpy()
    R, F = g.size, 128
    q = np.zeros((R, 2 * F), np.uint8)
    q[:, :] = 0x38
    s = np.zeros((2, R), np.float32)
    s[0] = gf
    s[1] = 37.0
    rng = np.random.default_rng(2)
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    dh[:, 0] = 0x3F80
    check_bwd(orc, q, s, dh, "bwd every gate")
    # zero products keep their sign: dH = +0 and -0 at every gate
    for zero in (0x0000, 0x8000):
        check_bwd(orc, q, s, np.full((R, F), zero, np.uint16), f"bwd every gate, dH = {zero:#06x}")


def test_backward_zero_gate_ties():
    """silu'(0) = 1/2: dH*U~/2 = 130.5 -> 130 and 133.5 -> 134 (ties to even)."""
    R, F = 2, 128
    q = np.zeros((R, 2 * F), np.uint8)
    q[:, F] = 0x38
    s = np.zeros((2, R), np.float32)
    s[0] = 1.0
    s[1] = [29.0, 89.0]
    dh = np.zeros((R, F), np.uint16)
    dh[:, 0] = [0x4110, 0x4040]
    *_, dgu = fgb.swiglu_bwd_quant(u8_dev(q), f32_dev(s), bf16_dev(dh), want_dgu=True)
    assert list(bits(dgu)[:, 0]) == [0x4302, 0x4306]


@pytest.mark.parametrize("R,F", [(1, 128), (3, 256), (130, 128), (257, 384), (64, 1024)])
def test_ragged_round_trip(orc, R, F):
    rng = np.random.default_rng(R * 7 + F)
    gu = wl.bf16_bits((rng.standard_normal((R, 2 * F)) * np.exp(rng.uniform(-3, 3, (R, 1)))).astype(np.float32))
    gu[:, :3] = 0
    gu[0, 5] = 0x8000                                   # -0 gate
    q_gu, s_gu = check_fwd(orc, gu, f"fwd {R}x{F}")
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    check_bwd(orc, q_gu, s_gu, dh, f"bwd {R}x{F}")


@pytest.mark.parametrize("floor", [1e-4, 3.0])
def test_amax_floor(orc, floor):
    """The fused casts with an absmax floor: rows of magnitude 10^U(-6, 1), so that
    some tiles of [G | U], H and [dG | dU] lie below the floor and others above."""
    rng = np.random.default_rng(31)
    R, F = 257, 256
    gu = wl.bf16_bits((rng.standard_normal((R, 2 * F)) * np.power(10.0, rng.uniform(-6, 1, (R, 1)))).astype(np.float32))
    q_gu, s_gu = check_fwd(orc, gu, f"fwd floor {floor}", floor)
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * np.power(10.0, rng.uniform(-4, 2, (R, 1)))).astype(np.float32))
    check_bwd(orc, q_gu, s_gu, dh, f"bwd floor {floor}", floor)


def test_stash_optional_and_strided(orc):
    rng = np.random.default_rng(9)
    R, F = 200, 256
    big = wl.bf16_bits(rng.standard_normal((R, 2 * F + 64)).astype(np.float32))
    gu = big[:, :2 * F]
    gud = bf16_dev(big)[:, :2 * F]
    q_gu, s_gu, q_h, s_h, h = fgb.swiglu_fwd_quant(gud, stash=False)
    assert q_gu is None and s_gu is None and h is None
    _, _, oq_h, os_h, _ = orc.swiglu_fwd_quant(gu)
    assert_codes_equal(q_h, oq_h, "strided q_h")
    assert_scales_equal(s_h, os_h, "strided s_h")


def test_moe_share(orc):
    """One GPU's MoE gate/up output, 8192 routed rows x [2048 | 2048], heavy-tailed
    gates; forward then backward with dH ~ N(0, 1e-3)."""
    rng = np.random.default_rng(4)
    R, F = 8192, 2048
    gu = wl.bf16_bits((rng.standard_t(3, (R, 2 * F)) * 2.0).astype(np.float32))
    q_gu, s_gu = check_fwd(orc, gu, "moe fwd")
    dh = wl.bf16_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    check_bwd(orc, q_gu, s_gu, dh, "moe bwd")


def wide_table():
    """bf16 bit patterns of 16 magnitude decades x 4096 Gaussian quantiles (and
    +-0): a uniformly drawn 16-bit index maps to a value of mixed magnitude."""
    from scipy.special import ndtri
    z = ndtri((np.arange(4096) + 0.5) / 4096.0)
    t = (z[None, :] * np.power(10.0, np.linspace(-3.0, 1.0, 16))[:, None]).ravel().astype(np.float32)
    t[0], t[1] = 0.0, -0.0
    return wl.bf16_bits(t)


def test_beyond_2g_elements(orc):
    """[G | U] of 270001 x [4096 | 4096] (2.2e9 elements, 4.4 GB of bf16) forward,
    then the backward with dH [270001, 4096]: bit-exact against the oracle on
    sampled rows (H and the stashes) and on 128-row blocks (both orientations of
    [dG | dU]) -- the row that holds element 2^31 of [G | U], its neighbours, the
    ragged last block.  The backward's inputs are the oracle's stash."""
    rng = np.random.default_rng(77)
    R, F = 270001, 4096
    assert R * 2 * F > (1 << 31)
    table = wide_table()
    print(f"generating {R * 3 * F * 2 / 1e9:.2f} GB of bf16 inputs", flush=True)
    gu = np.empty((R, 2 * F), np.uint16)
    dh = np.empty((R, F), np.uint16)
    for r0 in range(0, R, 1 << 13):
        n = min(1 << 13, R - r0)
        gu[r0:r0 + n] = table[rng.integers(0, 1 << 16, (n, 2 * F), dtype=np.uint16)]
        dh[r0:r0 + n] = table[rng.integers(0, 1 << 16, (n, F), dtype=np.uint16)]
    rb = (1 << 31) // (2 * F)                          # the row that holds element 2^31 of [G | U]
    rows = np.unique(np.concatenate([[0, 1, rb - 1, rb, rb + 1, R - 2, R - 1], rng.choice(R, 24, replace=False)]))
    blocks = sorted({0, rb // T, (R - 1) // T, *rng.choice(R // T, 2, replace=False).tolist()})

    gud = bf16_dev(gu)
    q_gu, s_gu, q_h, s_h, h = fgb.swiglu_fwd_quant(gud, want_h=True)
    del gud
    ri = torch.as_tensor(rows, device=q_gu.device)
    oq_gu, os_gu, oq_h, os_h, oh = orc.swiglu_fwd_quant(gu[rows])
    assert np.array_equal(bits(h[ri]), oh), "H differs on sampled rows"
    assert_codes_equal(q_h[ri], oq_h, "q_h beyond 2^31")
    assert_scales_equal(s_h[:, ri], os_h, "s_h beyond 2^31")
    assert_codes_equal(q_gu[ri], oq_gu, "q_gu beyond 2^31")
    assert_scales_equal(s_gu[:, ri], os_gu, "s_gu beyond 2^31")
    del q_h, s_h, h

    # the backward on the GPU's stash, whose sampled rows were just shown equal
    # to the oracle's; the oracle's backward takes the oracle's stash of each block
    q, s, qT, sT, _ = fgb.swiglu_bwd_quant(q_gu, s_gu, bf16_dev(dh))
    for b in blocks:
        r0, r1 = b * T, min((b + 1) * T, R)
        bq_gu, bs_gu, _, _, _ = orc.swiglu_fwd_quant(gu[r0:r1])
        assert_codes_equal(q_gu[r0:r1], bq_gu, f"q_gu block {b}")
        assert_scales_equal(s_gu[:, r0:r1], bs_gu, f"s_gu block {b}")
        _, oq, os_, oqT, osT = orc.swiglu_bwd_quant(bq_gu, bs_gu, dh[r0:r1])
        assert_codes_equal(q[r0:r1], oq, f"bwd q block {b}")
        assert_scales_equal(s[:, r0:r1], os_, f"bwd s block {b}")
        assert_codes_equal(qT[:, r0:r0 + T], oqT, f"bwd qT block {b}")
        assert_scales_equal(sT[b:b + 1], osT, f"bwd sT block {b}")
