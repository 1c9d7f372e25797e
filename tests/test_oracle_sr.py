"""Pins of the oracle's stochastic-rounding (SR) quantizers (CPU only).

What the pages fix (prime-rl PR #4073, conventions row "SR agreement"): SR picks
the lower- or upper-magnitude E4M3 neighbour using words from a stateless
seed/salt/counter Philox helper.  The reading pinned here: Philox4x32-10, the
upper neighbour taken when u < (|v| - lo)/(hi - lo) * 2^32, the tile scale of the
round-to-nearest quantizer, and word (r, c) = word c mod 4 of the block with
counter (c div 4, r, salt, 0) and key (seed low, seed high).

Pins, none of which reuses the oracle's code:
- Philox against the generator's published known-answer vectors (tests/golden);
- the cast against an exact rational construction from torch's E4M3 decode
  table, at the decision boundary itself (u = T - 1 rounds up, u = T does not);
- grid values never move; u = 0 rounds every off-grid magnitude up and
  u = 2^32 - 1 truncates toward zero;
- unbiasedness: the mean over many seeds of the dequantized tile converges to
  the input at the rate the rounding variance allows;
- scales are the round-to-nearest quantizer's bit for bit, and every SR code is
  one of the two neighbours of the exact scaled value;
- the same element draws the same word in every tiling: where both tilings' scales
  are 1, the 1x128, 128x1 and 128x128 SR codes agree byte for byte.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from fine_grained_block_amd import workloads as wl

T = 128
HERE = os.path.dirname(os.path.abspath(__file__))

# non-negative finite E4M3 magnitudes from torch's decoder (codes 0x00 .. 0x7E)
MAGS = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows.append([int(t, 16) for t in line])
    return rows


def test_philox_known_answers(orc):
    rows = kat_rows()
    assert len(rows) == 3
    for r in rows:
        out = orc.philox4x32_10(np.array(r[0:4], np.uint32), np.array(r[4:6], np.uint32))
        assert [int(v) for v in out] == r[6:10], [hex(int(v)) for v in out]


def test_sr_word_layout(orc):
    """word (r, c) is output word c mod 4 of the block at counter (c div 4, r, salt, 0),
    key (seed mod 2^32, seed div 2^32)."""
    seed, salt = 0x0123456789ABCDEF, 0x5A17
    w = orc.sr_words(seed, salt, 5, 3, 8, 8)
    for i in range(3):
        for j in range(8):
            blk = orc.philox4x32_10(np.array([(8 + j) // 4, 5 + i, salt, 0], np.uint32),
                                    np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32))
            assert w[i, j] == blk[(8 + j) % 4]


def exact_up_threshold(m):
    """T with: the upper neighbour is taken iff u < T (u integer), from the rational
    (m - lo)/(hi - lo) * 2^32; lo/hi from torch's decode table."""
    m = Fraction(float(m))
    a = int(np.searchsorted(MAGS, float(m), side="right")) - 1
    lo = Fraction(float(MAGS[a]))
    if lo == m:
        return a, 0
    hi = Fraction(float(MAGS[a + 1]))
    x = (m - lo) / (hi - lo) * 2 ** 32
    t = x.numerator // x.denominator + (1 if x.denominator != 1 else 0)   # ceil
    return a, t


def sample_values(g, n):
    """Magnitudes across the whole E4M3 range: subnormal range, fp32 denormals,
    every binade, just below 448, plus on-grid values."""
    parts = [
        np.exp2(g.uniform(-9, np.log2(448.0), n)),
        np.exp2(g.uniform(-30, -6, n // 4)),
        g.uniform(0, 2.0 ** -6, n // 4),
        np.array([2.0 ** -140, 1e-45, 2.0 ** -10, 2.0 ** -9, 2.0 ** -6 - 2.0 ** -30, 447.99997, 440.0, 432.5]),
        MAGS[g.integers(0, 127, n // 8)],
    ]
    return np.concatenate(parts).astype(np.float32)


def test_cast_at_the_decision_boundary(orc):
    g = np.random.default_rng(101)
    v = sample_values(g, 600)
    for sgn in (1.0, -1.0):
        vv = (sgn * v).astype(np.float32)
        lo_idx, thr = zip(*(exact_up_threshold(abs(float(x))) for x in vv))
        lo_idx, thr = np.array(lo_idx), np.array(thr, np.int64)
        sign = np.where(np.signbit(vv), 0x80, 0x00)
        on_grid = thr == 0
        # u = T - 1 -> upper neighbour, u = T -> lower (when 0 < T <= 2^32 - 1)
        inner = (~on_grid) & (thr <= 2 ** 32 - 1)
        got_up = orc.e4m3_encode_sr(vv[inner], (thr[inner] - 1).astype(np.uint32))
        got_lo = orc.e4m3_encode_sr(vv[inner], thr[inner].astype(np.uint32))
        assert np.array_equal(got_up, (sign[inner] | (lo_idx[inner] + 1)).astype(np.uint8))
        assert np.array_equal(got_lo, (sign[inner] | lo_idx[inner]).astype(np.uint8))
        # on-grid values keep their code for any word
        u = g.integers(0, 2 ** 32, on_grid.sum(), dtype=np.uint64).astype(np.uint32)
        got = orc.e4m3_encode_sr(vv[on_grid], u)
        assert np.array_equal(got, (sign[on_grid] | lo_idx[on_grid]).astype(np.uint8))


def test_extreme_words_are_directed_rounding(orc):
    """u = 0 takes the upper neighbour of every off-grid magnitude (ceil of |v|),
    u = 2^32 - 1 the lower one (truncation toward zero)."""
    g = np.random.default_rng(7)
    v = sample_values(g, 2000)
    v = np.concatenate([v, -v]).astype(np.float32)
    m = np.abs(v).astype(np.float64)
    lo = np.searchsorted(MAGS, m, side="right") - 1
    exact = MAGS[lo] == m
    hi = np.where(exact, lo, lo + 1)
    sign = np.where(np.signbit(v), 0x80, 0x00)
    up = orc.e4m3_encode_sr(v, np.zeros(v.size, np.uint32))
    dn = orc.e4m3_encode_sr(v, np.full(v.size, 0xFFFFFFFF, np.uint32))
    assert np.array_equal(up, (sign | hi).astype(np.uint8))
    assert np.array_equal(dn, (sign | lo).astype(np.uint8))


def test_specials(orc):
    v = np.array([np.nan, -np.nan, 448.0, -448.0, 449.0, np.inf, -np.inf, 0.0, -0.0], np.float32)
    for u in (0, 1, 0x80000000, 0xFFFFFFFF):
        got = orc.e4m3_encode_sr(v, np.full(v.size, u, np.uint32))
        nan_sign = np.signbit(v[:2])
        assert list(got[:2]) == [0xFF if s else 0x7F for s in nan_sign]
        assert list(got[2:]) == [0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x00, 0x80]


def test_scales_are_round_to_nearest_scales(orc):
    x = wl.normal_bf16((300, 700), 1.0, 11, 0)
    q, s = orc.quantize_1x128_sr(x, seed=3, salt=1)
    q0, s0 = orc.quantize_1x128(x)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    qT, sT = orc.quantize_128x1_sr(x, seed=3, salt=1)
    qT0, sT0 = orc.quantize_128x1(x)
    assert np.array_equal(sT.view(np.uint32), sT0.view(np.uint32))
    w = wl.normal_bf16((384, 640), 0.02, 11, 1)
    qw, qwT, sw = orc.quantize_128x128_sr(w, seed=3, salt=2)
    qw0, _, sw0 = orc.quantize_128x128(w)
    assert np.array_equal(sw.view(np.uint32), sw0.view(np.uint32))
    assert np.array_equal(qwT, qw.T)


def test_codes_are_neighbours_of_the_scaled_value(orc):
    """Every SR code is the lower or upper neighbour of v = fl32(x * fl32(448/a)),
    computed here from torch's bf16 decode and float32 arithmetic."""
    x = wl.normal_bf16((256, 512), 1.0, 12, 0)
    q, s = orc.quantize_1x128_sr(x, seed=99, salt=0)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    a = np.abs(xf).reshape(256, 4, T).max(axis=2)
    inv = (np.float32(448.0) / a.astype(np.float32)).astype(np.float32)
    v = (xf.reshape(256, 4, T) * inv[:, :, None]).astype(np.float32).reshape(256, 512)
    m = np.abs(v).astype(np.float64)
    lo = np.searchsorted(MAGS, m, side="right") - 1
    hi = np.where(MAGS[lo] == m, lo, np.minimum(lo + 1, 126))
    mag_code = (q & 0x7F).astype(np.int64)
    assert np.all((mag_code == lo) | (mag_code == hi))
    assert np.array_equal(q >> 7, np.signbit(v).astype(np.uint8))
    # and both neighbours do occur (the cast is not a deterministic rounding)
    off = lo != hi
    assert 0.2 < np.mean(mag_code[off] == hi[off]) < 0.8


def test_unbiased_over_seeds(orc):
    """E[dec(q)] = v for v = fl32(x * fl32(448/a)) (computed here in float32 from
    torch's bf16 decode): the mean over S seeds deviates from v by no more than the
    rounding variance allows (each draw is one of v's two grid neighbours)."""
    R, C, S = 4, 256, 400
    x = wl.normal_bf16((R, C), 1.0, 13, 0)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    a = np.abs(xf).reshape(R, C // T, T).max(axis=2)
    inv = (np.float32(448.0) / a.astype(np.float32)).astype(np.float32)
    v = (xf.reshape(R, C // T, T) * inv[:, :, None]).astype(np.float32).reshape(R, C).astype(np.float64)
    acc = np.zeros((R, C))
    for seed in range(S):
        q, _ = orc.quantize_1x128_sr(x, seed=seed, salt=7)
        acc += orc.e4m3_decode(q)
    mean = acc / S
    v = np.clip(v, -448.0, 448.0)     # fl32(a * fl32(448/a)) may exceed 448 by an ulp; it saturates
    m = np.abs(v)
    lo = np.searchsorted(MAGS, m, side="right") - 1
    step = MAGS[np.minimum(lo + 1, 126)] - MAGS[lo]
    sd = np.maximum(step / 2.0, 1e-30) / np.sqrt(S)
    z = np.abs(mean - v) / sd
    assert z.max() < 6.0, z.max()
    # round-to-nearest, by contrast, keeps its bias: some elements sit > 6 sd away
    q0, _ = orc.quantize_1x128(x)
    assert (np.abs(orc.e4m3_decode(q0) - v) / sd).max() > 6.0


def test_same_element_same_word_in_every_tiling(orc):
    """Values on the E4M3 grid with 448 in every 1x128 row tile, 128x1 column tile
    and 128x128 tile: all scales are 1 and every tiling sees the same v, so its SR
    codes must agree byte for byte -- the word depends only on (seed, salt, r, c)."""
    g = np.random.default_rng(21)
    R, C = 256, 384
    # off-grid values: the grid midpoints scaled by a non-dyadic factor stay off-grid
    vals = (MAGS[g.integers(1, 120, (R, C))] * 1.0 + MAGS[g.integers(1, 120, (R, C))] * 0.37)
    vals = np.minimum(vals, 447.0)
    vals[np.arange(R), (np.arange(R) * 131) % C] = 448.0          # one 448 in every row
    for c in range(C):                                               # and in every column tile
        for r0 in range(0, R, T):
            vals[r0 + (c * 37) % T, c] = 448.0
    sgn = np.where(g.random((R, C)) < 0.5, -1.0, 1.0)
    xb = torch.from_numpy((vals * sgn).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.all(np.abs(xf).reshape(R, C // T, T).max(axis=2) == 448.0)
    assert np.all(np.abs(xf).reshape(R // T, T, C).max(axis=1) == 448.0)
    seed, salt = 0xDEADBEEF12345678, 77
    q1, s1 = orc.quantize_1x128_sr(xb, seed, salt)
    qT, sT = orc.quantize_128x1_sr(xb, seed, salt)
    qw, qwT, sw = orc.quantize_128x128_sr(xb, seed, salt)
    assert np.all(s1 == 1.0) and np.all(sT == 1.0) and np.all(sw == 1.0)
    assert np.array_equal(q1, qT.T)
    assert np.array_equal(q1, qw)
    # and the words really differ between seeds and salts
    assert not np.array_equal(q1, orc.quantize_1x128_sr(xb, seed + 1, salt)[0])
    assert not np.array_equal(q1, orc.quantize_1x128_sr(xb, seed, salt + 1)[0])
