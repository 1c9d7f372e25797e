"""Pins for the oracle's tile quantizers (CPU only).

Dynamic tile quantization with scale = tile absmax / 448: "scratch: the
backward pass, unrolled", section "What is asserted, and from where" (1x128
activation tiles, 128x128 weight tiles, Wgrad operands re-tiled 128x1 from the
saved tensors); partial-sum-drift notes, section 3 row (a) (scale from the
in-block absmax, N_c = 128); prime-rl PR #4073 conventions table (/448, -0).

Pins, each independent of the oracle's own code:
* a vectorized numpy implementation whose cast is torch's float8_e4m3fn
  conversion (a library routine) -- bytes and scale bits equal;
* invariants: every tile's absmax element lands on +-448; zero tiles give
  s = +0 and sign-keeping zero codes; reconstruction error within half an
  E4M3 step; no NaN codes from finite input;
* transposition identities between the tilings;
* the requant special case (grid-valued input with 448 in every tile is an
  exact byte transpose), and hand-derived codes for one tile.
"""
import os

import numpy as np
import pytest
import torch

from fine_grained_block_amd import workloads as wl

T = 128


def bf16(a):
    return wl.bf16_bits(np.asarray(a, np.float32))


def to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_enc(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def numpy_1x128(xbits):
    """Vectorized 1x128 quantization (C a multiple of 128) using torch's cast."""
    x = to_f32(xbits)
    R, C = x.shape
    tiles = x.reshape(R, C // T, T)
    a = np.abs(tiles).max(axis=2)                                   # [R, C/128]
    s = (a / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(a == 0, np.float32(0), np.float32(448.0) / a).astype(np.float32)
    inv = np.minimum(inv, np.float32(np.finfo(np.float32).max))
    q = torch_enc(tiles * inv[:, :, None]).reshape(R, C)
    return q, s.T.copy()


def mixed_matrix(R, C, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((R, C)).astype(np.float32) * np.power(10.0, g.uniform(-5, 3, (R, 1))).astype(np.float32)
    x[g.random((R, C)) < 0.02] = -0.0
    x[g.random((R, C)) < 0.02] = 0.0
    x[: min(R, 3), : min(C, 128)] = 0.0
    return bf16(x)


@pytest.mark.parametrize("R,C", [(1, 128), (7, 256), (130, 384), (256, 512)])
def test_1x128_matches_vectorized_torch_cast(orc, R, C):
    x = mixed_matrix(R, C, R * 1000 + C)
    q, s = orc.quantize_1x128(x)
    q2, s2 = numpy_1x128(x)
    assert np.array_equal(q, q2)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_1x128_fprop_small_matches_vectorized(orc):
    d = wl.fprop_small()
    q, s = orc.quantize_1x128(d["x"])
    q2, s2 = numpy_1x128(d["x"])
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def check_tile_invariants(vals_f32, codes, scale):
    """One tile: absmax -> +-448; zero tile -> s = +0 and sign-kept zeros;
    |x - s*dec(q)| <= s * half E4M3 step of |x|/s (+ slack for fp32 rounding)."""
    a = np.abs(vals_f32).max() if vals_f32.size else 0.0
    assert np.float32(scale).view(np.uint32) == (np.float32(a) / np.float32(448.0)).view(np.uint32)
    assert not np.any((codes & 0x7F) == 0x7F)
    if a == 0:
        assert scale == 0 and not np.signbit(scale)
        assert np.array_equal(codes, np.where(np.signbit(vals_f32), 0x80, 0x00).astype(np.uint8))
        return
    # negative values (and -0) keep the sign bit
    assert np.all((codes[np.signbit(vals_f32)] & 0x80) == 0x80)
    with np.errstate(over="ignore"):
        if not np.isfinite(np.float32(448.0) / np.float32(a)):
            return          # inverse clamped to FLT_MAX: the 448 mapping is waived
    big = np.abs(vals_f32) == a
    assert np.all((codes[big] & 0x7F) == 0x7E)
    dec = torch_dec(codes)
    y = vals_f32.astype(np.float64) / float(scale)               # position on the E4M3 grid
    # half-step of E4M3 at |y|: 2^(floor(log2|y|)-4) for normals, 2^-10 in the subnormal range
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0**-6)))
    half = np.exp2(e - 4)
    err = np.abs(y - dec)
    assert np.all(err <= half * (1 + 1e-6) + 1e-6 * np.abs(y) + 1e-30)


def test_quantizer_invariants_mixed(orc):
    x = mixed_matrix(300, 640, 5)
    xf = to_f32(x)
    q, s = orc.quantize_1x128(x)
    for r in range(0, 300, 7):
        for j in range(5):
            check_tile_invariants(xf[r, j * T:(j + 1) * T], q[r, j * T:(j + 1) * T], s[j, r])
    qT, sT = orc.quantize_128x1(x)
    for c in range(0, 640, 11):
        for i in range(3):
            r0, r1 = i * T, min(300, (i + 1) * T)
            check_tile_invariants(xf[r0:r1, c], qT[c, r0:r1], sT[i, c])
    w = mixed_matrix(384, 256, 6)
    wf = to_f32(w)
    qw, qwT, sw = orc.quantize_128x128(w)
    for i in range(3):
        for j in range(2):
            blk = (slice(i * T, (i + 1) * T), slice(j * T, (j + 1) * T))
            check_tile_invariants(wf[blk].ravel(), qw[blk].ravel(), sw[i, j])


def test_quant_stress_invariants_sampled(orc):
    """The quant-stress distribution (scales 1e-6..1e3, zeros of both signs,
    tiny negatives, bf16 subnormals) on a slice of its rows."""
    d = wl.quant_stress(R=512, C=1024)
    x = d["x"]
    xf = to_f32(x)
    q, s = orc.quantize_1x128(x)
    q2, s2 = numpy_1x128(x)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    for r in range(0, 512, 3):
        for j in range(8):
            check_tile_invariants(xf[r, j * T:(j + 1) * T], q[r, j * T:(j + 1) * T], s[j, r])
    # every negative input (including -0, tiny negatives and subnormals) encodes with the sign bit
    assert np.all((q[np.signbit(xf)] & 0x80) == 0x80)
    assert np.any(q == 0x80)


@pytest.mark.parametrize("R,C", [(128, 128), (200, 256), (1, 384), (257, 130)])
def test_128x1_is_1x128_of_transpose(orc, R, C):
    x = mixed_matrix(R, C, 77 + R + C)
    qT, sT = orc.quantize_128x1(x)
    q1, s1 = orc.quantize_1x128(np.ascontiguousarray(x.T))
    Rp = -(-R // T) * T
    assert qT.shape == (C, Rp)
    assert np.array_equal(qT[:, :R], q1)
    assert np.all(qT[:, R:] == 0)
    assert np.array_equal(sT.view(np.uint32), s1.view(np.uint32))


def test_128x128_transpose_identity(orc):
    w = mixed_matrix(256, 384, 9)
    q, qT, s = orc.quantize_128x128(w)
    assert np.array_equal(qT, q.T)
    q2, qT2, s2 = orc.quantize_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(q2, qT) and np.array_equal(s2.view(np.uint32), s.T.view(np.uint32))


def test_128x128_matches_vectorized(orc):
    w = mixed_matrix(384, 256, 10)
    wf = to_f32(w)
    q, qT, s = orc.quantize_128x128(w)
    blocks = wf.reshape(3, T, 2, T).transpose(0, 2, 1, 3)
    a = np.abs(blocks).max(axis=(2, 3))
    s2 = (a / np.float32(448)).astype(np.float32)
    inv = np.where(a == 0, np.float32(0), np.float32(448) / np.where(a == 0, 1, a)).astype(np.float32)
    q2 = torch_enc(blocks * inv[:, :, None, None]).reshape(3, 2, T, T).transpose(0, 2, 1, 3).reshape(384, 256)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_requant_grid_special_case_is_byte_transpose(orc):
    """X on the E4M3 grid with +-448 in every 1x128 and every 128x1 tile: all
    scales are 1, so requant 128x1 is an exact byte transpose."""
    g = np.random.default_rng(3)
    R, C = 256, 384
    codes = g.integers(0, 256, (R, C)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN
    codes[np.arange(R), (np.arange(R) * 5) % C] = 0x7E   # 448 in each row segment ...
    for j in range(C // T):
        codes[np.arange(R), j * T + (np.arange(R) % T)] = 0xFE  # ... -448 in every row tile
    for c in range(C):
        codes[(c % T), c] = 0x7E                   # and in every column tile of rows 0..127
        codes[T + (c % T), c] = 0xFE               # and rows 128..255
    xf = torch_dec(codes).astype(np.float32)
    x = bf16(xf)                                    # exact: 4-bit significands
    assert np.array_equal(to_f32(x), xf)
    q, s = orc.quantize_1x128(x)
    assert np.all(s == 1.0) and np.array_equal(q, codes)
    qT, sT = orc.requant_128x1(q, s)
    assert np.all(sT == 1.0) and np.array_equal(qT, codes.T)


def test_requant_equals_128x1_of_dequantized(orc):
    """requant = 128x1 quantization of fl32(dec(q) * s)."""
    x = mixed_matrix(200, 256, 12)
    q, s = orc.quantize_1x128(x)
    v = (torch_dec(q) * s.T.repeat(T, axis=1)[:, :256].astype(np.float64)).astype(np.float32)
    # the product of two values with <= 24 significant bits is exact in fp64
    qT, sT = orc.requant_128x1(q, s)
    R, C = v.shape
    tiles = np.zeros((C, 256), np.float32)
    tiles[:, :R] = v.T
    tl = tiles.reshape(C, 2, T)
    a = np.abs(tl).max(axis=2)
    s2 = (a / np.float32(448)).astype(np.float32)
    inv = np.where(a == 0, np.float32(0), np.float32(448) / np.where(a == 0, 1, a)).astype(np.float32)
    q2 = torch_enc(tl * inv[:, :, None]).reshape(C, 256)
    q2[:, R:] = 0
    assert np.array_equal(qT, q2) and np.array_equal(sT.view(np.uint32), s2.T.view(np.uint32))


def test_amax_floor(orc):
    """vLLM order: floor the amax, then divide by 448 (prime-rl conventions table)."""
    x = bf16(np.full((1, 128), 1e-6, np.float32))
    q, s = orc.quantize_1x128(x, amax_floor=1e-4)
    assert s[0, 0] == np.float32(1e-4) / np.float32(448)
    q0, s0 = orc.quantize_1x128(x)
    assert np.all(q0 == 0x7E) and np.all(q < 0x7E)


def test_tiny_amax_inverse_clamped(orc):
    """448/amax overflows fp32 for amax below ~1.3e-36: the inverse is clamped
    to FLT_MAX so the codes stay finite (no NaN from 0 * inf)."""
    x = np.zeros((1, 128), np.uint16)
    x[0, :4] = [0x0001, 0x8002, 0x0000, 0x8000]      # bf16 subnormals and zeros
    q, s = orc.quantize_1x128(x)
    assert np.all((q & 0x7F) != 0x7F)
    assert q[0, 2] == 0x00 and q[0, 3] == 0x80 and (q[0, 1] & 0x80)


def test_hand_derived_tile(orc):
    """x_i = (i - 64)/16, i = 0..127: absmax 4, s = fl32(4/448), inv = 112,
    so q_i = enc(7 (i - 64)).  Codes worked out by hand:
      i=64 -> 0 -> 0x00; i=65 -> 7 = 1.75*4 -> 0x4E; i=63 -> -7 -> 0xCE;
      i=0 -> -448 -> 0xFE; i=127 -> 441 (nearest 448, midpoint 432) -> 0x7E;
      i=66 -> 14 = 1.75*8 -> 0x56; i=68 -> 28 = 1.75*16 -> 0x5E;
      i=69 -> 35 = 1.09375*32: between 32 (0x60) and 36 (0x61), nearer 36 -> 0x61;
      i=74 -> 70 = 1.09375*64: between 64 (0x68) and 72 (0x69), nearer 72 -> 0x69."""
    i = np.arange(128)
    x = bf16(((i - 64) / 16.0).reshape(1, 128))
    q, s = orc.quantize_1x128(x)
    assert s[0, 0] == np.float32(4.0) / np.float32(448.0)
    want = {64: 0x00, 65: 0x4E, 63: 0xCE, 0: 0xFE, 127: 0x7E, 66: 0x56, 68: 0x5E, 69: 0x61, 74: 0x69}
    for k, v in want.items():
        assert q[0, k] == v, (k, hex(q[0, k]), hex(v))


def test_per_tensor_scale_negative_control(orc):
    """Negative control: one scale for the whole tensor is not the method; its
    bytes differ from the 1x128 result on mixed-scale rows."""
    x = mixed_matrix(64, 256, 13)
    q, s = orc.quantize_1x128(x)
    xf = to_f32(x)
    a = np.float32(np.abs(xf).max())
    qt = torch_enc(xf * (np.float32(448) / a))
    assert not np.array_equal(q, qt)


# ---------------------------------------------------------------------------
# NaN tiles: the pages say nothing about NaN; the reading is that a NaN element
# makes its tile's scale NaN and every code of that tile the E4M3 NaN 0x7F (the
# GPU kernels follow the same rule), while every other tile is unaffected.
# ---------------------------------------------------------------------------

def _nan_input():
    g = np.random.default_rng(17)
    x = g.standard_normal((256, 384)).astype(np.float32)
    bits = wl.bf16_bits(x)
    clean = bits.copy()
    bits[5, 130] = 0x7FC0            # quiet NaN in row 5, column tile 1, row tile 0
    bits[200, 7] = 0xFFC1            # negative NaN with a payload: row 200, column tile 0, row tile 1
    return bits, clean


def test_nan_tile_1x128(orc):
    bits, clean = _nan_input()
    q, s = orc.quantize_1x128(bits)
    q0, s0 = orc.quantize_1x128(clean)
    nan_tiles = {(5, 1), (200, 0)}
    for r in range(256):
        for j in range(3):
            seg = slice(128 * j, 128 * j + 128)
            if (r, j) in nan_tiles:
                assert np.isnan(s[j, r]) and np.all(q[r, seg] == 0x7F)
            else:
                assert s[j, r].view(np.uint32) == s0[j, r].view(np.uint32)
                assert np.array_equal(q[r, seg], q0[r, seg])


def test_nan_tile_128x1_and_128x128(orc):
    bits, clean = _nan_input()
    qT, sT = orc.quantize_128x1(bits)
    qT0, sT0 = orc.quantize_128x1(clean)
    for c in range(384):
        for i in range(2):
            seg = slice(128 * i, 128 * i + 128)
            if (i, c) in {(0, 130), (1, 7)}:
                assert np.isnan(sT[i, c]) and np.all(qT[c, seg] == 0x7F)
            else:
                assert sT[i, c].view(np.uint32) == sT0[i, c].view(np.uint32)
                assert np.array_equal(qT[c, seg], qT0[c, seg])
    q, qt, s = orc.quantize_128x128(bits)
    q0, qt0, s0 = orc.quantize_128x128(clean)
    for i in range(2):
        for j in range(3):
            blk = (slice(128 * i, 128 * i + 128), slice(128 * j, 128 * j + 128))
            if (i, j) in {(0, 1), (1, 0)}:
                assert np.isnan(s[i, j]) and np.all(q[blk] == 0x7F) and np.all(qt[blk[::-1]] == 0x7F)
            else:
                assert s[i, j].view(np.uint32) == s0[i, j].view(np.uint32)
                assert np.array_equal(q[blk], q0[blk])


def test_nan_tile_requant_and_power_of_two(orc):
    bits, clean = _nan_input()
    q, s = orc.quantize_1x128(bits)
    qT, sT = orc.requant_128x1(q, s)
    # a NaN 1x128 tile dequantizes to NaN and makes every 128x1 tile it crosses NaN
    for c in range(384):
        for i in range(2):
            hit = (i == 0 and 128 <= c < 256) or (i == 1 and c < 128)
            assert np.isnan(sT[i, c]) == hit
            if hit:
                assert np.all(qT[c, 128 * i:128 * i + 128] == 0x7F)
    qe, e = orc.quantize_1x128_ue8m0(bits)
    assert e[1, 5] == 0xFF and np.all(qe[5, 128:256] == 0x7F)
    assert e[0, 200] == 0xFF and np.all(qe[200, :128] == 0x7F)
    assert e[0, 5] != 0xFF
    qs, ss = orc.quantize_1x128_sr(bits, 3, 4)
    assert np.isnan(ss[1, 5]) and np.all(qs[5, 128:256] == 0x7F)
    assert not np.isnan(ss[0, 5])


def test_inf_tile(orc):
    """An infinite element makes its tile's absmax Inf: s = Inf/448 = Inf and the
    multiplier 448/Inf = 0, so finite elements cast to +-0 (each with its sign)
    and the infinite element, Inf * 0, is NaN: code 0x7F.  Other tiles unchanged."""
    g = np.random.default_rng(23)
    bits = wl.bf16_bits(g.standard_normal((4, 256)).astype(np.float32))
    clean = bits.copy()
    bits[1, 3] = 0x7F80          # +Inf in row 1, tile 0
    bits[2, 200] = 0xFF80        # -Inf in row 2, tile 1
    q, s = orc.quantize_1x128(bits)
    q0, s0 = orc.quantize_1x128(clean)
    for r, j, c in [(1, 0, 3), (2, 1, 200)]:
        seg = slice(128 * j, 128 * j + 128)
        assert np.isinf(s[j, r]) and s[j, r] > 0
        assert q[r, c] == 0x7F
        others = [k for k in range(128 * j, 128 * j + 128) if k != c]
        sign = (bits[r, others] >> 15).astype(np.uint8) << 7
        assert np.array_equal(q[r, others], sign)                 # +-0 with the input's sign
    mask = np.ones_like(q, bool)
    mask[1, :128] = mask[2, 128:] = False
    assert np.array_equal(q[mask], q0[mask])
