"""Pins of the oracle's power-of-two (UE8M0) scale quantizers, independent of its
code: the exponent is checked against the two inequalities that define "the
smallest e with 448 * 2^e >= absmax", codes against torch's own E4M3 cast of
x * 2^-e, plus hand-derived tiles and the transposition identities."""
import numpy as np
import pytest
import torch

from fine_grained_block_amd import workloads as wl

T = 128


def bits_of(vals):
    return wl.bf16_bits(np.asarray(vals, np.float32))


def f32_of_bits(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_cast(v):
    """E4M3FN codes of float32 values (torch's RNE cast; no value here exceeds 448)."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_exponents(e, amax):
    """e (bytes) against amax: 448*2^(e-1) < amax <= 448*2^e, or e clamped at -127 / 127."""
    ex = e.astype(np.int64) - 127
    a = amax.astype(np.float64)
    lower_ok = (ex == -127) | (448.0 * np.exp2(ex - 1.0) < a)
    upper_ok = (ex == 127) | (a <= 448.0 * np.exp2(ex.astype(np.float64)))
    assert np.all(lower_ok) and np.all(upper_ok)


def stress_bits(R, C, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((R, C)).astype(np.float32) * np.power(10.0, g.uniform(-6, 3, (R, 1))).astype(np.float32)
    x[g.random((R, C)) < 0.02] = -0.0
    x[: min(R, 2), : min(C, 128)] = 0.0
    return wl.bf16_bits(x)


@pytest.mark.parametrize("R,C", [(1, 128), (7, 200), (130, 384), (64, 1024)])
def test_1x128_ue8m0_rule_and_codes(orc, R, C):
    x = stress_bits(R, C, R + C)
    q, e = orc.quantize_1x128_ue8m0(x)
    xf = f32_of_bits(x)
    nb = -(-C // T)
    assert e.shape == (nb, R)
    for j in range(nb):
        seg = xf[:, j * T:(j + 1) * T]
        amax = np.abs(seg).max(axis=1)
        check_exponents(e[j], amax)
        ex = e[j].astype(np.int64) - 127
        scaled = (seg.astype(np.float64) * np.exp2(-ex.astype(np.float64))[:, None]).astype(np.float32)
        assert np.abs(scaled).max() <= 448.0
        assert np.array_equal(q[:, j * T:(j + 1) * T], torch_cast(scaled))


def test_128x1_ue8m0_is_1x128_of_transpose(orc):
    x = stress_bits(300, 136, 3)
    qT, eT = orc.quantize_128x1_ue8m0(x)
    q2, e2 = orc.quantize_1x128_ue8m0(np.ascontiguousarray(x.T))
    assert np.array_equal(qT[:, :300], q2)
    assert np.all(qT[:, 300:] == 0)
    assert np.array_equal(eT, e2)


def test_128x128_ue8m0_tiles(orc):
    w = stress_bits(256, 384, 4)
    q, qT, e = orc.quantize_128x128_ue8m0(w)
    assert np.array_equal(q.T, qT)
    wf = f32_of_bits(w)
    for i in range(2):
        for j in range(3):
            tile = wf[i * T:(i + 1) * T, j * T:(j + 1) * T]
            check_exponents(e[i:i + 1, j], np.array([np.abs(tile).max()]))
            ex = int(e[i, j]) - 127
            assert np.array_equal(q[i * T:(i + 1) * T, j * T:(j + 1) * T],
                                  torch_cast((tile.astype(np.float64) * 2.0 ** -ex).astype(np.float32)))


def test_hand_derived_exponents(orc):
    """Tiles whose absmax sits on and beside a power-of-two boundary of 448."""
    cases = [(448.0, 127),     # 448 * 2^0 >= 448
             (450.0, 128),     # just above: 2^1
             (224.0, 126),     # 448 * 2^-1 = 224 exactly
             (225.0, 127),
             (1.75, 119),      # 448 * 2^-8 = 1.75
             (1.0, 119),       # 448 * 2^-9 = 0.875 < 1 <= 1.75
             (0.875, 118),
             (0.0, 0)]         # all-zero tile: e = -127
    x = np.zeros((len(cases), T), np.float32)
    for r, (a, _) in enumerate(cases):
        x[r, 5] = -a
        x[r, 9] = a / 4
    q, e = orc.quantize_1x128_ue8m0(wl.bf16_bits(x))
    assert list(e[0]) == [b for _, b in cases]
    # the absmax element lands on +-448 exactly when a = 448 * 2^e
    assert q[0, 5] == 0xFE and q[2, 5] == 0xFE and q[4, 5] == 0xFE
    assert q[7, 5] == 0x80 and q[7, 9] == 0x00          # -0 kept, +0 kept


def test_tiny_and_huge_tiles_clamp(orc):
    """bf16 subnormals need e < -127: the exponent clamps at -127 (byte 0); the
    bf16 maximum needs e = 120."""
    x = np.zeros((2, T), np.uint16)
    x[0, 0] = 0x0001                       # 2^-133
    x[1, 0] = 0x7F7F                       # largest finite bf16
    q, e = orc.quantize_1x128_ue8m0(x)
    assert e[0, 0] == 0 and e[0, 1] == 127 + 120
    big = float(f32_of_bits(np.array([0x7F7F]))[0])
    assert big <= 448.0 * 2.0 ** 120 and big > 448.0 * 2.0 ** 119
    assert q[0, 0] == 0x08                  # 2^-133 * 2^127 = 2^-6, the smallest normal E4M3
    assert q[1, 0] == torch_cast(np.float32([big * 2.0 ** -120]))[0]


def test_requant_ue8m0_is_128x1_of_dequantized(orc):
    """The requant step equals the 128x1 rule applied to dec(q) * 2^e, computed here
    with torch's decode and exact power-of-two scaling."""
    x = stress_bits(200, 256, 9)
    q, e = orc.quantize_1x128_ue8m0(x)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    scale = np.exp2(e.astype(np.float64) - 127.0)                 # [C/128, R]
    v = (dec * np.repeat(scale.T, T, axis=1)[:, :256]).astype(np.float32)
    qT, eT = orc.requant_128x1_ue8m0(q, e)
    # v is not bf16 in general: check the rule directly on the fp32 values
    for i in range(2):
        blk = v[i * T:(i + 1) * T]
        check_exponents(eT[i], np.abs(blk).max(axis=0))
        ex = eT[i].astype(np.int64) - 127
        scaled = (blk.astype(np.float64) * np.exp2(-ex.astype(np.float64))[None, :]).astype(np.float32)
        assert np.array_equal(qT[:, i * T:i * T + blk.shape[0]], torch_cast(scaled.T))
    assert np.all(qT[:, 200:] == 0)


def test_e8m0_decode_table(orc):
    d = orc.e8m0_decode(np.arange(256, dtype=np.uint8))
    assert d[127] == 1.0 and d[128] == 2.0 and d[0] == 2.0 ** -127 and d[254] == 2.0 ** 127
    assert np.isnan(d[255])
    assert np.all(np.diff(d[:255]) > 0)


def test_two_stage_weight_requant_is_ue8m0_rule_on_dequantized(orc):
    """Second stage of the two-stage weight cast: v = fl32(dec(q) * s) with the
    first stage's fp32 tile scales (torch's decode; the float32 product of two
    float32 values is the exact product rounded once), then the UE8M0 rule per
    128x128 tile of v, checked by its two inequalities and torch's cast."""
    K, N = 256, 384
    w = stress_bits(K, N, 11)
    q, _, s = orc.quantize_128x128(w)
    q2, q2T, e = orc.requant_128x128_ue8m0(q, s)
    assert np.array_equal(q2.T, q2T)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    v = dec * np.repeat(np.repeat(s, T, axis=0), T, axis=1)          # float32 * float32
    for i in range(K // T):
        for j in range(N // T):
            tile = v[i * T:(i + 1) * T, j * T:(j + 1) * T]
            check_exponents(e[i:i + 1, j], np.array([np.abs(tile).max()]))
            ex = int(e[i, j]) - 127
            scaled = (tile.astype(np.float64) * 2.0 ** -ex).astype(np.float32)
            assert np.abs(scaled).max() <= 448.0
            assert np.array_equal(q2[i * T:(i + 1) * T, j * T:(j + 1) * T], torch_cast(scaled))


def test_two_stage_requant_of_power_of_two_weights_is_identity(orc):
    """A first stage that already has power-of-two scales comes back unchanged:
    the decoded tile's absmax is a code times 2^e, so the rule picks e again and
    every scaled value is an E4M3 value."""
    w = stress_bits(384, 256, 12)
    q, _, e = orc.quantize_128x128_ue8m0(w)
    s = np.exp2(e.astype(np.float64) - 127.0).astype(np.float32)
    q2, _, e2 = orc.requant_128x128_ue8m0(q, s)
    assert np.array_equal(e2, e)
    assert np.array_equal(q2, q)


def test_two_stage_requant_floors(orc):
    """The pages' minimum power-of-two scales (conventions row "Activation
    floors"): an amax floor of 1e-10 gives 2^-42 (1e-10 / 448 lies in
    (2^-43, 2^-42]); flooring the scale itself at 1e-10 gives 2^-33, the same
    exponent as an amax floor of 448 * 2^-33.  A tile whose values are tiny
    but non-zero takes the floor when the floor is larger."""
    q = np.zeros((128, 256), np.uint8)
    q[0, 130] = 0x01                                   # dec = 2^-9 in tile (0, 1)
    s = np.array([[1.0, 2.0 ** -40]], np.float32)      # tile (0, 1) holds 2^-49
    for floor, want in [(1e-10, -42), (448.0 * 2.0 ** -33, -33)]:
        _, _, e = orc.requant_128x128_ue8m0(q, s, amax_floor=floor)
        assert int(e[0, 0]) - 127 == want and int(e[0, 1]) - 127 == want
    _, _, e = orc.requant_128x128_ue8m0(q, s)
    assert int(e[0, 0]) == 0                            # all-zero tile, no floor: -127
    assert int(e[0, 1]) - 127 == -57                    # 448 * 2^-58 < 2^-49 <= 448 * 2^-57
