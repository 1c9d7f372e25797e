"""Pins for the oracle's number formats (CPU only).

The E4M3 format: prime-rl PR #4073, "Trainer / vLLM quantization conventions"
table (448 denominator, -0 = 0x80 kept distinct, RN cast), read as OCP
E4M3FN with ties-to-even and saturation.  Each pin below is independent of the
oracle's own code: torch's float8/bfloat16 casts (library routines), a
threshold construction from the 127 finite magnitudes, and hand-derived codes.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_all_codes(orc):
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    t = torch_decode_all()
    assert np.array_equal(d, t, equal_nan=True)
    # -0 is distinct from +0 (sign bit kept)
    assert d[0x80] == 0.0 and np.signbit(d[0x80]) and not np.signbit(d[0x00])


def test_decode_golden_codes(orc):
    """Hand-derived values of E4M3FN codes (tests/golden/e4m3_codes.txt)."""
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), val))
    assert len(rows) >= 10
    for code, val in rows:
        got = orc.e4m3_decode(np.array([code], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            exp = float.fromhex(val) if val.startswith(("0x", "-0x")) else float(val)
            assert got == exp and math.copysign(1, got) == math.copysign(1, exp), (hex(code), got, exp)


def _thresholds():
    """Nearest-value encoder as a step function of the fp32 bit pattern.

    The 127 finite non-negative E4M3 magnitudes (codes 0x00..0x7E, decoded by
    torch) are increasing; the midpoint between neighbours c and c+1 is exactly
    representable in fp32.  A non-negative float below the midpoint encodes to
    c, above it to c+1, and on it to whichever of c, c+1 is even.  Everything
    above the last midpoint is nearest to 448 (code 0x7E), which is also the
    saturating result; NaN patterns encode to 0x7F.  Negative patterns take the
    code of their magnitude with bit 7 set."""
    vals = torch_decode_all()[:127]
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2.0
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)   # exact in fp32
    return mids32.view(np.uint32).astype(np.int64)


def _segments(mid_bits):
    """(start, code) runs of the nearest-value encoder over magnitude bit
    patterns 0 .. 2^31-1: below midpoint c the code is c, on it the even one of
    c and c+1, above it c+1; after the last midpoint 0x7E up to +inf; NaNs 0x7F."""
    starts, codes = [0], [0]
    for c, m in enumerate(mid_bits):
        starts += [int(m), int(m) + 1]
        codes += [c if c % 2 == 0 else c + 1, c + 1]
    starts.append(0x7F800001)
    codes.append(0x7F)
    return np.array(starts, np.int64), np.array(codes, np.uint8)


def _expected_codes(start, n, segs):
    """Expected codes for the bit patterns start .. start+n-1 (one sign only)."""
    starts, codes = segs
    sign = np.uint8(0x80) if start >= (1 << 31) else np.uint8(0)
    m0 = start & 0x7FFFFFFF
    m1 = m0 + n
    assert m1 <= (1 << 31)
    ends = np.append(starts[1:], 1 << 31)
    lo = np.clip(starts, m0, m1)
    hi = np.clip(ends, m0, m1)
    return np.repeat(codes, hi - lo) | sign


def test_encode_exhaustive_all_fp32(orc):
    """Every one of the 2^32 fp32 bit patterns, against the threshold construction."""
    segs = _segments(_thresholds())
    chunk = 1 << 27
    for start in range(0, 1 << 32, chunk):
        got = orc.e4m3_encode_bits_range(start, chunk)
        exp = _expected_codes(start, chunk, segs)
        if not np.array_equal(got, exp):
            bad = np.nonzero(got != exp)[0][:8]
            raise AssertionError([(hex(start + int(i)), hex(got[i]), hex(exp[i])) for i in bad])


def test_encode_matches_torch_cast(orc):
    """torch's float -> float8_e4m3fn cast (RNE) for |f| <= 448 and NaN."""
    g = np.random.default_rng(1234)
    bits = g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = np.concatenate([f, np.float32([0.0, -0.0, 448.0, -448.0, 2.0**-10, -2.0**-10,
                                       3 * 2.0**-11, 2.0**-6, 240.0, 232.0, 0.0009765625])])
    # plus a dense sample of the quantizer's working range
    f = np.concatenate([f, (g.standard_normal(1 << 20) * 100).astype(np.float32)])
    keep = np.isnan(f) | (np.abs(f) <= 448)
    f = f[keep]
    got = orc.e4m3_encode(f)
    t = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], t[~nan])
    assert np.all((got[nan] & 0x7F) == 0x7F)


def test_encode_saturates_and_keeps_sign(orc):
    f = np.float32([464.0, 500.0, 1e30, np.inf, -464.0, -np.inf, 449.0, -1e-30, -0.0, 0.0, -2.0**-10])
    got = orc.e4m3_encode(f)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E, 0x80, 0x80, 0x00, 0x80]


def test_encode_decode_roundtrip_all_finite_codes(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes)


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_fp32_inputs(orc):
    g = np.random.default_rng(7)
    bits = g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    specials = np.uint32([0, 0x80000000, 0x00000001, 0x00008000, 0x00018000, 0x7F7FFFFF,
                          0x7F7F8000, 0x7F7F7FFF, 0x3F808000, 0x3F818000, 0x807FFFFF, 0x00800000])
    f = np.concatenate([bits, specials]).view(np.float32)
    f = f[~np.isnan(f)]
    got = orc.bf16_round(f.astype(np.float64))
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, t)


def _round_to_odd_f32(x):
    """fp64 -> fp32 with round-to-odd (truncate, then set the last bit if inexact)."""
    t = x.astype(np.float32)
    back = t.astype(np.float64)
    inexact = back != x
    over = np.abs(back) > np.abs(x)
    t = np.where(inexact & over, np.nextafter(t, np.float32(0)), t)
    b = t.view(np.uint32) | inexact.astype(np.uint32)
    return b.view(np.float32)


def test_bf16_round_matches_round_to_odd_route(orc):
    """One-step RNE of a double equals RNE(bf16) of its round-to-odd fp32 image
    (round-to-odd with >= 2 extra bits makes the double rounding innocuous)."""
    g = np.random.default_rng(8)
    x = g.standard_normal(1 << 20) * np.exp(g.uniform(-80, 80, 1 << 20))
    # doubles exactly on and next to bf16 rounding midpoints
    base = g.standard_normal(4096).astype(np.float32)
    bb = (base.view(np.uint32) & 0xFFFF0000) | 0x8000
    mid = bb.view(np.float32).astype(np.float64)
    x = np.concatenate([x, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    got = orc.bf16_round(x)
    ro = _round_to_odd_f32(x)
    t = torch.from_numpy(ro).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, t)
