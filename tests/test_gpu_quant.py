"""GPU quantizers against the CPU oracle: codes and scale bit patterns must be
identical (padding bytes included).  Small ragged shapes first, then the full
quant-stress and linear workloads."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import assert_codes_equal, assert_scales_equal, bf16_dev, u8_dev, f32_dev, host

pytestmark = pytest.mark.gpu
T = 128


def stress(R, C, seed):
    """Mixed magnitudes, signed zeros, zero tiles, tiny negatives, bf16 subnormals."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((R, C)).astype(np.float32) * np.power(10.0, g.uniform(-6, 3, (R, 1))).astype(np.float32)
    x[g.random((R, C)) < 0.02] = -0.0
    x[g.random((R, C)) < 0.02] = 0.0
    x[: min(R, 3), : min(C, 128)] = 0.0
    if R > 130 and C > 2:
        x[:128, 1] = -0.0
    tiny = g.random((R, C)) < 0.01
    x[tiny] = -np.abs(x[tiny]) * 1e-7
    bits = wl.bf16_bits(x)
    sub = g.random((R, C)) < 0.001
    bits[sub] = (0x8000 | g.integers(1, 0x80, int(sub.sum()))).astype(np.uint16)
    return bits


SMALL = [(1, 128), (3, 8), (130, 200), (64, 384), (257, 136), (128, 128), (5, 1024)]


@pytest.mark.parametrize("R,C", SMALL)
def test_1x128_small(orc, R, C):
    x = stress(R, C, 1000 + R * 7 + C)
    q, s = fgb.quantize_1x128(bf16_dev(x))
    oq, os_ = orc.quantize_1x128(x)
    assert_codes_equal(q, oq, f"q[{R}x{C}]")
    assert_scales_equal(s, os_, f"s[{R}x{C}]")


@pytest.mark.parametrize("R,C", SMALL)
def test_128x1_small(orc, R, C):
    x = stress(R, C, 2000 + R * 7 + C)
    qT, sT = fgb.quantize_128x1(bf16_dev(x))
    oqT, osT = orc.quantize_128x1(x)
    assert_codes_equal(qT, oqT, f"qT[{R}x{C}]")
    assert_scales_equal(sT, osT, f"sT[{R}x{C}]")


@pytest.mark.parametrize("R,C", SMALL)
def test_dual_small(orc, R, C):
    """One read, both orientations: each output equals the oracle's 1x128 or 128x1 result."""
    x = stress(R, C, 2500 + R * 7 + C)
    q, s, qT, sT = fgb.quantize_dual(bf16_dev(x))
    oq, os_ = orc.quantize_1x128(x)
    oqT, osT = orc.quantize_128x1(x)
    assert_codes_equal(q, oq, f"dual q[{R}x{C}]")
    assert_scales_equal(s, os_, f"dual s[{R}x{C}]")
    assert_codes_equal(qT, oqT, f"dual qT[{R}x{C}]")
    assert_scales_equal(sT, osT, f"dual sT[{R}x{C}]")


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384), (384, 128)])
def test_128x128_small(orc, K, N):
    w = stress(K, N, 3000 + K + N)
    q, qT, s = fgb.quantize_128x128(bf16_dev(w))
    oq, oqT, os_ = orc.quantize_128x128(w)
    assert_codes_equal(q, oq, "q")
    assert_codes_equal(qT, oqT, "qT")
    assert_scales_equal(s, os_, "s")
    # one layout at a time
    q1, qT1, s1 = fgb.quantize_128x128(bf16_dev(w), want_qT=False)
    assert qT1 is None
    assert_codes_equal(q1, oq, "q only")
    q2, qT2, s2 = fgb.quantize_128x128(bf16_dev(w), want_q=False)
    assert q2 is None
    assert_codes_equal(qT2, oqT, "qT only")
    assert_scales_equal(s2, os_, "s (qT only)")


@pytest.mark.parametrize("R,C", [(200, 256), (300, 136), (1, 8), (128, 1024)])
def test_requant_small(orc, R, C):
    x = stress(R, C, 4000 + R + C)
    oq, os_ = orc.quantize_1x128(x)
    qT, sT = fgb.requant_128x1(u8_dev(oq), f32_dev(os_))
    oqT, osT = orc.requant_128x1(oq, os_)
    assert_codes_equal(qT, oqT, "qT")
    assert_scales_equal(sT, osT, "sT")


def test_amax_floor(orc):
    x = stress(130, 256, 5)
    for fl in (1e-4, 3.0):
        q, s = fgb.quantize_1x128(bf16_dev(x), amax_floor=fl)
        oq, os_ = orc.quantize_1x128(x, amax_floor=fl)
        assert_codes_equal(q, oq, f"q floor {fl}")
        assert_scales_equal(s, os_, f"s floor {fl}")
        qT, sT = fgb.quantize_128x1(bf16_dev(x), amax_floor=fl)
        oqT, osT = orc.quantize_128x1(x, amax_floor=fl)
        assert_codes_equal(qT, oqT, f"qT floor {fl}")
        assert_scales_equal(sT, osT, f"sT floor {fl}")
        q, s, qT, sT = fgb.quantize_dual(bf16_dev(x), amax_floor=fl)
        assert_codes_equal(q, oq, f"dual q floor {fl}")
        assert_scales_equal(s, os_, f"dual s floor {fl}")
        assert_codes_equal(qT, oqT, f"dual qT floor {fl}")
        assert_scales_equal(sT, osT, f"dual sT floor {fl}")
    w = stress(256, 256, 6)
    q, qT, s = fgb.quantize_128x128(bf16_dev(w), amax_floor=2.0)
    oq, oqT, os_ = orc.quantize_128x128(w, amax_floor=2.0)
    assert_codes_equal(q, oq, "q floor")
    assert_scales_equal(s, os_, "s floor")


def test_strided_operands(orc):
    """Row strides larger than the row: inputs and outputs are views of wider buffers."""
    R, C = 150, 256
    x = stress(R, C, 7)
    wide = torch.zeros((R, C + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :C] = bf16_dev(x)
    qbuf = torch.full((R, C + 32), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.zeros((2, R + 10), dtype=torch.float32, device="cuda")
    fgb.quantize_1x128(wide[:, :C], q=qbuf[:, :C], s=sbuf[:, :R])
    oq, os_ = orc.quantize_1x128(x)
    assert_codes_equal(qbuf[:, :C], oq, "q strided")
    assert np.all(host(qbuf[:, C:]) == 0xAB), "wrote outside the view"
    assert_scales_equal(sbuf[:, :R], os_, "s strided")
    qTbuf = torch.full((C, 384), 0xCD, dtype=torch.uint8, device="cuda")
    fgb.quantize_128x1(wide[:, :C], qT=qTbuf[:, :256])
    oqT, _ = orc.quantize_128x1(x)
    assert_codes_equal(qTbuf[:, :256], oqT, "qT strided")
    assert np.all(host(qTbuf[:, 256:]) == 0xCD)
    # dual: all four outputs as views of wider buffers
    qbuf.fill_(0xAB)
    qTbuf.fill_(0xCD)
    sbuf.zero_()
    sTbuf = torch.zeros((2, C + 8), dtype=torch.float32, device="cuda")
    fgb.quantize_dual(wide[:, :C], q=qbuf[:, :C], s=sbuf[:, :R], qT=qTbuf[:, :256], sT=sTbuf[:, :C])
    _, osT = orc.quantize_128x1(x)
    assert_codes_equal(qbuf[:, :C], oq, "dual q strided")
    assert_scales_equal(sbuf[:, :R], os_, "dual s strided")
    assert_codes_equal(qTbuf[:, :256], oqT, "dual qT strided")
    assert_scales_equal(sTbuf[:, :C], osT, "dual sT strided")
    assert np.all(host(qbuf[:, C:]) == 0xAB) and np.all(host(qTbuf[:, 256:]) == 0xCD)
    assert np.all(host(sbuf[:, R:]) == 0) and np.all(host(sTbuf[:, C:]) == 0)


@pytest.mark.parametrize("R,C,ld", [(300, 4096, 4096), (257, 8192, 8192), (200, 1000, 4096), (384, 4096, 4096),
                                    (256, 1024, 4096)])
def test_pitch_multiple_of_8k(orc, R, C, ld):
    """Row pitches that are multiples of 8 KB, where the 128x128 and dual casts run
    their blocks column-first (the other pitches run them row-first): ragged rows, and
    a view of C columns of a wider buffer (ragged last column tile); the weight cast
    where the shape is whole 128x128 tiles (it requires them).  Bit-exact."""
    x = stress(R, C, 4100 + R + C)
    buf = torch.zeros((R, ld), dtype=torch.bfloat16, device="cuda")
    buf[:, :C] = bf16_dev(x)
    xv = buf[:, :C]
    oq, os_ = orc.quantize_1x128(x)
    oqT, osT = orc.quantize_128x1(x)
    q, s, qT, sT = fgb.quantize_dual(xv)
    assert_codes_equal(q, oq, f"dual q[{R}x{C}/{ld}]")
    assert_scales_equal(s, os_, f"dual s[{R}x{C}/{ld}]")
    assert_codes_equal(qT, oqT, f"dual qT[{R}x{C}/{ld}]")
    assert_scales_equal(sT, osT, f"dual sT[{R}x{C}/{ld}]")
    q1, s1 = fgb.quantize_1x128(xv)
    assert_codes_equal(q1, oq, f"1x128 q[{R}x{C}/{ld}]")
    assert_scales_equal(s1, os_, f"1x128 s[{R}x{C}/{ld}]")
    if R % 128 or C % 128:
        return
    wq, wqT, ws = fgb.quantize_128x128(xv)
    owq, owqT, ows = orc.quantize_128x128(x)
    assert_codes_equal(wq, owq, f"128x128 q[{R}x{C}/{ld}]")
    assert_codes_equal(wqT, owqT, f"128x128 qT[{R}x{C}/{ld}]")
    assert_scales_equal(ws, ows, f"128x128 s[{R}x{C}/{ld}]")


def test_128x128_pitch_8k_single_and_batched(orc):
    """The 128x128 cast at an 8 KB pitch (column-first blocks), one matrix and a stack."""
    E, K, N = 2, 384, 4096
    ws = [stress(K, N, 4200 + e) for e in range(E)]
    for e in range(E):
        q, qT, s = fgb.quantize_128x128(bf16_dev(ws[e]))
        oq, oqT, os_ = orc.quantize_128x128(ws[e])
        assert_codes_equal(q, oq, f"single q[{e}]")
        assert_codes_equal(qT, oqT, f"single qT[{e}]")
        assert_scales_equal(s, os_, f"single s[{e}]")
    q, qT, s = fgb.quantize_128x128_batched(torch.stack([bf16_dev(x) for x in ws]))
    for e in range(E):
        oq, oqT, os_ = orc.quantize_128x128(ws[e])
        assert_codes_equal(q[e], oq, f"batched q[{e}]")
        assert_codes_equal(qT[e], oqT, f"batched qT[{e}]")
        assert_scales_equal(s[e], os_, f"batched s[{e}]")


def test_deterministic_repeat():
    x = bf16_dev(stress(512, 1024, 8))
    a = [fgb.quantize_1x128(x), fgb.quantize_1x128(x)]
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])
    b = [fgb.quantize_128x1(x), fgb.quantize_128x1(x)]
    assert torch.equal(b[0][0], b[1][0]) and torch.equal(b[0][1], b[1][1])


# ---------------------------------------------------------------------------
# full workloads
# ---------------------------------------------------------------------------

def test_quant_stress_full(orc):
    """Workload 5: [16384, 7168], all three tilings plus requant, bit-exact."""
    d = wl.quant_stress()
    x = d["x"]
    xd = bf16_dev(x)
    q, s = fgb.quantize_1x128(xd)
    oq, os_ = orc.quantize_1x128(x)
    assert_codes_equal(q, oq, "stress 1x128 q")
    assert_scales_equal(s, os_, "stress 1x128 s")
    assert int((oq == 0x80).sum()) > 0
    qT, sT = fgb.quantize_128x1(xd)
    oqT, osT = orc.quantize_128x1(x)
    assert_codes_equal(qT, oqT, "stress 128x1 qT")
    assert_scales_equal(sT, osT, "stress 128x1 sT")
    dq, ds, dqT, dsT = fgb.quantize_dual(xd)
    assert_codes_equal(dq, oq, "stress dual q")
    assert_scales_equal(ds, os_, "stress dual s")
    assert_codes_equal(dqT, oqT, "stress dual qT")
    assert_scales_equal(dsT, osT, "stress dual sT")
    del qT, sT, oqT, osT, dq, ds, dqT, dsT
    qw, qwT, sw = fgb.quantize_128x128(xd)
    oqw, oqwT, osw = orc.quantize_128x128(x)
    assert_codes_equal(qw, oqw, "stress 128x128 q")
    assert_codes_equal(qwT, oqwT, "stress 128x128 qT")
    assert_scales_equal(sw, osw, "stress 128x128 s")
    del qw, qwT, oqw, oqwT
    rq, rs = fgb.requant_128x1(q, s)
    orq, ors = orc.requant_128x1(oq, os_)
    assert_codes_equal(rq, orq, "stress requant qT")
    assert_scales_equal(rs, ors, "stress requant sT")


def test_linear_workload_quantizers_full(orc):
    """Workload 2 operands: X and dY 1x128, W 128x128 (both layouts), dY 128x1, requant X."""
    d = wl.linear_dsv3_attn()
    for name in ("x", "dy"):
        q, s = fgb.quantize_1x128(bf16_dev(d[name]))
        oq, os_ = orc.quantize_1x128(d[name])
        assert_codes_equal(q, oq, f"{name} 1x128")
        assert_scales_equal(s, os_, f"{name} 1x128 s")
        if name == "x":
            rq, rs = fgb.requant_128x1(q, s)
            orq, ors = orc.requant_128x1(oq, os_)
            assert_codes_equal(rq, orq, "x requant")
            assert_scales_equal(rs, ors, "x requant s")
    qT, sT = fgb.quantize_128x1(bf16_dev(d["dy"]))
    oqT, osT = orc.quantize_128x1(d["dy"])
    assert_codes_equal(qT, oqT, "dy 128x1")
    assert_scales_equal(sT, osT, "dy 128x1 s")
    q, s, qT, sT = fgb.quantize_dual(bf16_dev(d["dy"]))
    oq, os_ = orc.quantize_1x128(d["dy"])
    assert_codes_equal(q, oq, "dy dual 1x128")
    assert_scales_equal(s, os_, "dy dual 1x128 s")
    assert_codes_equal(qT, oqT, "dy dual 128x1")
    assert_scales_equal(sT, osT, "dy dual 128x1 s")
    q, qT, s = fgb.quantize_128x128(bf16_dev(d["w"]))
    oq, oqT, os_ = orc.quantize_128x128(d["w"])
    assert_codes_equal(q, oq, "w q")
    assert_codes_equal(qT, oqT, "w qT")
    assert_scales_equal(s, os_, "w s")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_128x128_batched_equals_single(orc, ue8m0):
    """A stack of E weights in one launch: every matrix bit-exact against the
    oracle's single-matrix quantization (fp32 scales, or E8M0 bytes)."""
    E, K, N = 3, 256, 384
    ws = [stress(K, N, 9600 + e) for e in range(E)]
    w = torch.stack([bf16_dev(x) for x in ws])
    q, qT, s = fgb.quantize_128x128_batched(w, ue8m0=ue8m0)
    for e in range(E):
        if ue8m0:
            oq, oqT, oe = orc.quantize_128x128_ue8m0(ws[e])
            os_ = orc.e8m0_decode(oe).astype(np.float32)
        else:
            oq, oqT, os_ = orc.quantize_128x128(ws[e])
        assert_codes_equal(q[e], oq, f"batched q[{e}]")
        assert_codes_equal(qT[e], oqT, f"batched qT[{e}]")
        assert_scales_equal(s[e], os_, f"batched s[{e}]")


# ---------------------------------------------------------------------------
# beyond 2^31 elements: the bf16 input is larger than 4 GiB
# ---------------------------------------------------------------------------

def wide_table():
    """bf16 bit patterns of 16 magnitude decades x 4096 Gaussian quantiles (and
    +-0): a uniformly drawn 16-bit index maps to a value of mixed magnitude."""
    from scipy.special import ndtri
    z = ndtri((np.arange(4096) + 0.5) / 4096.0)
    t = (z[None, :] * np.power(10.0, np.linspace(-4.0, 2.0, 16))[:, None]).ravel().astype(np.float32)
    t[0], t[1] = 0.0, -0.0
    return wl.bf16_bits(t)


def test_quantizers_beyond_2g_elements(orc):
    """X [300001, 7168] bf16 (4.30 GB, 2.15e9 elements): 1x128, 128x1, dual and
    requant on all of it, 128x128 on its first 299904 rows.  Bit-exact against
    the oracle on sampled rows (1x128) and 128-row blocks (the rest): the row
    that holds element 2^31, its neighbours and the ragged last block."""
    g = np.random.default_rng(31)
    R, C = 300001, 7168
    assert R * C > (1 << 31) and 299904 * C > (1 << 31)
    table = wide_table()
    print(f"generating {R * C * 2 / 1e9:.2f} GB of bf16 input", flush=True)
    x = np.empty((R, C), np.uint16)
    for r0 in range(0, R, 1 << 14):
        n = min(1 << 14, R - r0)
        x[r0:r0 + n] = table[g.integers(0, 1 << 16, (n, C), dtype=np.uint16)]
    rb = (1 << 31) // C                              # the row that holds element 2^31
    rows = np.unique(np.concatenate([[0, 1, rb - 1, rb, rb + 1, R - 2, R - 1], g.choice(R, 40, replace=False)]))
    blocks = sorted({0, rb // T, (R - 1) // T, *g.choice(R // T, 2, replace=False).tolist()})
    xd = bf16_dev(x)
    ri = torch.as_tensor(rows, device=xd.device)

    def block_cols(t, b):                            # columns of one 128-row block of a [C, Rp] output
        return t[:, b * T:(b + 1) * T]

    q, s = fgb.quantize_1x128(xd)
    oq, os_ = orc.quantize_1x128(x[rows])
    assert_codes_equal(q[ri], oq, "1x128 q beyond 2^31")
    assert_scales_equal(s[:, ri], os_, "1x128 s beyond 2^31")
    rq, rs = fgb.requant_128x1(q, s)
    for b in blocks:
        xb = x[b * T:min((b + 1) * T, R)]
        orq, ors = orc.requant_128x1(*orc.quantize_1x128(xb))
        assert_codes_equal(block_cols(rq, b), orq, f"requant qT block {b}")
        assert_scales_equal(rs[b:b + 1], ors, f"requant sT block {b}")
    del q, s, rq, rs
    qT, sT = fgb.quantize_128x1(xd)
    dq, ds, dqT, dsT = fgb.quantize_dual(xd)
    assert_codes_equal(dq[ri], oq, "dual q beyond 2^31")
    assert_scales_equal(ds[:, ri], os_, "dual s beyond 2^31")
    del dq, ds
    for b in blocks:
        oqT, osT = orc.quantize_128x1(x[b * T:min((b + 1) * T, R)])
        assert_codes_equal(block_cols(qT, b), oqT, f"128x1 qT block {b}")
        assert_scales_equal(sT[b:b + 1], osT, f"128x1 sT block {b}")
        assert_codes_equal(block_cols(dqT, b), oqT, f"dual qT block {b}")
        assert_scales_equal(dsT[b:b + 1], osT, f"dual sT block {b}")
    del qT, sT, dqT, dsT
    K = 299904
    qw, qwT, sw = fgb.quantize_128x128(xd[:K])
    for b in sorted({0, rb // T, K // T - 1}):
        oqw, oqwT, osw = orc.quantize_128x128(x[b * T:(b + 1) * T])
        assert_codes_equal(qw[b * T:(b + 1) * T], oqw, f"128x128 q block {b}")
        assert_codes_equal(block_cols(qwT, b), oqwT, f"128x128 qT block {b}")
        assert_scales_equal(sw[b:b + 1], osw, f"128x128 s block {b}")


def test_128x128_batched_floor(orc):
    """The batched weight cast with an absmax floor: every matrix as the oracle's
    single-matrix quantization under the same floor."""
    E, K, N = 3, 256, 384
    ws = [stress(K, N, 9700 + e) for e in range(E)]
    w = torch.stack([bf16_dev(x) for x in ws])
    q, qT, s = fgb.quantize_128x128_batched(w, amax_floor=2.0)
    for e in range(E):
        oq, oqT, os_ = orc.quantize_128x128(ws[e], amax_floor=2.0)
        assert_codes_equal(q[e], oq, f"batched floor q[{e}]")
        assert_codes_equal(qT[e], oqT, f"batched floor qT[{e}]")
        assert_scales_equal(s[e], os_, f"batched floor s[{e}]")


def test_128x128_batched_beyond_4gib(orc):
    """The batched weight cast over 80 experts of [7168, 4096] (4.70 GB of bf16,
    2.35e9 elements): the first expert, the one that holds element 2^31 and the
    last, bit-exact against the oracle's single-matrix quantization."""
    g = np.random.default_rng(41)
    E, K, N = 80, 7168, 4096
    assert E * K * N > (1 << 31) and E * K * N * 2 > (1 << 32)
    table = wide_table()
    print(f"generating {E * K * N * 2 / 1e9:.2f} GB of bf16 weights", flush=True)
    w = np.empty((E, K, N), np.uint16)
    for e in range(E):
        w[e] = table[g.integers(0, 1 << 16, (K, N), dtype=np.uint16)]
    q, qT, s = fgb.quantize_128x128_batched(bf16_dev(w.reshape(E * K, N)).view(E, K, N))
    for e in (0, (1 << 31) // (K * N), E - 1):
        oq, oqT, os_ = orc.quantize_128x128(w[e])
        assert_codes_equal(q[e], oq, f"batched q[{e}]")
        assert_codes_equal(qT[e], oqT, f"batched qT[{e}]")
        assert_scales_equal(s[e], os_, f"batched s[{e}]")
