"""GPU block-scaled GEMMs against the CPU oracle.

Acceptance per output (tests/parity.py gemm_bound): the matrix core's in-block
truncation bound computed from the operands, plus fp32 rounding of the
promotion chain, plus half a bf16 ulp of r for BF16 outputs (Fprop, Dgrad);
r is the oracle's exact-to-fp64 value.
Small shapes are compared on every output; the full workloads on sampled rows
and columns (edges and tile boundaries included)."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import (assert_codes_equal, assert_scales_equal, bf16_dev, bf16_host_f64, check_gemm, f32_dev,
                    host, hw_bound_dgrad, hw_bound_fprop, hw_bound_wgrad, model_dgrad, model_fprop, model_wgrad,
                    sample_idx, u8_dev)

pytestmark = pytest.mark.gpu
T = 128


def rand_codes(g, shape):
    c = g.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C
    return c


def rand_scales(g, shape):
    return np.exp(g.uniform(-10, 2, shape)).astype(np.float32)


# ---------------------------------------------------------------------------
# arbitrary codes and scales, every output compared
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 384, 640), (1, 128, 128), (129, 256, 256),
                                   (64, 128, 0), (513, 640, 1152), (300, 896, 256), (700, 1792, 384)])
def test_fprop_small(orc, M, N, K):
    g = np.random.default_rng(M * 31 + N * 7 + K)
    qx, qwT = rand_codes(g, (M, K)), rand_codes(g, (N, K))
    sx, sw = rand_scales(g, (K // T, M)), rand_scales(g, (K // T, N // T))
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw))
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw)
    check_gemm(bf16_host_f64(y), r, aabs, True, f"fprop {M}x{N}x{K}", hw_bound_fprop(qx, sx, qwT, sw), K // T, stated=False)


@pytest.mark.parametrize("M,K,N", [(300, 384, 640), (1, 128, 128), (200, 256, 1152), (333, 896, 384)])
def test_dgrad_small(orc, M, K, N):
    g = np.random.default_rng(M * 13 + N * 5 + K)
    qdy, qw = rand_codes(g, (M, N)), rand_codes(g, (K, N))
    sdy, sw = rand_scales(g, (N // T, M)), rand_scales(g, (K // T, N // T))
    dx = fgb.gemm_dgrad(u8_dev(qdy), f32_dev(sdy), u8_dev(qw), f32_dev(sw))
    r, aabs = orc.gemm_dgrad(qdy, sdy, qw, sw)
    check_gemm(bf16_host_f64(dx), r, aabs, True, f"dgrad {M}x{K}x{N}", hw_bound_dgrad(qdy, sdy, qw, sw), N // T, stated=False)


@pytest.mark.parametrize("K,N,M", [(256, 384, 300), (128, 128, 1), (384, 256, 1024), (128, 256, 129),
                                   (256, 896, 300), (896, 896, 200)])
def test_wgrad_small(orc, K, N, M):
    g = np.random.default_rng(K * 3 + N * 11 + M)
    Mp = -(-M // T) * T
    qxT, qdyT = rand_codes(g, (K, Mp)), rand_codes(g, (N, Mp))
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    nb = Mp // T
    sxT, sdyT = rand_scales(g, (nb, K)), rand_scales(g, (nb, N))
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M)
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M)
    hw = hw_bound_wgrad(qxT, sxT, qdyT, sdyT, M)
    check_gemm(host(dw), r, aabs, False, f"wgrad {K}x{N}x{M}", hw, nb, stated=False)
    # accumulate: dW += X^T dY
    prev = g.standard_normal((K, N)).astype(np.float32)
    dw2 = f32_dev(prev)
    fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M, dw=dw2, accumulate=True)
    check_gemm(host(dw2), r + prev, aabs + np.abs(prev), False, "wgrad accumulate", hw, nb + 1, stated=False)


@pytest.mark.parametrize("M,N", [(2048, 8448)])
def test_tail_round_split(orc, M, N):
    """A dense grid of 8 x 33 = 264 tiles of 256 x 256 on 256 CUs: the 8 tiles
    beyond the first round are computed as column halves by 16 blocks.  Fprop
    and Wgrad, every output compared."""
    g = np.random.default_rng(M + N)
    K = 128
    qx, qwT = rand_codes(g, (M, K)), rand_codes(g, (N, K))
    sx, sw = rand_scales(g, (K // T, M)), rand_scales(g, (K // T, N // T))
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw))
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw)
    check_gemm(bf16_host_f64(y), r, aabs, True, f"fprop {M}x{N}x{K}", hw_bound_fprop(qx, sx, qwT, sw), K // T, stated=False)
    Mc = 200                                        # Wgrad contraction, ragged
    Mp = T * 2
    qxT, qdyT = rand_codes(g, (M, Mp)), rand_codes(g, (N, Mp))
    qxT[:, Mc:] = 0
    qdyT[:, Mc:] = 0
    sxT, sdyT = rand_scales(g, (2, M)), rand_scales(g, (2, N))
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), Mc)
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, Mc)
    check_gemm(host(dw), r, aabs, False, f"wgrad {M}x{N}x{Mc}", hw_bound_wgrad(qxT, sxT, qdyT, sdyT, Mc), 2, stated=False)


@pytest.mark.parametrize("K,N,M", [(7168, 7168, 4096), (2432, 4608, 777)])
def test_wgrad_accumulate_multi_tile(orc, K, N, M):
    """Accumulating Wgrad over many tiles: at 7168 x 7168 over 4096 tokens (3
    rounds of 256 x 224 tiles plus 128 tiles run as column halves) and on a
    ragged 10 x 18 tile grid.  Sampled outputs against the oracle's X^T dY plus
    the old contents; every output against the property that the accumulating
    call adds the old value to the plain call's result in one fp32 addition."""
    g = np.random.default_rng(K + 3 * N + 7 * M)
    Mp = -(-M // T) * T
    nb = Mp // T
    qxT, qdyT = rand_codes(g, (K, Mp)), rand_codes(g, (N, Mp))
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    sxT, sdyT = rand_scales(g, (nb, K)), rand_scales(g, (nb, N))
    prev = g.standard_normal((K, N)).astype(np.float32)
    a, sa, b, sb = u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT)
    plain = fgb.gemm_wgrad(a, sa, b, sb, M)
    acc = f32_dev(prev)
    fgb.gemm_wgrad(a, sa, b, sb, M, dw=acc, accumulate=True)
    torch.cuda.synchronize()
    want = plain + f32_dev(prev)
    bad = int((want.view(torch.int32) != acc.view(torch.int32)).sum())
    assert bad == 0, f"{bad} outputs differ from the plain result plus the old value"
    rows, cols = sample_idx(K, 80, K), sample_idx(N, 80, N)
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols)
    hw = hw_bound_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols)
    pv = prev[np.ix_(rows, cols)].astype(np.float64)
    check_gemm(host(acc)[np.ix_(rows, cols)], r + pv, aabs + np.abs(pv), False,
               f"wgrad accumulate {K}x{N}x{M}", hw, nb + 1, stated=False)


SMALL_INT_CODES = np.array([0x00, 0x80, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8, 0x4C, 0xCC, 0x50, 0xD0],
                           np.uint8)   # 0, -0, +-1, +-2, +-3, +-4, +-6, +-8


@pytest.mark.parametrize("M,N,K", [(300, 384, 640), (129, 256, 2048), (300, 896, 512)])
def test_exact_mma_all_kinds(orc, M, N, K):
    """Operands whose products stay inside the matrix core's exact window (every
    product is a small integer, so no in-block truncation): Fprop and Wgrad must
    equal the oracle up to fp32 rounding of the promotion chain (hw bound = 0)."""
    g = np.random.default_rng(M + N + K)
    pick = lambda shape: SMALL_INT_CODES[g.integers(0, SMALL_INT_CODES.size, shape)]
    qx, qwT = pick((M, K)), pick((N, K))
    sx, sw = rand_scales(g, (K // T, M)), rand_scales(g, (K // T, N // T))
    assert np.all(hw_bound_fprop(qx, sx, qwT, sw, np.arange(4), np.arange(4)) == 0)
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw))
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw)
    check_gemm(bf16_host_f64(y), r, aabs, True, "exact-mma fprop", np.zeros_like(r), K // T)
    Mp = -(-M // T) * T
    qxT, qdyT = pick((K, Mp)), pick((N, Mp))
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    sxT, sdyT = rand_scales(g, (Mp // T, K)), rand_scales(g, (Mp // T, N))
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M)
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M)
    check_gemm(host(dw), r, aabs, False, "exact-mma wgrad", np.zeros_like(r), Mp // T)


def test_exact_mma_dgrad(orc):
    g = np.random.default_rng(77)
    M, K, N = 257, 384, 1024
    pick = lambda shape: SMALL_INT_CODES[g.integers(0, SMALL_INT_CODES.size, shape)]
    qdy, qw = pick((M, N)), pick((K, N))
    sdy, sw = rand_scales(g, (N // T, M)), rand_scales(g, (K // T, N // T))
    dx = fgb.gemm_dgrad(u8_dev(qdy), f32_dev(sdy), u8_dev(qw), f32_dev(sw))
    r, aabs = orc.gemm_dgrad(qdy, sdy, qw, sw)
    check_gemm(bf16_host_f64(dx), r, aabs, True, "exact-mma dgrad", np.zeros_like(r), N // T)


def test_wgrad_empty_contraction(orc):
    K, N = 128, 256
    z = torch.zeros((K, 0), dtype=torch.uint8, device="cuda")
    zs = torch.zeros((0, K), dtype=torch.float32, device="cuda")
    dw = torch.full((K, N), 7.0, device="cuda")
    fgb.gemm_wgrad(z, zs, torch.zeros((N, 0), dtype=torch.uint8, device="cuda"),
                   torch.zeros((0, N), dtype=torch.float32, device="cuda"), 0, dw=dw)
    assert torch.all(dw == 0)
    dw.fill_(7.0)
    fgb.gemm_wgrad(z, zs, torch.zeros((N, 0), dtype=torch.uint8, device="cuda"),
                   torch.zeros((0, N), dtype=torch.float32, device="cuda"), 0, dw=dw, accumulate=True)
    assert torch.all(dw == 7.0)


def test_strided_gemm(orc):
    """Operand and output row strides larger than the row."""
    g = np.random.default_rng(5)
    M, N, K = 200, 256, 384
    qx, qwT = rand_codes(g, (M, K)), rand_codes(g, (N, K))
    sx, sw = rand_scales(g, (K // T, M)), rand_scales(g, (K // T, N // T))
    qxb = torch.zeros((M, K + 128), dtype=torch.uint8, device="cuda")
    qxb[:, :K] = u8_dev(qx)
    sxb = torch.zeros((K // T, M + 8), dtype=torch.float32, device="cuda")
    sxb[:, :M] = f32_dev(sx)
    yb = torch.zeros((M, N + 64), dtype=torch.bfloat16, device="cuda")
    fgb.gemm_fprop(qxb[:, :K], sxb[:, :M], u8_dev(qwT), f32_dev(sw), y=yb[:, :N])
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw)
    check_gemm(bf16_host_f64(yb[:, :N]), r, aabs, True, "fprop strided", hw_bound_fprop(qx, sx, qwT, sw), K // T, stated=False)
    assert torch.all(yb[:, N:] == 0)


def test_gemm_deterministic():
    g = np.random.default_rng(9)
    M, N, K = 512, 512, 1024
    qx, qwT = u8_dev(rand_codes(g, (M, K))), u8_dev(rand_codes(g, (N, K)))
    sx, sw = f32_dev(rand_scales(g, (K // T, M))), f32_dev(rand_scales(g, (K // T, N // T)))
    a = fgb.gemm_fprop(qx, sx, qwT, sw)
    b = fgb.gemm_fprop(qx, sx, qwT, sw)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# the whole path from bf16 inputs
# ---------------------------------------------------------------------------

def run_linear(d):
    """Quantize and run Fprop, Dgrad, Wgrad on the GPU; return everything."""
    x, w, dy = bf16_dev(d["x"]), bf16_dev(d["w"]), bf16_dev(d["dy"])
    out = {}
    out["qx"], out["sx"] = fgb.quantize_1x128(x)
    out["qw"], out["qwT"], out["sw"] = fgb.quantize_128x128(w)
    out["y"] = fgb.gemm_fprop(out["qx"], out["sx"], out["qwT"], out["sw"])
    out["qdy"], out["sdy"] = fgb.quantize_1x128(dy)
    out["dx"] = fgb.gemm_dgrad(out["qdy"], out["sdy"], out["qw"], out["sw"])
    out["qdyT"], out["sdyT"] = fgb.quantize_128x1(dy)
    out["qxT"], out["sxT"] = fgb.requant_128x1(out["qx"], out["sx"])
    out["dw"] = fgb.gemm_wgrad(out["qxT"], out["sxT"], out["qdyT"], out["sdyT"], d["M"])
    torch.cuda.synchronize()
    return out


def check_linear(orc, d, k_rows, k_cols, seed, full=False):
    g = run_linear(d)
    o = {}
    o["qx"], o["sx"] = orc.quantize_1x128(d["x"])
    o["qw"], o["qwT"], o["sw"] = orc.quantize_128x128(d["w"])
    o["qdy"], o["sdy"] = orc.quantize_1x128(d["dy"])
    o["qdyT"], o["sdyT"] = orc.quantize_128x1(d["dy"])
    o["qxT"], o["sxT"] = orc.requant_128x1(o["qx"], o["sx"])
    for k in ("qx", "qw", "qwT", "qdy", "qdyT", "qxT"):
        assert_codes_equal(g[k], o[k], k)
    for k in ("sx", "sw", "sdy", "sdyT", "sxT"):
        assert_scales_equal(g[k], o[k], k)
    M, K, N = d["M"], d["K"], d["N"]
    rows = None if full else sample_idx(M, k_rows, seed)
    colsN = None if full else sample_idx(N, k_cols, seed + 1)
    colsK = None if full else sample_idx(K, k_cols, seed + 2)
    pick = lambda a, r, c: a if r is None else a[np.ix_(r, c)]
    r, aabs = orc.gemm_fprop(o["qx"], o["sx"], o["qwT"], o["sw"], rows, colsN)
    hw = hw_bound_fprop(o["qx"], o["sx"], o["qwT"], o["sw"], rows, colsN)
    check_gemm(pick(bf16_host_f64(g["y"]), rows, colsN), r, aabs, True, "fprop", hw, K // T,
               model=model_fprop(o["qx"], o["sx"], o["qwT"], o["sw"], rows, colsN))
    r, aabs = orc.gemm_dgrad(o["qdy"], o["sdy"], o["qw"], o["sw"], rows, colsK)
    hw = hw_bound_dgrad(o["qdy"], o["sdy"], o["qw"], o["sw"], rows, colsK)
    check_gemm(pick(bf16_host_f64(g["dx"]), rows, colsK), r, aabs, True, "dgrad", hw, N // T,
               model=model_dgrad(o["qdy"], o["sdy"], o["qw"], o["sw"], rows, colsK))
    rowsK = None if full else sample_idx(K, k_rows, seed + 3)
    r, aabs = orc.gemm_wgrad(o["qxT"], o["sxT"], o["qdyT"], o["sdyT"], M, rowsK, colsN)
    hw = hw_bound_wgrad(o["qxT"], o["sxT"], o["qdyT"], o["sdyT"], M, rowsK, colsN)
    check_gemm(pick(host(g["dw"]), rowsK, colsN), r, aabs, False, "wgrad", hw, -(-M // T),
               model=model_wgrad(o["qxT"], o["sxT"], o["qdyT"], o["sdyT"], M, rowsK, colsN))


def test_fprop_small_workload_full(orc):
    """Workload 1 (X [256,512] with 0.1 % x50 outliers, W [512,256]): every output."""
    d = wl.fprop_small()
    x, w = bf16_dev(d["x"]), bf16_dev(d["w"])
    qx, sx = fgb.quantize_1x128(x)
    qw, qwT, sw = fgb.quantize_128x128(w)
    y = fgb.gemm_fprop(qx, sx, qwT, sw)
    oqx, osx = orc.quantize_1x128(d["x"])
    oqw, oqwT, osw = orc.quantize_128x128(d["w"])
    assert_codes_equal(qx, oqx, "qx")
    assert_scales_equal(sx, osx, "sx")
    assert_codes_equal(qwT, oqwT, "qwT")
    r, aabs = orc.gemm_fprop(oqx, osx, oqwT, osw)
    check_gemm(bf16_host_f64(y), r, aabs, True, "workload-1 fprop", hw_bound_fprop(oqx, osx, oqwT, osw),
               d["K"] // T, model=model_fprop(oqx, osx, oqwT, osw))


def test_linear_ragged_full(orc):
    """A linear with a ragged token count, every output of all three GEMMs."""
    d = {"x": wl.normal_bf16((333, 384), 1.0, 90, 0), "w": wl.normal_bf16((384, 256), 0.02, 90, 1),
         "dy": wl.normal_bf16((333, 256), 1e-3, 90, 2), "M": 333, "K": 384, "N": 256}
    check_linear(orc, d, 0, 0, 0, full=True)


def test_linear_dsv3_attn_sampled(orc):
    """Workload 2: X [4096,7168], W [7168,7168], dY [4096,7168]; quantizers bit-exact,
    GEMMs on sampled rows/columns."""
    check_linear(orc, wl.linear_dsv3_attn(), 96, 96, 11)


def test_ffn_up_sampled(orc):
    """Workload 3 up projection: X [8192,7168] Student-t(3), W_up [7168,18432]."""
    check_linear(orc, wl.ffn_dense_up(), 64, 64, 21)


def test_ffn_down_sampled(orc):
    """Workload 3 down projection: contraction 18432 = 144 blocks."""
    check_linear(orc, wl.ffn_dense_down(), 64, 64, 31)


def test_zero_gradient_patterns(orc):
    """Leading zero rows, sparse zero rows, zero blocks, all-zero dY (TE PR #3573
    zero-gradient tests, adapted to 128 tiles): finite outputs, exact zeros."""
    g = np.random.default_rng(3)
    M, K, N = 384, 256, 384
    dy = g.standard_normal((M, N)).astype(np.float32) * 1e-3
    dy[:40] = 0.0
    dy[100:300:7] = 0.0
    dy[256:384, 128:256] = 0.0
    w = g.standard_normal((K, N)).astype(np.float32) * 0.02
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:17] = 0.0
    d = {"x": wl.bf16_bits(x), "w": wl.bf16_bits(w), "dy": wl.bf16_bits(dy), "M": M, "K": K, "N": N}
    out = run_linear(d)
    dx = bf16_host_f64(out["dx"])
    assert np.all(np.isfinite(dx)) and np.all(np.isfinite(host(out["dw"])))
    assert np.all(dx[np.all(dy == 0, axis=1)] == 0)
    assert np.all(bf16_host_f64(out["y"])[:17] == 0)
    d["dy"] = np.zeros((M, N), np.uint16)
    out = run_linear(d)
    assert torch.all(out["dw"] == 0) and torch.all(out["sdyT"] == 0)


# ---------------------------------------------------------------------------
# operands beyond 4 GiB: the host cuts the output into pieces whose operand
# slices fit the kernel's 32-bit offsets (rows of X, or columns of W)
# ---------------------------------------------------------------------------

def gauss_code_table():
    """E4M3 codes of 256 equally spaced quantiles of N(0, 160^2) clipped to +-448:
    a byte drawn uniformly maps to a code distributed like a quantized Gaussian
    tile (absmax near 448), the operating range of the method."""
    from scipy.special import ndtri
    z = ndtri((np.arange(256) + 0.5) / 256.0) * 160.0
    v = torch.from_numpy(np.clip(z, -448.0, 448.0).astype(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def big_codes(g, rows, cols):
    """Gaussian-distributed E4M3 codes, generated in row chunks to bound host memory."""
    table = gauss_code_table()
    c = np.empty((rows, cols), np.uint8)
    step = 1 << 16
    for r0 in range(0, rows, step):
        c[r0:r0 + min(step, rows - r0)] = table[g.integers(0, 256, (min(step, rows - r0), cols), dtype=np.uint8)]
    return c


@pytest.mark.parametrize("side", ["x_rows", "w_cols"])
def test_fprop_operand_beyond_4gib(orc, side):
    """Fprop with one operand of 4.43 GB: X [540672, 8192] (cut after row
    524288) or W^T [540672, 8192] (cut after column 523264).  Sampled outputs
    on both sides of the cut against the oracle."""
    g = np.random.default_rng(4242)
    K, big, small = 8192, 540672, 256
    M, N = (big, small) if side == "x_rows" else (small, big)
    print(f"[{side}] generating {max(M, N) * K / 1e9:.2f} GB of codes", flush=True)
    qx, qwT = big_codes(g, M, K), big_codes(g, N, K)
    sx, sw = rand_scales(g, (K // T, M)), rand_scales(g, (K // T, N // T))
    assert max(M, N) * K > (1 << 32)
    y = fgb.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qwT), f32_dev(sw))
    torch.cuda.synchronize()
    cut = 524288 if side == "x_rows" else 523264
    near = np.array([0, 1, cut - 2, cut - 1, cut, cut + 1, big - 2, big - 1], np.int64)
    wide = np.unique(np.concatenate([near, g.choice(big, 56, replace=False)]))
    rows = wide if side == "x_rows" else np.arange(M, dtype=np.int64)[::8]
    cols = np.arange(N, dtype=np.int64)[::8] if side == "x_rows" else wide
    r, aabs = orc.gemm_fprop(qx, sx, qwT, sw, rows=rows, cols=cols)
    ri, ci = torch.as_tensor(rows, device=y.device), torch.as_tensor(cols, device=y.device)
    got = bf16_host_f64(y[ri][:, ci].contiguous())
    check_gemm(got, r, aabs, True, f"fprop beyond 4 GiB ({side})",
               hw_bound_fprop(qx, sx, qwT, sw, rows=rows, cols=cols), K // T,
               model=model_fprop(qx, sx, qwT, sw, rows, cols))


def test_wgrad_operand_beyond_4gib(orc):
    """Wgrad over 600000 tokens (4688 contraction blocks): X^T [7168, 600064] is
    4.30 GB, so the host cuts dW's rows after 6912.  Sampled rows on both sides of
    the cut and at the ends, sampled columns, against the oracle."""
    g = np.random.default_rng(4343)
    K, N, M = 7168, 256, 600000
    Mp = -(-M // T) * T
    nb = Mp // T
    print(f"generating {K * Mp / 1e9:.2f} GB of codes", flush=True)
    qxT, qdyT = big_codes(g, K, Mp), big_codes(g, N, Mp)
    qxT[:, M:] = 0
    qdyT[:, M:] = 0
    assert (K - 1) * Mp + T > (1 << 32)
    sxT, sdyT = rand_scales(g, (nb, K)), rand_scales(g, (nb, N))
    dw = fgb.gemm_wgrad(u8_dev(qxT), f32_dev(sxT), u8_dev(qdyT), f32_dev(sdyT), M)
    torch.cuda.synchronize()
    cut = 6912
    rows = np.unique(np.concatenate([[0, 1, cut - 2, cut - 1, cut, cut + 1, K - 2, K - 1], g.choice(K, 8, replace=False)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], g.choice(N, 11, replace=False)]))
    r, aabs = orc.gemm_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols)
    ri, ci = torch.as_tensor(rows, device=dw.device), torch.as_tensor(cols, device=dw.device)
    got = host(dw[ri][:, ci].contiguous()).astype(np.float64)
    check_gemm(got, r, aabs, False, "wgrad beyond 4 GiB", hw_bound_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols), nb,
               model=model_wgrad(qxT, sxT, qdyT, sdyT, M, rows, cols))


def test_dgrad_operand_beyond_4gib(orc):
    """Dgrad with W [540672, 8192] (4.43 GB): dX's columns are cut after 523264,
    and each piece takes its own rows of W's 128x128 scale grid.  Sampled columns
    on both sides of the cut, every row, against the oracle."""
    g = np.random.default_rng(4444)
    M, K, N = 256, 540672, 8192
    print(f"generating {K * N / 1e9:.2f} GB of codes", flush=True)
    qdy, qw = big_codes(g, M, N), big_codes(g, K, N)
    assert (K - 1) * N + T > (1 << 32)
    sdy, sw = rand_scales(g, (N // T, M)), rand_scales(g, (K // T, N // T))
    dx = fgb.gemm_dgrad(u8_dev(qdy), f32_dev(sdy), u8_dev(qw), f32_dev(sw))
    torch.cuda.synchronize()
    cut = 523264
    cols = np.unique(np.concatenate([[0, 1, cut - 2, cut - 1, cut, cut + 1, K - 2, K - 1], g.choice(K, 56, replace=False)]))
    rows = np.arange(M, dtype=np.int64)[::8]
    r, aabs = orc.gemm_dgrad(qdy, sdy, qw, sw, rows, cols)
    ri, ci = torch.as_tensor(rows, device=dx.device), torch.as_tensor(cols, device=dx.device)
    got = bf16_host_f64(dx[ri][:, ci].contiguous())
    check_gemm(got, r, aabs, True, "dgrad beyond 4 GiB", hw_bound_dgrad(qdy, sdy, qw, sw, rows, cols), N // T,
               model=model_dgrad(qdy, sdy, qw, sw, rows, cols))
