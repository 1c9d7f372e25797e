"""Grouped (MoE expert) GEMMs against the CPU oracle: per-expert segments of a
128-aligned, zero-padded row layout, including empty experts; one expert
equals the dense GEMM bit for bit."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import workloads as wl

from parity import (assert_codes_equal, assert_scales_equal, bf16_dev, bf16_host_f64, check_gemm, f32_dev,
                    host, hw_bound_dgrad, hw_bound_fprop, hw_bound_wgrad, model_dgrad, model_fprop,
                    model_grouped_rows, model_grouped_wgrad, sample_idx, u8_dev)

pytestmark = pytest.mark.gpu
T = 128


def grouped_inputs(loads, K, N, seed):
    g = np.random.default_rng(seed)
    offsets = wl.moe_layout(loads)
    R = int(offsets[-1])
    x = np.zeros((R, K), np.float32)
    dy = np.zeros((R, N), np.float32)
    for e, n in enumerate(loads):
        a = offsets[e]
        x[a:a + n] = g.standard_normal((n, K))
        dy[a:a + n] = g.standard_normal((n, N)) * 1e-3
    ws = np.stack([wl.bf16_bits(g.standard_normal((K, N)).astype(np.float32) * 0.02) for _ in loads])
    return offsets, wl.bf16_bits(x), wl.bf16_bits(dy), ws


def offsets_dev(offsets):
    return torch.from_numpy(np.asarray(offsets, np.int32)).cuda()


def wgrad_hw_grouped(offsets, qxT, sxT, qdyT, sdyT, rows, cols):
    E = len(offsets) - 1
    out = np.zeros((E, rows.size, cols.size))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            out[e] = hw_bound_wgrad(qxT[:, a:b], sxT[a // T:b // T], qdyT[:, a:b], sdyT[a // T:b // T], b - a,
                                    rows, cols)
    return out


def quant_weights_gpu(ws):
    qs = [fgb.quantize_128x128(bf16_dev(w)) for w in ws]
    return (torch.stack([q[0] for q in qs]), torch.stack([q[1] for q in qs]), torch.stack([q[2] for q in qs]))


def quant_weights_orc(orc, ws):
    qs = [orc.quantize_128x128(w) for w in ws]
    return np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]), np.stack([q[2] for q in qs])


@pytest.mark.parametrize("loads", [[130, 0, 1, 256, 70], [0, 0, 300], [128]])
def test_grouped_small_full(orc, loads):
    K, N = 256, 384
    offsets, x, dy, ws = grouped_inputs(np.array(loads), K, N, sum(loads))
    od = offsets_dev(offsets)
    qx, sx = fgb.quantize_1x128(bf16_dev(x))
    qdy, sdy = fgb.quantize_1x128(bf16_dev(dy))
    qw, qwT, sw = quant_weights_gpu(ws)
    y = fgb.gemm_fprop_grouped(od, qx, sx, qwT, sw)
    dx = fgb.gemm_dgrad_grouped(od, qdy, sdy, qw, sw)
    qxT, sxT = fgb.requant_128x1(qx, sx)
    qdyT, sdyT = fgb.quantize_128x1(bf16_dev(dy))
    dw = fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT)

    oqx, osx = orc.quantize_1x128(x)
    oqdy, osdy = orc.quantize_1x128(dy)
    oqw, oqwT, osw = quant_weights_orc(orc, ws)
    assert_codes_equal(qwT.reshape(-1, K), oqwT.reshape(-1, K), "grouped qwT")
    oqxT, osxT = orc.requant_128x1(oqx, osx)
    oqdyT, osdyT = orc.quantize_128x1(dy)
    R = int(offsets[-1])
    hwf, hwd = np.zeros((R, N)), np.zeros((R, K))
    hww = np.zeros((len(loads), K, N))
    for e in range(len(loads)):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            hwf[a:b] = hw_bound_fprop(oqx[a:b], osx[:, a:b], oqwT[e], osw[e])
            hwd[a:b] = hw_bound_dgrad(oqdy[a:b], osdy[:, a:b], oqw[e], osw[e])
            hww[e] = hw_bound_wgrad(oqxT[:, a:b], osxT[a // T:b // T], oqdyT[:, a:b], osdyT[a // T:b // T], b - a)
    nbw = max(1, max(int(offsets[e + 1] - offsets[e]) // T for e in range(len(loads))))
    r, aabs = orc.gemm_fprop_grouped(offsets, oqx, osx, oqwT, osw)
    check_gemm(bf16_host_f64(y), r, aabs, True, f"fprop grouped {loads}", hwf, K // T,
               model=model_grouped_rows(offsets, model_fprop, oqx, osx, oqwT, osw))
    r, aabs = orc.gemm_dgrad_grouped(offsets, oqdy, osdy, oqw, osw)
    check_gemm(bf16_host_f64(dx), r, aabs, True, f"dgrad grouped {loads}", hwd, N // T,
               model=model_grouped_rows(offsets, model_dgrad, oqdy, osdy, oqw, osw))
    r, aabs = orc.gemm_wgrad_grouped(offsets, oqxT, osxT, oqdyT, osdyT)
    check_gemm(host(dw).reshape(r.shape), r, aabs, False, f"wgrad grouped {loads}", hww, nbw,
               model=model_grouped_wgrad(offsets, oqxT, osxT, oqdyT, osdyT))
    for e, n in enumerate(loads):
        if n == 0:
            assert torch.all(dw[e] == 0)
    # accumulate leaves empty experts unchanged and adds the old value to every
    # other output in one fp32 addition
    prev = torch.full_like(dw, 3.0)
    fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT, dw=prev, accumulate=True)
    for e, n in enumerate(loads):
        if n == 0:
            assert torch.all(prev[e] == 3.0)
    assert torch.equal((dw + 3.0).view(torch.int32), prev.view(torch.int32))
    check_gemm(host(prev).reshape(r.shape), r + 3.0, aabs + 3.0, False, f"wgrad grouped accumulate {loads}", hww,
               nbw + 1, stated=False)


def test_single_expert_equals_dense_bitwise():
    g = np.random.default_rng(4)
    R, K, N = 384, 512, 256
    qx = u8_dev(g.integers(0, 0x7E, (R, K)).astype(np.uint8))
    sx = f32_dev(np.exp(g.uniform(-5, 2, (K // T, R))).astype(np.float32))
    qwT = u8_dev(g.integers(0, 0x7E, (N, K)).astype(np.uint8))
    sw = f32_dev(np.exp(g.uniform(-5, 2, (K // T, N // T))).astype(np.float32))
    y1 = fgb.gemm_fprop(qx, sx, qwT, sw)
    y2 = fgb.gemm_fprop_grouped(offsets_dev([0, R]), qx, sx, qwT[None].contiguous(), sw[None].contiguous())
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.fixture(scope="module")
def moe():
    """Workload 4: 32 experts, 8192 tokens routed top-8 (Zipf 1.1, 3 empty)."""
    return wl.moe_grouped()


def test_moe_gate_up_sampled(orc, moe):
    d = moe
    offsets, E = d["offsets"], d["E"]
    od = offsets_dev(offsets)
    K, N = d["d_model"], d["d_ff2"]
    qx, sx = fgb.quantize_1x128(bf16_dev(d["x"]))
    qws = [fgb.quantize_128x128(bf16_dev(d["w_up"][e])) for e in range(E)]
    qw = torch.stack([q[0] for q in qws]); qwT = torch.stack([q[1] for q in qws]); sw = torch.stack([q[2] for q in qws])
    del qws
    y = fgb.gemm_fprop_grouped(od, qx, sx, qwT, sw)
    qdy, sdy = fgb.quantize_1x128(bf16_dev(d["dy_up"]))
    dx = fgb.gemm_dgrad_grouped(od, qdy, sdy, qw, sw)
    qxT, sxT = fgb.requant_128x1(qx, sx)
    qdyT, sdyT = fgb.quantize_128x1(bf16_dev(d["dy_up"]))
    dw = fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT)
    torch.cuda.synchronize()

    oqx, osx = orc.quantize_1x128(d["x"])
    assert_codes_equal(qx, oqx, "moe qx")
    assert_scales_equal(sx, osx, "moe sx")
    oqdy, osdy = orc.quantize_1x128(d["dy_up"])
    oqxT, osxT = orc.requant_128x1(oqx, osx)
    oqdyT, osdyT = orc.quantize_128x1(d["dy_up"])
    assert_codes_equal(qxT, oqxT, "moe qxT")
    assert_codes_equal(qdyT, oqdyT, "moe qdyT")
    # weights of a few experts (bit-exact), GEMM outputs sampled in every expert
    experts = [e for e in range(E) if d["loads"][e] > 0]
    check_e = sorted(set([experts[0], experts[-1], int(np.argmax(d["loads"]))]))
    yh, dxh = bf16_host_f64(y), bf16_host_f64(dx)
    for e in check_e:
        oq, oqT, os_ = orc.quantize_128x128(d["w_up"][e])
        assert_codes_equal(qwT[e], oqT, f"moe qwT[{e}]")
        assert_scales_equal(sw[e], os_, f"moe sw[{e}]")
        a, b = int(offsets[e]), int(offsets[e + 1])
        rows = a + sample_idx(b - a, 32, e)
        cols = sample_idx(N, 48, e + 100)
        r, aabs = orc.gemm_fprop(oqx[a:b], osx[:, a:b], oqT, os_, rows - a, cols)
        hw = hw_bound_fprop(oqx[a:b], osx[:, a:b], oqT, os_, rows - a, cols)
        check_gemm(yh[np.ix_(rows, cols)], r, aabs, True, f"moe fprop e{e}", hw, K // T,
                   model=model_fprop(oqx[a:b], osx[:, a:b], oqT, os_, rows - a, cols))
        colsK = sample_idx(K, 48, e + 200)
        r, aabs = orc.gemm_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK)
        hw = hw_bound_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK)
        check_gemm(dxh[np.ix_(rows, colsK)], r, aabs, True, f"moe dgrad e{e}", hw, N // T,
                   model=model_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK))
    wrows = sample_idx(K, 32, 7)
    wcols = sample_idx(N, 32, 8)
    r, aabs = orc.gemm_wgrad_grouped(offsets, oqxT, osxT, oqdyT, osdyT, experts=list(range(E)),
                                     rows=wrows, cols=wcols)
    hw = wgrad_hw_grouped(offsets, oqxT, osxT, oqdyT, osdyT, wrows, wcols)
    dwh = np.stack([host(dw[e])[np.ix_(wrows, wcols)] for e in range(E)])
    check_gemm(dwh, r, aabs, False, "moe wgrad (all experts)", hw, int(np.diff(offsets).max()) // T,
               model=model_grouped_wgrad(offsets, oqxT, osxT, oqdyT, osdyT, wrows, wcols))
    for e in range(E):
        if d["loads"][e] == 0:
            assert torch.all(dw[e] == 0)


def test_moe_down_sampled(orc, moe):
    d = moe
    offsets, E = d["offsets"], d["E"]
    od = offsets_dev(offsets)
    K, N = d["d_ff"], d["d_model"]
    qh, sh = fgb.quantize_1x128(bf16_dev(d["h"]))
    qws = [fgb.quantize_128x128(bf16_dev(d["w_down"][e])) for e in range(E)]
    qw = torch.stack([q[0] for q in qws]); qwT = torch.stack([q[1] for q in qws]); sw = torch.stack([q[2] for q in qws])
    del qws
    y = fgb.gemm_fprop_grouped(od, qh, sh, qwT, sw)
    qdy, sdy = fgb.quantize_1x128(bf16_dev(d["dy_down"]))
    dx = fgb.gemm_dgrad_grouped(od, qdy, sdy, qw, sw)
    qhT, shT = fgb.requant_128x1(qh, sh)
    qdyT, sdyT = fgb.quantize_128x1(bf16_dev(d["dy_down"]))
    dw = fgb.gemm_wgrad_grouped(od, qhT, shT, qdyT, sdyT)
    torch.cuda.synchronize()
    oqh, osh = orc.quantize_1x128(d["h"])
    oqdy, osdy = orc.quantize_1x128(d["dy_down"])
    oqhT, oshT = orc.requant_128x1(oqh, osh)
    oqdyT, osdyT = orc.quantize_128x1(d["dy_down"])
    assert_codes_equal(qh, oqh, "moe qh")
    assert_codes_equal(qdyT, oqdyT, "moe down qdyT")
    yh, dxh = bf16_host_f64(y), bf16_host_f64(dx)
    for e in [e for e in range(E) if d["loads"][e] > 0][::7]:
        oq, oqT, os_ = orc.quantize_128x128(d["w_down"][e])
        a, b = int(offsets[e]), int(offsets[e + 1])
        rows = a + sample_idx(b - a, 24, e)
        cols = sample_idx(N, 32, e + 1)
        r, aabs = orc.gemm_fprop(oqh[a:b], osh[:, a:b], oqT, os_, rows - a, cols)
        hw = hw_bound_fprop(oqh[a:b], osh[:, a:b], oqT, os_, rows - a, cols)
        check_gemm(yh[np.ix_(rows, cols)], r, aabs, True, f"moe down fprop e{e}", hw, K // T,
                   model=model_fprop(oqh[a:b], osh[:, a:b], oqT, os_, rows - a, cols))
        colsK = sample_idx(K, 32, e + 2)
        r, aabs = orc.gemm_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK)
        hw = hw_bound_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK)
        check_gemm(dxh[np.ix_(rows, colsK)], r, aabs, True, f"moe down dgrad e{e}", hw, N // T,
                   model=model_dgrad(oqdy[a:b], osdy[:, a:b], oq, os_, rows - a, colsK))
    wrows = sample_idx(K, 24, 9)
    wcols = sample_idx(N, 24, 10)
    r, aabs = orc.gemm_wgrad_grouped(offsets, oqhT, oshT, oqdyT, osdyT, rows=wrows, cols=wcols)
    hw = wgrad_hw_grouped(offsets, oqhT, oshT, oqdyT, osdyT, wrows, wcols)
    dwh = np.stack([host(dw[e])[np.ix_(wrows, wcols)] for e in range(E)])
    check_gemm(dwh, r, aabs, False, "moe down wgrad (all experts)", hw, int(np.diff(offsets).max()) // T,
               model=model_grouped_wgrad(offsets, oqhT, oshT, oqdyT, osdyT, wrows, wcols))


@pytest.mark.parametrize("E,N", [(100, 256), (70, 896)])
def test_grouped_many_experts_tail_rows_untouched(orc, E, N):
    """More experts than one wave has lanes (the tile search walks them in
    chunks of 64), half-height row tiles, a 224-wide tile (N = 896), and rows
    past offsets[E] that no expert owns: those output rows keep what they held."""
    K = 256
    g = np.random.default_rng(E)
    loads = g.integers(1, 300, E)
    loads[g.random(E) < 0.3] = 0
    offsets, x, dy, ws = grouped_inputs(loads, K, N, E + 1)
    R_used = int(offsets[-1])
    R_pad = R_used + 384
    x = np.concatenate([x, np.zeros((R_pad - R_used, K), np.uint16)])
    dy = np.concatenate([dy, np.zeros((R_pad - R_used, N), np.uint16)])
    od = offsets_dev(offsets)
    qx, sx = fgb.quantize_1x128(bf16_dev(x))
    qdy, sdy = fgb.quantize_1x128(bf16_dev(dy))
    qw, qwT, sw = quant_weights_gpu(ws)
    sentinel = torch.full((R_pad, max(N, K)), 7.0, dtype=torch.bfloat16, device="cuda")
    y = sentinel[:, :N].clone()
    dx = sentinel[:, :K].clone()
    fgb.gemm_fprop_grouped(od, qx, sx, qwT, sw, y=y)
    fgb.gemm_dgrad_grouped(od, qdy, sdy, qw, sw, dx=dx)
    qxT, sxT = fgb.requant_128x1(qx, sx)
    qdyT, sdyT = fgb.quantize_128x1(bf16_dev(dy))
    dw = fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT)
    torch.cuda.synchronize()
    assert torch.all(y[R_used:] == 7.0) and torch.all(dx[R_used:] == 7.0)

    oqx, osx = orc.quantize_1x128(x)
    oqdy, osdy = orc.quantize_1x128(dy)
    oqw, oqwT, osw = quant_weights_orc(orc, ws)
    oqxT, osxT = orc.requant_128x1(oqx, osx)
    oqdyT, osdyT = orc.quantize_128x1(dy)
    # every expert, a few rows each (its first and last rows, the 128/256 boundaries)
    rows = np.concatenate([int(offsets[e]) + sample_idx(int(offsets[e + 1] - offsets[e]), 6, e)
                           for e in range(E) if offsets[e + 1] > offsets[e]])
    cols, colsK = sample_idx(N, 40, 1), sample_idx(K, 40, 2)
    hwf, hwd = np.zeros((rows.size, cols.size)), np.zeros((rows.size, colsK.size))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        pick = np.nonzero((rows >= a) & (rows < b))[0]
        if pick.size:
            hwf[pick] = hw_bound_fprop(oqx[a:b], osx[:, a:b], oqwT[e], osw[e], rows[pick] - a, cols)
            hwd[pick] = hw_bound_dgrad(oqdy[a:b], osdy[:, a:b], oqw[e], osw[e], rows[pick] - a, colsK)
    r, aabs = orc.gemm_fprop_grouped(offsets, oqx, osx, oqwT, osw, rows=rows, cols=cols)
    check_gemm(bf16_host_f64(y)[np.ix_(rows, cols)], r, aabs, True, f"fprop grouped E={E}", hwf, K // T,
               model=model_grouped_rows(offsets, model_fprop, oqx, osx, oqwT, osw, rows, cols))
    r, aabs = orc.gemm_dgrad_grouped(offsets, oqdy, osdy, oqw, osw, rows=rows, cols=colsK)
    check_gemm(bf16_host_f64(dx)[np.ix_(rows, colsK)], r, aabs, True, f"dgrad grouped E={E}", hwd, N // T,
               model=model_grouped_rows(offsets, model_dgrad, oqdy, osdy, oqw, osw, rows, colsK))
    wr, wc = sample_idx(K, 24, 3), sample_idx(N, 24, 4)
    r, aabs = orc.gemm_wgrad_grouped(offsets, oqxT, osxT, oqdyT, osdyT, rows=wr, cols=wc)
    hw = wgrad_hw_grouped(offsets, oqxT, osxT, oqdyT, osdyT, wr, wc)
    nbw = max(1, int(np.diff(offsets).max()) // T)
    check_gemm(host(dw)[:, wr][:, :, wc], r, aabs, False, f"wgrad grouped E={E}", hw, nbw,
               model=model_grouped_wgrad(offsets, oqxT, osxT, oqdyT, osdyT, wr, wc))


def test_grouped_all_experts_empty():
    """offsets all zero: no row tile exists; outputs keep their contents and
    every expert's dW is zero."""
    E, R_pad, K, N = 5, 256, 256, 256
    od = offsets_dev([0] * (E + 1))
    qx = torch.zeros((R_pad, K), dtype=torch.uint8, device="cuda")
    sx = torch.ones((K // T, R_pad), dtype=torch.float32, device="cuda")
    qwT = torch.ones((E, N, K), dtype=torch.uint8, device="cuda")
    sw = torch.ones((E, K // T, N // T), dtype=torch.float32, device="cuda")
    y = torch.full((R_pad, N), 5.0, dtype=torch.bfloat16, device="cuda")
    fgb.gemm_fprop_grouped(od, qx, sx, qwT, sw, y=y)
    qxT = torch.ones((K, R_pad), dtype=torch.uint8, device="cuda")
    sxT = torch.ones((R_pad // T, K), dtype=torch.float32, device="cuda")
    qdyT = torch.ones((N, R_pad), dtype=torch.uint8, device="cuda")
    sdyT = torch.ones((R_pad // T, N), dtype=torch.float32, device="cuda")
    dw = torch.full((E, K, N), 9.0, dtype=torch.float32, device="cuda")
    fgb.gemm_wgrad_grouped(od, qxT, sxT, qdyT, sdyT, dw=dw)
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
    assert torch.all(dw == 0.0)
