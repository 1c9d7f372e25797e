"""The Python binding's argument checks, on the CPU: every tensor a wrapper
passes to the C ABI must have the exact dtype, device, shape and layout the
call needs, or the wrapper raises FgbError before any library call.  The C ABI
sees only pointers and sizes, so these checks are what keeps a short output or
a host-resident scale array from reaching a kernel.

Tensors here are CPU tensors that report is_cuda (a subclass), and the library
is replaced by a recorder: no HIP call is made."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb

U8, F32, BF16, I32 = torch.uint8, torch.float32, torch.bfloat16, torch.int32


class DevTensor(torch.Tensor):
    """A CPU tensor that passes the binding's device-tensor check."""
    @property
    def is_cuda(self):
        return True


def d(shape, dtype):
    return torch.Tensor._make_subclass(DevTensor, torch.zeros(shape, dtype=dtype))


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(fgb, "lib", lambda: r)
    monkeypatch.setattr(fgb, "_stream", lambda t: None)
    monkeypatch.setattr(fgb, "_new", lambda shape, dtype, dev: d(shape, dtype))   # outputs the wrapper makes
    return r


def expect_error(fn, *args, **kw):
    with pytest.raises(fgb.FgbError):
        fn(*args, **kw)


def test_quantizers_check_outputs(rec):
    R, C = 200, 256
    x = d((R, C), BF16)
    fgb.quantize_1x128(x)
    fgb.quantize_1x128(x, q=d((R, C), U8), s=d((2, R), F32))
    assert rec.calls == ["fgb_quantize_1x128", "fgb_quantize_1x128"]
    expect_error(fgb.quantize_1x128, x, q=d((R - 1, C), U8))              # short codes
    expect_error(fgb.quantize_1x128, x, s=d((1, R), F32))                 # short scales
    expect_error(fgb.quantize_1x128, x, s=d((2, R), torch.float64))       # wrong dtype
    expect_error(fgb.quantize_1x128, x, s=torch.zeros((2, R)))            # host scales
    expect_error(fgb.quantize_1x128, torch.zeros((R, C), dtype=BF16))     # host input
    expect_error(fgb.quantize_1x128, d((R, C), F32))                      # fp32 input
    expect_error(fgb.quantize_1x128, x, q=d((C, R), U8).t())              # column-major codes
    fgb.quantize_128x1(x)
    expect_error(fgb.quantize_128x1, x, qT=d((C, R), U8))                 # rows not padded to 256
    expect_error(fgb.quantize_128x1, x, sT=d((1, C), F32))
    fgb.quantize_dual(x)
    expect_error(fgb.quantize_dual, x, qT=d((C, 128), U8))
    expect_error(fgb.quantize_dual, x, s=d((2, R + 1), F32)[:, :R].t().t()[:1])
    w = d((256, 384), BF16)
    fgb.quantize_128x128(w)
    expect_error(fgb.quantize_128x128, w, s=d((2, 2), F32))
    expect_error(fgb.quantize_128x128, w, s=d((3, 2), F32).t())           # non-contiguous scales
    expect_error(fgb.quantize_128x128, w, qT=d((384, 255), U8))
    q = d((R, C), U8)
    fgb.requant_128x1(q, d((2, R), F32))
    expect_error(fgb.requant_128x1, q, d((2, R - 1), F32))                # short input scales
    expect_error(fgb.requant_128x1, q, d((2, R), F32), qT=d((C, 255), U8))
    wb = d((3, 256, 384), BF16)
    fgb.quantize_128x128_batched(wb)
    expect_error(fgb.quantize_128x128_batched, wb, s=d((2, 2, 3), F32))
    expect_error(fgb.quantize_128x128_batched, wb, qT=d((3, 256, 384), U8))
    fgb.requant_128x128_ue8m0(d((256, 384), U8), d((2, 3), F32))
    expect_error(fgb.requant_128x128_ue8m0, d((256, 384), U8), d((2, 2), F32))


def test_swiglu_checks(rec):
    R, F = 130, 256
    gu = d((R, 2 * F), BF16)
    fgb.swiglu_fwd_quant(gu, want_h=True)
    expect_error(fgb.swiglu_fwd_quant, gu, q_h=d((R, F - 1), U8))
    expect_error(fgb.swiglu_fwd_quant, gu, h=d((R - 1, F), BF16))
    expect_error(fgb.swiglu_fwd_quant, d((R, 2 * F + 1), BF16))
    qg, sg, dh = d((R, 2 * F), U8), d((4, R), F32), d((R, F), BF16)
    fgb.swiglu_bwd_quant(qg, sg, dh)
    expect_error(fgb.swiglu_bwd_quant, qg, sg, d((R, F - 8), BF16))
    expect_error(fgb.swiglu_bwd_quant, qg, d((3, R), F32), dh)
    expect_error(fgb.swiglu_bwd_quant, qg, sg, dh, qT=d((2 * F, R), U8))


def test_gemm_checks(rec):
    M, K, N = 200, 256, 384
    qx, sx, qwT, sw = d((M, K), U8), d((2, M), F32), d((N, K), U8), d((2, 3), F32)
    fgb.gemm_fprop(qx, sx, qwT, sw)
    expect_error(fgb.gemm_fprop, qx, sx, qwT, sw, y=d((M, N - 1), BF16))       # short output
    expect_error(fgb.gemm_fprop, qx, sx, qwT, sw, y=d((M, N), F32))            # wrong output dtype
    expect_error(fgb.gemm_fprop, qx, sx, qwT, torch.zeros((2, 3)))             # host weight scales
    expect_error(fgb.gemm_fprop, qx, sx, qwT, d((2, 2), F32))                  # short weight scales
    expect_error(fgb.gemm_fprop, qx, d((2, M - 1), F32), qwT, sw)              # short row scales
    expect_error(fgb.gemm_fprop, qx, sx, d((N, K + 128), U8), sw)              # contraction mismatch
    qdy, sdy, qw = d((M, N), U8), d((3, M), F32), d((K, N), U8)
    fgb.gemm_dgrad(qdy, sdy, qw, sw)
    expect_error(fgb.gemm_dgrad, qdy, sdy, qw, sw, dx=d((M - 1, K), BF16))
    expect_error(fgb.gemm_dgrad, qdy, sdy, d((K, N - 128), U8), sw)
    qxT, sxT, qdyT, sdyT = d((K, 256), U8), d((2, K), F32), d((N, 256), U8), d((2, N), F32)
    fgb.gemm_wgrad(qxT, sxT, qdyT, sdyT, M)
    expect_error(fgb.gemm_wgrad, qxT, sxT, qdyT, sdyT, M, dw=d((K, N - 4), F32))
    expect_error(fgb.gemm_wgrad, qxT, sxT, qdyT, sdyT, 257)                   # operands shorter than M
    expect_error(fgb.gemm_wgrad, qxT, d((1, K), F32), qdyT, sdyT, M)           # too few scale rows
    expect_error(fgb.gemm_wgrad, qxT, sxT, d((N, 128), U8), sdyT, M)           # padded widths differ
    expect_error(fgb.gemm_wgrad, qxT, sxT, qdyT, sdyT, M, dw=torch.zeros((K, N)))
    assert rec.calls == ["fgb_gemm_fprop", "fgb_gemm_dgrad", "fgb_gemm_wgrad"]


def test_grouped_gemm_checks(rec):
    E, R, K, N = 3, 512, 256, 384
    off = d((E + 1,), I32)
    qx, sx, qwT, sw = d((R, K), U8), d((2, R), F32), d((E, N, K), U8), d((E, 2, 3), F32)
    fgb.gemm_fprop_grouped(off, qx, sx, qwT, sw)
    expect_error(fgb.gemm_fprop_grouped, off, qx, sx, qwT, d((E, 2, 2), F32))   # short scales
    expect_error(fgb.gemm_fprop_grouped, off, qx, sx, d((E - 1, N, K), U8), sw)  # experts != E
    expect_error(fgb.gemm_fprop_grouped, off, qx, sx, qwT, sw, y=d((R, N - 128), BF16))
    expect_error(fgb.gemm_fprop_grouped, torch.zeros(E + 1, dtype=I32), qx, sx, qwT, sw)   # host offsets
    expect_error(fgb.gemm_fprop_grouped, d((E + 1,), torch.int64), qx, sx, qwT, sw)
    qdy, sdy, qw = d((R, N), U8), d((3, R), F32), d((E, K, N), U8)
    fgb.gemm_dgrad_grouped(off, qdy, sdy, qw, sw)
    expect_error(fgb.gemm_dgrad_grouped, off, qdy, sdy, d((E, K, N + 128), U8), sw)
    expect_error(fgb.gemm_dgrad_grouped, off, qdy, sdy, qw, sw, dx=d((R, K), F32))
    qxT, sxT, qdyT, sdyT = d((K, R), U8), d((4, K), F32), d((N, R), U8), d((4, N), F32)
    fgb.gemm_wgrad_grouped(off, qxT, sxT, qdyT, sdyT)
    expect_error(fgb.gemm_wgrad_grouped, off, qxT, sxT, qdyT, sdyT, dw=d((E, K, N - 1), F32))
    expect_error(fgb.gemm_wgrad_grouped, off, qxT, d((3, K), F32), qdyT, sdyT)
    expect_error(fgb.gemm_wgrad_grouped, off, qxT, sxT, d((N, R - 128), U8), sdyT)
    assert rec.calls == ["fgb_gemm_fprop_grouped", "fgb_gemm_dgrad_grouped", "fgb_gemm_wgrad_grouped"]
