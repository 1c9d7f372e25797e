"""The C-ABI library on a host without a GPU: it loads, exports every entry point
declared in include/fgb.h, and rejects invalid arguments with the documented
status before any HIP call (only argument errors and empty no-ops are called
here, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import fine_grained_block_amd as fgb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_ALIGN, E_LD, E_UNSUP, E_HIP, E_ARG = 0, -1, -2, -3, -4, -5, -6, -7
P = ctypes.c_void_p
A = P(0x10000)         # 16-byte aligned placeholder addresses (never dereferenced)
B = P(0x20000)
C_ = P(0x30000)
D = P(0x40000)
MIS = P(0x10004)       # misaligned


def header_functions():
    text = open(os.path.join(ROOT, "include", "fgb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgb_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fgb.lib()
    names = header_functions()
    assert len(names) == 33
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(fgb.SIGNATURES)


def test_version_and_status_strings():
    L = fgb.lib()
    assert L.fgb_version() == 0x000100
    for st in (OK, E_NULL, E_SHAPE, E_ALIGN, E_LD, E_UNSUP, E_HIP, E_ARG):
        assert L.fgb_status_string(st)
    assert L.fgb_status_string(12345) == b"unknown status"


def q1(x=A, R=4, C=128, ldx=128, fl=0.0, q=B, ldq=128, s=C_, lds=4):
    return fgb.lib().fgb_quantize_1x128(x, R, C, ldx, fl, q, ldq, s, lds, None)


def test_quantize_1x128_validation():
    assert q1(C=12) == E_SHAPE
    assert q1(R=-1) == E_SHAPE
    assert q1(x=P(0)) == E_NULL
    assert q1(q=P(0)) == E_NULL
    assert q1(s=P(0)) == E_NULL
    assert q1(ldx=64) == E_LD
    assert q1(ldq=64) == E_LD
    assert q1(lds=3) == E_LD
    assert q1(x=MIS) == E_ALIGN
    assert q1(ldx=132) == E_ALIGN
    assert q1(fl=-1.0) == E_ARG
    assert q1(fl=float("nan")) == E_ARG
    assert q1(fl=float("inf")) == E_ARG
    assert q1(R=0, x=P(0), q=P(0), s=P(0)) == OK      # empty: no launch
    assert q1(C=0, x=P(0), q=P(0), s=P(0)) == OK


def test_quantize_128x1_validation():
    L = fgb.lib()
    f = lambda **k: L.fgb_quantize_128x1(k.get("x", A), k.get("R", 200), k.get("C", 128), k.get("ldx", 128),
                                         k.get("fl", 0.0), k.get("q", B), k.get("ldq", 256), k.get("s", C_),
                                         k.get("lds", 128), None)
    assert f(ldq=200) == E_LD          # must cover roundup(200, 128) = 256
    assert f(ldq=264, q=P(0x20008)) == E_ALIGN
    assert f(C=100) == E_SHAPE
    assert f(lds=127) == E_LD
    assert f(R=0) == OK


def test_quantize_dual_validation():
    L = fgb.lib()
    E = P(0x50000)
    f = lambda **k: L.fgb_quantize_dual(k.get("x", A), k.get("R", 200), k.get("C", 128), k.get("ldx", 128),
                                        k.get("fl", 0.0), k.get("q", B), k.get("ldq", 128), k.get("s", C_),
                                        k.get("lds", 200), k.get("qT", D), k.get("ldqT", 256), k.get("sT", E),
                                        k.get("ldsT", 128), None)
    assert f(C=100) == E_SHAPE
    assert f(fl=-1.0) == E_ARG
    assert f(x=None) == E_NULL
    assert f(q=None) == E_NULL
    assert f(sT=None) == E_NULL
    assert f(ldq=120) == E_LD
    assert f(lds=199) == E_LD
    assert f(ldqT=200) == E_LD         # must cover roundup(200, 128) = 256
    assert f(ldsT=127) == E_LD
    assert f(qT=P(0x40008), ldqT=264) == E_ALIGN
    assert f(R=0) == OK and f(C=0) == OK


def test_quantize_128x128_validation():
    L = fgb.lib()
    f = lambda **k: L.fgb_quantize_128x128(k.get("w", A), k.get("K", 256), k.get("N", 128), k.get("ldw", 128),
                                           0.0, k.get("q", B), k.get("ldq", 128), k.get("qT", C_),
                                           k.get("ldqT", 256), k.get("s", D), None)
    assert f(K=200) == E_SHAPE
    assert f(N=100) == E_SHAPE
    assert f(q=P(0), qT=P(0)) == E_NULL
    assert f(ldqT=128) == E_LD
    assert f(s=P(0)) == E_NULL
    assert f(K=0) == OK


def test_requant_validation():
    L = fgb.lib()
    f = lambda **k: L.fgb_requant_128x1(k.get("q", A), k.get("R", 128), k.get("C", 256), k.get("ldq", 256),
                                        k.get("s", B), k.get("lds", 128), k.get("qT", C_), k.get("ldqT", 128),
                                        k.get("sT", D), k.get("ldsT", 256), None)
    assert f(s=P(0)) == E_NULL
    assert f(lds=100) == E_LD
    assert f(ldsT=255) == E_LD
    assert f(C=20) == E_SHAPE
    assert f(R=0) == OK


def test_gemm_validation():
    L = fgb.lib()
    fp = lambda **k: L.fgb_gemm_fprop(k.get("M", 64), k.get("N", 128), k.get("K", 256), k.get("qx", A),
                                      k.get("ldqx", 256), k.get("sx", B), k.get("ldsx", 64), k.get("qw", C_),
                                      k.get("ldqw", 256), k.get("sw", D), k.get("y", P(0x50000)),
                                      k.get("ldy", 128), None)
    assert fp(K=200) == E_SHAPE
    assert fp(N=64) == E_SHAPE
    assert fp(qx=P(0)) == E_NULL
    assert fp(y=P(0)) == E_NULL
    assert fp(ldqx=128) == E_LD
    assert fp(ldsx=63) == E_LD
    assert fp(ldqx=264) == E_ALIGN
    assert fp(qw=P(0x30008)) == E_ALIGN
    assert fp(M=0) == OK
    dg = lambda **k: L.fgb_gemm_dgrad(k.get("M", 64), k.get("K", 128), k.get("N", 256), A, 256, B,
                                      k.get("ldsdy", 64), C_, 256, D, P(0x50000), k.get("lddx", 128), None)
    assert dg(N=130) == E_SHAPE
    assert dg(lddx=100) == E_LD
    assert dg(M=0) == OK
    wg = lambda **k: L.fgb_gemm_wgrad(k.get("K", 128), k.get("N", 128), k.get("M", 200), A, k.get("ldqx", 256),
                                      B, 128, C_, 256, D, 128, P(0x50000), k.get("lddw", 128), 0, None)
    assert wg(ldqx=200) == E_LD        # must cover roundup(200, 128)
    assert wg(lddw=64) == E_LD
    assert wg(K=100) == E_SHAPE
    assert wg(M=-1) == E_SHAPE
    assert wg(K=0) == OK


def test_grouped_validation():
    L = fgb.lib()
    g = lambda **k: L.fgb_gemm_fprop_grouped(k.get("E", 4), k.get("off", P(0x60000)), k.get("R", 512),
                                             k.get("N", 128), k.get("K", 256), A, B, C_, D,
                                             k.get("y", P(0x50000)), None)
    assert g(R=500) == E_SHAPE
    assert g(off=P(0)) == E_NULL
    assert g(off=P(0x60002)) == E_ALIGN
    assert g(E=0) == OK
    assert g(E=-1) == E_SHAPE
    # operands whose byte offsets do not fit 32 bits; more than 65535 experts
    assert g(R=1 << 20, K=8192) == E_UNSUP
    # every offset fits, but the grid (one block per tile) would not fit an int
    assert g(E=65535, R=1 << 25, N=1 << 25, K=128) == E_UNSUP
    assert g(E=1 << 16) == E_SHAPE
    w = lambda **k: L.fgb_gemm_wgrad_grouped(k.get("E", 4), P(0x60000), k.get("R", 512), 128, 128, A, B, C_, D,
                                             k.get("dw", P(0x50000)), 0, None)
    assert w(dw=P(0)) == E_NULL
    assert w(R=130) == E_SHAPE
    assert w(E=0) == OK
    assert w(R=1 << 26) == E_UNSUP


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(fgb.FgbError):
        fgb.quantize_1x128(x)


def test_stochastic_rounding_validation():
    """The _sr twins validate exactly like their round-to-nearest twins (no launch
    on any error, empty inputs are no-ops)."""
    L = fgb.lib()
    U64, U32 = ctypes.c_uint64, ctypes.c_uint32
    seed, salt = U64(123), U32(4)

    def q1(R=256, C=256, x=A, ldx=256, fl=0.0, q=B, ldq=256, s=C_, lds=256):
        return L.fgb_quantize_1x128_sr(x, R, C, ldx, fl, q, ldq, s, lds, seed, salt, None)

    assert q1(C=12) == E_SHAPE
    assert q1(x=P(0)) == E_NULL
    assert q1(ldq=64) == E_LD
    assert q1(x=MIS) == E_ALIGN
    assert q1(fl=-1.0) == E_ARG
    assert q1(R=0, x=P(0), q=P(0), s=P(0)) == OK
    assert L.fgb_quantize_128x1_sr(A, 200, 256, 256, 0.0, B, 128, C_, 256, seed, salt, None) == E_LD
    assert L.fgb_quantize_128x1_sr(A, 200, 12, 256, 0.0, B, 256, C_, 256, seed, salt, None) == E_SHAPE
    assert L.fgb_quantize_dual_sr(A, 256, 256, 256, 0.0, B, 256, C_, 256, P(0), 256, D, 256,
                                  seed, salt, None) == E_NULL
    assert L.fgb_quantize_128x128_sr(A, 200, 256, 256, 0.0, B, 256, C_, 256, D, seed, salt, None) == E_SHAPE
    assert L.fgb_quantize_128x128_sr(A, 256, 256, 256, 0.0, P(0), 256, P(0), 256, D, seed, salt, None) == E_NULL
    with pytest.raises(fgb.FgbError):
        fgb._quant_call("fgb_quantize_1x128", True, (1, 2), (A, 1, 8, 8, 0.0, B, 8, C_, 1, None))


def test_swiglu_validation():
    L = fgb.lib()

    def fwd(R=256, F=256, gu=A, ldgu=512, fl=0.0, qg=B, ldqg=512, sg=C_, ldsg=256, qh=D, ldqh=256, sh=C_, ldsh=256,
            h=P(0), ldh=0):
        return L.fgb_swiglu_fwd_quant(gu, R, F, ldgu, fl, qg, ldqg, sg, ldsg, qh, ldqh, sh, ldsh, h, ldh, None)

    assert fwd(F=200) == E_SHAPE
    assert fwd(R=-1) == E_SHAPE
    assert fwd(ldgu=256) == E_LD
    assert fwd(gu=MIS) == E_ALIGN
    assert fwd(qg=P(0)) == E_NULL                        # stash codes without scales
    assert fwd(qh=P(0)) == E_NULL
    assert fwd(ldqh=128) == E_LD
    assert fwd(h=MIS, ldh=256) == E_ALIGN
    assert fwd(fl=-1.0) == E_ARG
    assert fwd(R=0, gu=P(0), qh=P(0), sh=P(0)) == OK

    def bwd(R=256, F=256, qg=A, ldqg=512, sg=B, ldsg=256, dh=C_, lddh=256, fl=0.0, q=D, ldq=512, s=B, lds=256,
            qT=A, ldqT=256, sT=B, ldsT=512, dgu=P(0), lddgu=0):
        return L.fgb_swiglu_bwd_quant(qg, R, F, ldqg, sg, ldsg, dh, lddh, fl, q, ldq, s, lds, qT, ldqT, sT, ldsT,
                                      dgu, lddgu, None)

    assert bwd(F=100) == E_SHAPE
    assert bwd(qg=P(0)) == E_NULL
    assert bwd(lddh=128) == E_LD
    assert bwd(ldqT=200) == E_LD
    assert bwd(ldsT=256) == E_LD
    assert bwd(qT=P(0x10008)) == E_ALIGN
    assert bwd(dgu=MIS, lddgu=512) == E_ALIGN
    assert bwd(F=0, qg=P(0)) == OK


def rq2(q=A, K=128, N=256, ldq=256, s=C_, fl=0.0, q2=B, ldq2=256, q2T=D, ldq2T=128, s2=C_):
    return fgb.lib().fgb_requant_128x128_ue8m0(q, K, N, ldq, s, fl, q2, ldq2, q2T, ldq2T, s2, None)


def test_requant_128x128_ue8m0_validation():
    assert rq2(K=100) == E_SHAPE
    assert rq2(N=200) == E_SHAPE
    assert rq2(K=-128) == E_SHAPE
    assert rq2(fl=-1.0) == E_ARG
    assert rq2(fl=float("nan")) == E_ARG
    assert rq2(q=P(0)) == E_NULL
    assert rq2(s=P(0)) == E_NULL
    assert rq2(s2=P(0)) == E_NULL
    assert rq2(q2=P(0), q2T=P(0)) == E_NULL
    assert rq2(ldq=128) == E_LD
    assert rq2(ldq2=128) == E_LD
    assert rq2(ldq2T=64) == E_LD
    assert rq2(q=MIS) == E_ALIGN
    assert rq2(K=0) == OK and rq2(N=0) == OK          # empty: nothing to do


def qb(E=2, w=A, K=128, N=256, fl=0.0, q=B, qT=D, s=C_):
    return fgb.lib().fgb_quantize_128x128_batched(E, w, K, N, fl, q, qT, s, None)


def test_quantize_128x128_batched_validation():
    assert qb(K=100) == E_SHAPE
    assert qb(N=200) == E_SHAPE
    assert qb(E=-1) == E_SHAPE
    assert qb(E=65536) == E_SHAPE
    assert qb(fl=-2.0) == E_ARG
    assert qb(w=P(0)) == E_NULL
    assert qb(q=P(0), qT=P(0)) == E_NULL
    assert qb(s=P(0)) == E_NULL
    assert qb(w=MIS) == E_ALIGN
    assert qb(E=0) == OK and qb(K=0) == OK


def test_probe_library_exports_and_argument_errors():
    """libfgb_probe.so (the benchmark's clock and staging probes, include/fgb_probe.h): every
    declared function is exported, and bad arguments return -1 before any HIP call."""
    path = os.path.join(ROOT, "fine_grained_block_amd", "libfgb_probe.so")
    if not os.path.exists(path):
        pytest.skip("libfgb_probe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fgb_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fgb_\w+)\s*\(", text)))
    assert names == ["fgb_probe_clock", "fgb_probe_clock_begin", "fgb_probe_clock_end", "fgb_probe_staging"]
    L = ctypes.CDLL(path)
    for n in names:
        assert hasattr(L, n), n
    L.fgb_probe_clock.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), P]
    L.fgb_probe_clock_begin.argtypes = [ctypes.c_int, ctypes.c_double, P]
    L.fgb_probe_clock_end.argtypes = [ctypes.POINTER(ctypes.c_double), P]
    L.fgb_probe_staging.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), P]
    mhz = ctypes.c_double(0.0)
    cyc = (ctypes.c_double * 3)()
    assert L.fgb_probe_staging(0, cyc, None) == -1
    assert L.fgb_probe_staging(10**7 + 1, cyc, None) == -1
    assert L.fgb_probe_staging(10, None, None) == -1
    assert L.fgb_probe_clock(0, ctypes.byref(mhz), None) == -1
    assert L.fgb_probe_clock(10, None, None) == -1
    assert L.fgb_probe_clock_begin(0, 100.0, None) == -1
    assert L.fgb_probe_clock_begin(4097, 100.0, None) == -1
    assert L.fgb_probe_clock_begin(8, 0.0, None) == -1
    assert L.fgb_probe_clock_begin(8, 2e6, None) == -1
    assert L.fgb_probe_clock_end(ctypes.byref(mhz), None) == -1      # no sample running
