"""fine_grained_block_amd -- fine-grained block-scaled FP8 linear layers on MI355X.

Thin Python binding over ``libfgb.so`` (C ABI in ``include/fgb.h``).  Every
function here only marshals torch tensors into pointers, leading dimensions
and the current HIP stream; all computation runs in the library's HIP kernels.
There is no fallback: if ``libfgb.so`` is missing or a call fails, an
exception is raised.

Layouts (all row-major, bf16 = ``torch.bfloat16``, E4M3 codes = ``torch.uint8``,
scales = ``torch.float32``):

* ``quantize_1x128(x[R, C])`` -> ``q[R, C]``, ``s[ceil(C/128), R]``
* ``quantize_128x1(x[R, C])`` -> ``qT[C, roundup(R,128)]``, ``sT[ceil(R/128), C]``
* ``quantize_128x128(w[K, N])`` -> ``q[K, N]``, ``qT[N, K]``, ``s[K/128, N/128]``
* ``requant_128x1(q[R, C], s)`` -> ``qT``, ``sT`` as ``quantize_128x1``
* ``gemm_fprop(qx, sx, qwT, sw)`` -> ``y[M, N]`` bf16 (Y = X W)
* ``gemm_dgrad(qdy, sdy, qw, sw)`` -> ``dx[M, K]`` bf16 (dX = dY W^T)
* ``gemm_wgrad(qxT, sxT, qdyT, sdyT, M)`` -> ``dw[K, N]`` fp32 (dW = X^T dY)
* ``gemm_*_grouped(offsets, ...)`` -- the same per expert segment.
* ``quantize_dual(x[R, C])`` -> both ``quantize_1x128`` and ``quantize_128x1`` outputs from one read.

Every quantizer and GEMM takes ``ue8m0=True`` for the power-of-two-scale twin
(``..._ue8m0`` entry points): scales are exact powers of two in fp32 and the
GEMMs let the matrix core apply them.

The 1x128, 128x1, dual and 128x128 quantizers take ``sr=(seed, salt)`` for the
stochastic-rounding twin (``..._sr`` entry points): same scales, the cast picks
the lower or upper E4M3 neighbour with one Philox4x32-10 word per element.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfgb.so")
TILE = 128

STATUS = {0: "FGB_OK", -1: "FGB_E_NULL", -2: "FGB_E_SHAPE", -3: "FGB_E_ALIGN", -4: "FGB_E_LD",
          -5: "FGB_E_UNSUPPORTED", -6: "FGB_E_HIP", -7: "FGB_E_ARG"}

# name -> ctypes argument types (P = pointer, I = int64, F = float, N = int)
_P, _I, _F, _N = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_U64, _U32 = ctypes.c_uint64, ctypes.c_uint32
SIGNATURES = {
    "fgb_quantize_1x128": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P],
    "fgb_quantize_128x1": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P],
    "fgb_quantize_dual": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_quantize_128x128": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _P],
    "fgb_requant_128x1": [_P, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_gemm_fprop": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P],
    "fgb_gemm_dgrad": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P],
    "fgb_gemm_wgrad": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _I, _P, _I, _N, _P],
    "fgb_gemm_fprop_grouped": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P],
    "fgb_gemm_dgrad_grouped": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P],
    "fgb_gemm_wgrad_grouped": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _N, _P],
    "fgb_quantize_1x128_ue8m0": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P],
    "fgb_quantize_128x1_ue8m0": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P],
    "fgb_quantize_dual_ue8m0": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_quantize_128x128_ue8m0": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _P],
    "fgb_requant_128x1_ue8m0": [_P, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_requant_128x128_ue8m0": [_P, _I, _I, _I, _P, _F, _P, _I, _P, _I, _P, _P],
    "fgb_quantize_128x128_batched": [_I, _P, _I, _I, _F, _P, _P, _P, _P],
    "fgb_quantize_128x128_batched_ue8m0": [_I, _P, _I, _I, _F, _P, _P, _P, _P],
    "fgb_gemm_fprop_ue8m0": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P],
    "fgb_gemm_dgrad_ue8m0": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P],
    "fgb_gemm_wgrad_ue8m0": [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _I, _P, _I, _N, _P],
    "fgb_gemm_fprop_grouped_ue8m0": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P],
    "fgb_gemm_dgrad_grouped_ue8m0": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P],
    "fgb_gemm_wgrad_grouped_ue8m0": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _N, _P],
    "fgb_quantize_1x128_sr": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _U64, _U32, _P],
    "fgb_quantize_128x1_sr": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _U64, _U32, _P],
    "fgb_quantize_dual_sr": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _I, _P, _I, _U64, _U32, _P],
    "fgb_quantize_128x128_sr": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _U64, _U32, _P],
    "fgb_swiglu_fwd_quant": [_P, _I, _I, _I, _F, _P, _I, _P, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_swiglu_bwd_quant": [_P, _I, _I, _I, _P, _I, _P, _I, _F, _P, _I, _P, _I, _P, _I, _P, _I, _P, _I, _P],
    "fgb_status_string": [_N],
    "fgb_version": [],
}


class FgbError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfgb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FgbError(f"{LIB_PATH} is missing: build it with "
                           "`python -m fine_grained_block_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.fgb_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, name: str):
    if status != 0:
        msg = lib().fgb_status_string(status).decode()
        raise FgbError(f"{name}: {STATUS.get(status, status)} ({msg})")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _rows(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise FgbError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise FgbError(f"{name}: expected a device tensor")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise FgbError(f"{name}: expected a 2-D row-major tensor")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _cdiv(a, b):
    return -(-a // b)


def _fn(name: str, ue8m0: bool):
    """The entry point `name`, or its power-of-two-scale twin `name`_ue8m0."""
    return getattr(lib(), name + "_ue8m0" if ue8m0 else name)


def _quant_call(name: str, ue8m0: bool, sr, args):
    """Call quantizer `name` (round to nearest), its _ue8m0 twin, or with sr = (seed,
    salt) its stochastic-rounding twin `name`_sr; the stream stays the last argument."""
    if sr is None:
        return _fn(name, ue8m0)(*args)
    if ue8m0:
        raise FgbError(f"{name}: stochastic rounding uses absmax/448 scales (no ue8m0 twin)")
    seed, salt = sr
    return getattr(lib(), name + "_sr")(*args[:-1], ctypes.c_uint64(seed), ctypes.c_uint32(salt), args[-1])


def version() -> int:
    return lib().fgb_version()


# ---------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------

def quantize_1x128(x: torch.Tensor, amax_floor: float = 0.0, q=None, s=None, ue8m0: bool = False, sr=None):
    R, C = x.shape
    ldx = _rows(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((_cdiv(C, TILE), R), dtype=torch.float32, device=x.device)
    _check(_quant_call("fgb_quantize_1x128", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor, _ptr(q),
                       _rows(q, torch.uint8, "q"), _ptr(s), _rows(s, torch.float32, "s"), _stream(x))),
           "quantize_1x128")
    return q, s


def quantize_128x1(x: torch.Tensor, amax_floor: float = 0.0, qT=None, sT=None, ue8m0: bool = False, sr=None):
    R, C = x.shape
    ldx = _rows(x, torch.bfloat16, "x")
    if qT is None:
        qT = torch.empty((C, _cdiv(R, TILE) * TILE), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty((_cdiv(R, TILE), C), dtype=torch.float32, device=x.device)
    _check(_quant_call("fgb_quantize_128x1", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor, _ptr(qT),
                       _rows(qT, torch.uint8, "qT"), _ptr(sT), _rows(sT, torch.float32, "sT"), _stream(x))),
           "quantize_128x1")
    return qT, sT


def quantize_dual(x: torch.Tensor, amax_floor: float = 0.0, q=None, s=None, qT=None, sT=None, ue8m0: bool = False,
                  sr=None):
    """Both orientations from one read: (q, s) as quantize_1x128, (qT, sT) as quantize_128x1."""
    R, C = x.shape
    ldx = _rows(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((_cdiv(C, TILE), R), dtype=torch.float32, device=x.device)
    if qT is None:
        qT = torch.empty((C, _cdiv(R, TILE) * TILE), dtype=torch.uint8, device=x.device)
    if sT is None:
        sT = torch.empty((_cdiv(R, TILE), C), dtype=torch.float32, device=x.device)
    _check(_quant_call("fgb_quantize_dual", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor,
                       _ptr(q), _rows(q, torch.uint8, "q"), _ptr(s), _rows(s, torch.float32, "s"),
                       _ptr(qT), _rows(qT, torch.uint8, "qT"), _ptr(sT), _rows(sT, torch.float32, "sT"),
                       _stream(x))), "quantize_dual")
    return q, s, qT, sT


def quantize_128x128(w: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True, want_qT: bool = True,
                     q=None, qT=None, s=None, ue8m0: bool = False, sr=None):
    K, N = w.shape
    ldw = _rows(w, torch.bfloat16, "w")
    if want_q and q is None:
        q = torch.empty((K, N), dtype=torch.uint8, device=w.device)
    if want_qT and qT is None:
        qT = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((_cdiv(K, TILE), _cdiv(N, TILE)), dtype=torch.float32, device=w.device)
    ldq = _rows(q, torch.uint8, "q") if q is not None else 0
    ldqT = _rows(qT, torch.uint8, "qT") if qT is not None else 0
    _check(_quant_call("fgb_quantize_128x128", ue8m0, sr, (_ptr(w), K, N, ldw, amax_floor, _ptr(q), ldq, _ptr(qT),
                       ldqT, _ptr(s), _stream(w))), "quantize_128x128")
    return q, qT, s


def quantize_128x128_batched(w: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True, want_qT: bool = True,
                             q=None, qT=None, s=None, ue8m0: bool = False):
    """E stacked weights w [E, K, N] (contiguous bf16) in one launch -> (q [E, K, N],
    qT [E, N, K], s [E, K/128, N/128]), each matrix as quantize_128x128 alone."""
    if w.dim() != 3:
        raise FgbError("quantize_128x128_batched: w must be [E, K, N]")
    E, K, N = w.shape
    dev = w.device
    if want_q and q is None:
        q = torch.empty((E, K, N), dtype=torch.uint8, device=dev)
    if want_qT and qT is None:
        qT = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    if s is None:
        s = torch.empty((E, _cdiv(K, TILE), _cdiv(N, TILE)), dtype=torch.float32, device=dev)
    for t, dt, shape in ((w, torch.bfloat16, (E, K, N)), (q, torch.uint8, (E, K, N)), (qT, torch.uint8, (E, N, K)),
                         (s, torch.float32, (E, _cdiv(K, TILE), _cdiv(N, TILE)))):
        if t is not None and (t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous()):
            raise FgbError(f"quantize_128x128_batched: expected contiguous {dt} {shape}")
    _check(_fn("fgb_quantize_128x128_batched", ue8m0)(E, _ptr(w), K, N, amax_floor, _ptr(q), _ptr(qT), _ptr(s),
                                                      _stream(w)), "quantize_128x128_batched")
    return q, qT, s


def requant_128x1(q: torch.Tensor, s: torch.Tensor, qT=None, sT=None, ue8m0: bool = False):
    R, C = q.shape
    ldq = _rows(q, torch.uint8, "q")
    if qT is None:
        qT = torch.empty((C, _cdiv(R, TILE) * TILE), dtype=torch.uint8, device=q.device)
    if sT is None:
        sT = torch.empty((_cdiv(R, TILE), C), dtype=torch.float32, device=q.device)
    _check(_fn("fgb_requant_128x1", ue8m0)(_ptr(q), R, C, ldq, _ptr(s), _rows(s, torch.float32, "s"),
                                   _ptr(qT), _rows(qT, torch.uint8, "qT"), _ptr(sT),
                                   _rows(sT, torch.float32, "sT"), _stream(q)), "requant_128x1")
    return qT, sT


def requant_128x128_ue8m0(q: torch.Tensor, s: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True,
                          want_qT: bool = True, q2=None, q2T=None, s2=None):
    """Second stage of the two-stage weight cast: a 128x128 E4M3 weight (codes q
    [K, N], fp32 tile scales s [K/128, N/128] as quantize_128x128 returns them)
    requantized to power-of-two tiles -> (q2 [K, N], q2T [N, K], s2 [K/128, N/128])."""
    K, N = q.shape
    ldq = _rows(q, torch.uint8, "q")
    if s.dtype != torch.float32 or tuple(s.shape) != (_cdiv(K, TILE), _cdiv(N, TILE)) or not s.is_contiguous():
        raise FgbError(f"requant_128x128_ue8m0: s must be contiguous float32 [{_cdiv(K, TILE)}, {_cdiv(N, TILE)}]")
    if want_q and q2 is None:
        q2 = torch.empty((K, N), dtype=torch.uint8, device=q.device)
    if want_qT and q2T is None:
        q2T = torch.empty((N, K), dtype=torch.uint8, device=q.device)
    if s2 is None:
        s2 = torch.empty((_cdiv(K, TILE), _cdiv(N, TILE)), dtype=torch.float32, device=q.device)
    ldq2 = _rows(q2, torch.uint8, "q2") if q2 is not None else 0
    ldq2T = _rows(q2T, torch.uint8, "q2T") if q2T is not None else 0
    _check(_fn("fgb_requant_128x128", True)(_ptr(q), K, N, ldq, _ptr(s), amax_floor, _ptr(q2), ldq2, _ptr(q2T),
                                            ldq2T, _ptr(s2), _stream(q)), "requant_128x128_ue8m0")
    return q2, q2T, s2


# ---------------------------------------------------------------------------
# SwiGLU with fused casts ([G | U] is one [R, 2F] bf16 tensor)
# ---------------------------------------------------------------------------

def swiglu_fwd_quant(gu: torch.Tensor, amax_floor: float = 0.0, stash: bool = True, want_h: bool = False,
                     q_gu=None, s_gu=None, q_h=None, s_h=None, h=None):
    """H = bf16(silu(G) U): returns (q_gu, s_gu, q_h, s_h, h) -- the 1x128 stash of
    [G | U] (None when stash=False), the 1x128 codes/scales of H, and H (when want_h)."""
    R, F2 = gu.shape
    F = F2 // 2
    ldgu = _rows(gu, torch.bfloat16, "gu")
    dev = gu.device
    if stash:
        q_gu = torch.empty((R, F2), dtype=torch.uint8, device=dev) if q_gu is None else q_gu
        s_gu = torch.empty((_cdiv(F2, TILE), R), dtype=torch.float32, device=dev) if s_gu is None else s_gu
    q_h = torch.empty((R, F), dtype=torch.uint8, device=dev) if q_h is None else q_h
    s_h = torch.empty((_cdiv(F, TILE), R), dtype=torch.float32, device=dev) if s_h is None else s_h
    if want_h and h is None:
        h = torch.empty((R, F), dtype=torch.bfloat16, device=dev)
    _check(lib().fgb_swiglu_fwd_quant(
        _ptr(gu), R, F, ldgu, amax_floor,
        _ptr(q_gu), _rows(q_gu, torch.uint8, "q_gu") if q_gu is not None else 0,
        _ptr(s_gu), _rows(s_gu, torch.float32, "s_gu") if s_gu is not None else 0,
        _ptr(q_h), _rows(q_h, torch.uint8, "q_h"), _ptr(s_h), _rows(s_h, torch.float32, "s_h"),
        _ptr(h), _rows(h, torch.bfloat16, "h") if h is not None else 0, _stream(gu)), "swiglu_fwd_quant")
    return q_gu, s_gu, q_h, s_h, h


def swiglu_bwd_quant(q_gu: torch.Tensor, s_gu: torch.Tensor, dh: torch.Tensor, amax_floor: float = 0.0,
                     want_dgu: bool = False, q=None, s=None, qT=None, sT=None, dgu=None):
    """[dG | dU] from the stash and dH, quantized both ways: returns (q, s, qT, sT, dgu)
    with (q, s) as quantize_1x128 and (qT, sT) as quantize_128x1 of [dG | dU]
    (dgu itself when want_dgu)."""
    R, F2 = q_gu.shape
    F = F2 // 2
    dev = q_gu.device
    q = torch.empty((R, F2), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((_cdiv(F2, TILE), R), dtype=torch.float32, device=dev) if s is None else s
    qT = torch.empty((F2, _cdiv(R, TILE) * TILE), dtype=torch.uint8, device=dev) if qT is None else qT
    sT = torch.empty((_cdiv(R, TILE), F2), dtype=torch.float32, device=dev) if sT is None else sT
    if want_dgu and dgu is None:
        dgu = torch.empty((R, F2), dtype=torch.bfloat16, device=dev)
    _check(lib().fgb_swiglu_bwd_quant(
        _ptr(q_gu), R, F, _rows(q_gu, torch.uint8, "q_gu"), _ptr(s_gu), _rows(s_gu, torch.float32, "s_gu"),
        _ptr(dh), _rows(dh, torch.bfloat16, "dh"), amax_floor,
        _ptr(q), _rows(q, torch.uint8, "q"), _ptr(s), _rows(s, torch.float32, "s"),
        _ptr(qT), _rows(qT, torch.uint8, "qT"), _ptr(sT), _rows(sT, torch.float32, "sT"),
        _ptr(dgu), _rows(dgu, torch.bfloat16, "dgu") if dgu is not None else 0, _stream(q_gu)),
        "swiglu_bwd_quant")
    return q, s, qT, sT, dgu


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def gemm_fprop(qx, sx, qwT, sw, y=None, ue8m0: bool = False):
    M, K = qx.shape
    N = qwT.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qx.device)
    _check(_fn("fgb_gemm_fprop", ue8m0)(M, N, K, _ptr(qx), _rows(qx, torch.uint8, "qx"), _ptr(sx),
                                _rows(sx, torch.float32, "sx") if K else M, _ptr(qwT),
                                _rows(qwT, torch.uint8, "qwT"), _ptr(sw), _ptr(y),
                                _rows(y, torch.bfloat16, "y"), _stream(qx)), "gemm_fprop")
    return y


def gemm_dgrad(qdy, sdy, qw, sw, dx=None, ue8m0: bool = False):
    M, N = qdy.shape
    K = qw.shape[0]
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=qdy.device)
    _check(_fn("fgb_gemm_dgrad", ue8m0)(M, K, N, _ptr(qdy), _rows(qdy, torch.uint8, "qdy"), _ptr(sdy),
                                _rows(sdy, torch.float32, "sdy") if N else M, _ptr(qw),
                                _rows(qw, torch.uint8, "qw"), _ptr(sw), _ptr(dx),
                                _rows(dx, torch.bfloat16, "dx"), _stream(qdy)), "gemm_dgrad")
    return dx


def gemm_wgrad(qxT, sxT, qdyT, sdyT, M: int, dw=None, accumulate: bool = False, ue8m0: bool = False):
    K = qxT.shape[0]
    N = qdyT.shape[0]
    if dw is None:
        dw = torch.empty((K, N), dtype=torch.float32, device=qxT.device)
    _check(_fn("fgb_gemm_wgrad", ue8m0)(K, N, M, _ptr(qxT), _rows(qxT, torch.uint8, "qxT"), _ptr(sxT),
                                _rows(sxT, torch.float32, "sxT") if M else K, _ptr(qdyT),
                                _rows(qdyT, torch.uint8, "qdyT"), _ptr(sdyT),
                                _rows(sdyT, torch.float32, "sdyT") if M else N, _ptr(dw),
                                _rows(dw, torch.float32, "dw"), 1 if accumulate else 0,
                                _stream(qxT)), "gemm_wgrad")
    return dw


def _offsets(offsets: torch.Tensor):
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1:
        raise FgbError("offsets: expected a 1-D int32 device tensor of E+1 entries")
    return offsets.numel() - 1


def _contiguous(t):
    if not t.is_contiguous():
        raise ValueError("grouped GEMM operands must be contiguous tensors")


def gemm_fprop_grouped(offsets, qx, sx, qwT, sw, y=None, ue8m0: bool = False):
    E = _offsets(offsets)
    R_pad, K = qx.shape
    N = qwT.shape[1]
    if y is None:
        y = torch.empty((R_pad, N), dtype=torch.bfloat16, device=qx.device)
    for t in (qx, sx, qwT, sw, y):
        _contiguous(t)
    _check(_fn("fgb_gemm_fprop_grouped", ue8m0)(E, _ptr(offsets), R_pad, N, K, _ptr(qx), _ptr(sx), _ptr(qwT),
                                        _ptr(sw), _ptr(y), _stream(qx)), "gemm_fprop_grouped")
    return y


def gemm_dgrad_grouped(offsets, qdy, sdy, qw, sw, dx=None, ue8m0: bool = False):
    E = _offsets(offsets)
    R_pad, N = qdy.shape
    K = qw.shape[1]
    if dx is None:
        dx = torch.empty((R_pad, K), dtype=torch.bfloat16, device=qdy.device)
    for t in (qdy, sdy, qw, sw, dx):
        _contiguous(t)
    _check(_fn("fgb_gemm_dgrad_grouped", ue8m0)(E, _ptr(offsets), R_pad, K, N, _ptr(qdy), _ptr(sdy), _ptr(qw),
                                        _ptr(sw), _ptr(dx), _stream(qdy)), "gemm_dgrad_grouped")
    return dx


def gemm_wgrad_grouped(offsets, qxT, sxT, qdyT, sdyT, dw=None, accumulate: bool = False, ue8m0: bool = False):
    E = _offsets(offsets)
    K, R_pad = qxT.shape
    N = qdyT.shape[0]
    if dw is None:
        dw = torch.empty((E, K, N), dtype=torch.float32, device=qxT.device)
    for t in (qxT, sxT, qdyT, sdyT, dw):
        _contiguous(t)
    _check(_fn("fgb_gemm_wgrad_grouped", ue8m0)(E, _ptr(offsets), R_pad, K, N, _ptr(qxT), _ptr(sxT), _ptr(qdyT),
                                        _ptr(sdyT), _ptr(dw), 1 if accumulate else 0, _stream(qxT)),
           "gemm_wgrad_grouped")
    return dw
