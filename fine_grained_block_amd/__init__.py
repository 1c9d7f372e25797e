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


def _cdiv(a, b):
    return -(-a // b)


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI sees pointers and sizes only, so every tensor is
# checked here -- dtype, device, exact shape, layout -- before any call: a
# short or misplaced buffer must raise, never reach a kernel.
# ---------------------------------------------------------------------------

def _input(t, dtype, name: str, ndim: int = 2):
    """A caller's input tensor: a device tensor of `dtype` with `ndim` dims; returns its device."""
    if not isinstance(t, torch.Tensor):
        raise FgbError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise FgbError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise FgbError(f"{name}: expected a device tensor, got one on {t.device}")
    if t.dim() != ndim:
        raise FgbError(f"{name}: expected {ndim} dimensions, got shape {tuple(t.shape)}")
    return t.device


def _mat(t, dtype, shape, dev, name: str) -> int:
    """A 2-D row-major tensor of exactly `shape` and `dtype` on `dev` (rows may
    be strided); returns its leading dimension in elements."""
    if not isinstance(t, torch.Tensor):
        raise FgbError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise FgbError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != dev:
        raise FgbError(f"{name}: expected a device tensor on {dev}, got one on {t.device}")
    shape = tuple(int(v) for v in shape)
    if tuple(t.shape) != shape:
        raise FgbError(f"{name}: expected shape {shape}, got {tuple(t.shape)}")
    rows, cols = shape
    if rows == 0 or cols == 0:
        return max(cols, 1)                     # empty: nothing is addressed
    if cols > 1 and t.stride(1) != 1:
        raise FgbError(f"{name}: expected a row-major tensor (unit column stride)")
    if rows > 1:
        if t.stride(0) < cols:
            raise FgbError(f"{name}: row stride {t.stride(0)} is smaller than the row length {cols}")
        return t.stride(0)
    return max(cols, 1)


def _dense(t, dtype, shape, dev, name: str):
    """A contiguous tensor of exactly `shape` and `dtype` on `dev`."""
    if not isinstance(t, torch.Tensor):
        raise FgbError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise FgbError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != dev:
        raise FgbError(f"{name}: expected a device tensor on {dev}, got one on {t.device}")
    shape = tuple(int(v) for v in shape)
    if tuple(t.shape) != shape:
        raise FgbError(f"{name}: expected shape {shape}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise FgbError(f"{name}: expected a contiguous tensor")


def _new(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


_U8, _F32, _BF16 = torch.uint8, torch.float32, torch.bfloat16


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
    dev = _input(x, _BF16, "x")
    R, C = x.shape
    ldx = _mat(x, _BF16, (R, C), dev, "x")
    q = _new((R, C), _U8, dev) if q is None else q
    s = _new((_cdiv(C, TILE), R), _F32, dev) if s is None else s
    ldq = _mat(q, _U8, (R, C), dev, "q")
    lds = _mat(s, _F32, (_cdiv(C, TILE), R), dev, "s")
    _check(_quant_call("fgb_quantize_1x128", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor, _ptr(q), ldq, _ptr(s), lds,
                                                         _stream(x))), "quantize_1x128")
    return q, s


def quantize_128x1(x: torch.Tensor, amax_floor: float = 0.0, qT=None, sT=None, ue8m0: bool = False, sr=None):
    dev = _input(x, _BF16, "x")
    R, C = x.shape
    ldx = _mat(x, _BF16, (R, C), dev, "x")
    Rp = _cdiv(R, TILE) * TILE
    qT = _new((C, Rp), _U8, dev) if qT is None else qT
    sT = _new((_cdiv(R, TILE), C), _F32, dev) if sT is None else sT
    ldqT = _mat(qT, _U8, (C, Rp), dev, "qT")
    ldsT = _mat(sT, _F32, (_cdiv(R, TILE), C), dev, "sT")
    _check(_quant_call("fgb_quantize_128x1", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor, _ptr(qT), ldqT, _ptr(sT),
                                                         ldsT, _stream(x))), "quantize_128x1")
    return qT, sT


def quantize_dual(x: torch.Tensor, amax_floor: float = 0.0, q=None, s=None, qT=None, sT=None, ue8m0: bool = False,
                  sr=None):
    """Both orientations from one read: (q, s) as quantize_1x128, (qT, sT) as quantize_128x1."""
    dev = _input(x, _BF16, "x")
    R, C = x.shape
    ldx = _mat(x, _BF16, (R, C), dev, "x")
    Rp = _cdiv(R, TILE) * TILE
    q = _new((R, C), _U8, dev) if q is None else q
    s = _new((_cdiv(C, TILE), R), _F32, dev) if s is None else s
    qT = _new((C, Rp), _U8, dev) if qT is None else qT
    sT = _new((_cdiv(R, TILE), C), _F32, dev) if sT is None else sT
    ldq = _mat(q, _U8, (R, C), dev, "q")
    lds = _mat(s, _F32, (_cdiv(C, TILE), R), dev, "s")
    ldqT = _mat(qT, _U8, (C, Rp), dev, "qT")
    ldsT = _mat(sT, _F32, (_cdiv(R, TILE), C), dev, "sT")
    _check(_quant_call("fgb_quantize_dual", ue8m0, sr, (_ptr(x), R, C, ldx, amax_floor, _ptr(q), ldq, _ptr(s), lds,
                                                        _ptr(qT), ldqT, _ptr(sT), ldsT, _stream(x))),
           "quantize_dual")
    return q, s, qT, sT


def quantize_128x128(w: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True, want_qT: bool = True,
                     q=None, qT=None, s=None, ue8m0: bool = False, sr=None):
    dev = _input(w, _BF16, "w")
    K, N = w.shape
    ldw = _mat(w, _BF16, (K, N), dev, "w")
    if want_q and q is None:
        q = _new((K, N), _U8, dev)
    if want_qT and qT is None:
        qT = _new((N, K), _U8, dev)
    s = _new((_cdiv(K, TILE), _cdiv(N, TILE)), _F32, dev) if s is None else s
    ldq = _mat(q, _U8, (K, N), dev, "q") if q is not None else 0
    ldqT = _mat(qT, _U8, (N, K), dev, "qT") if qT is not None else 0
    _dense(s, _F32, (_cdiv(K, TILE), _cdiv(N, TILE)), dev, "s")
    _check(_quant_call("fgb_quantize_128x128", ue8m0, sr, (_ptr(w), K, N, ldw, amax_floor, _ptr(q), ldq, _ptr(qT),
                                                           ldqT, _ptr(s), _stream(w))), "quantize_128x128")
    return q, qT, s


def quantize_128x128_batched(w: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True, want_qT: bool = True,
                             q=None, qT=None, s=None, ue8m0: bool = False):
    """E stacked weights w [E, K, N] (contiguous bf16) in one launch -> (q [E, K, N],
    qT [E, N, K], s [E, K/128, N/128]), each matrix as quantize_128x128 alone."""
    dev = _input(w, _BF16, "w", ndim=3)
    E, K, N = w.shape
    if want_q and q is None:
        q = _new((E, K, N), _U8, dev)
    if want_qT and qT is None:
        qT = _new((E, N, K), _U8, dev)
    s = _new((E, _cdiv(K, TILE), _cdiv(N, TILE)), _F32, dev) if s is None else s
    _dense(w, _BF16, (E, K, N), dev, "w")
    if q is not None:
        _dense(q, _U8, (E, K, N), dev, "q")
    if qT is not None:
        _dense(qT, _U8, (E, N, K), dev, "qT")
    _dense(s, _F32, (E, _cdiv(K, TILE), _cdiv(N, TILE)), dev, "s")
    _check(_fn("fgb_quantize_128x128_batched", ue8m0)(E, _ptr(w), K, N, amax_floor, _ptr(q), _ptr(qT), _ptr(s),
                                                      _stream(w)), "quantize_128x128_batched")
    return q, qT, s


def requant_128x1(q: torch.Tensor, s: torch.Tensor, qT=None, sT=None, ue8m0: bool = False):
    dev = _input(q, _U8, "q")
    R, C = q.shape
    ldq = _mat(q, _U8, (R, C), dev, "q")
    lds = _mat(s, _F32, (_cdiv(C, TILE), R), dev, "s")
    Rp = _cdiv(R, TILE) * TILE
    qT = _new((C, Rp), _U8, dev) if qT is None else qT
    sT = _new((_cdiv(R, TILE), C), _F32, dev) if sT is None else sT
    ldqT = _mat(qT, _U8, (C, Rp), dev, "qT")
    ldsT = _mat(sT, _F32, (_cdiv(R, TILE), C), dev, "sT")
    _check(_fn("fgb_requant_128x1", ue8m0)(_ptr(q), R, C, ldq, _ptr(s), lds, _ptr(qT), ldqT, _ptr(sT), ldsT,
                                           _stream(q)), "requant_128x1")
    return qT, sT


def requant_128x128_ue8m0(q: torch.Tensor, s: torch.Tensor, amax_floor: float = 0.0, want_q: bool = True,
                          want_qT: bool = True, q2=None, q2T=None, s2=None):
    """Second stage of the two-stage weight cast: a 128x128 E4M3 weight (codes q
    [K, N], fp32 tile scales s [K/128, N/128] as quantize_128x128 returns them)
    requantized to power-of-two tiles -> (q2 [K, N], q2T [N, K], s2 [K/128, N/128])."""
    dev = _input(q, _U8, "q")
    K, N = q.shape
    ldq = _mat(q, _U8, (K, N), dev, "q")
    _dense(s, _F32, (_cdiv(K, TILE), _cdiv(N, TILE)), dev, "s")
    if want_q and q2 is None:
        q2 = _new((K, N), _U8, dev)
    if want_qT and q2T is None:
        q2T = _new((N, K), _U8, dev)
    s2 = _new((_cdiv(K, TILE), _cdiv(N, TILE)), _F32, dev) if s2 is None else s2
    ldq2 = _mat(q2, _U8, (K, N), dev, "q2") if q2 is not None else 0
    ldq2T = _mat(q2T, _U8, (N, K), dev, "q2T") if q2T is not None else 0
    _dense(s2, _F32, (_cdiv(K, TILE), _cdiv(N, TILE)), dev, "s2")
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
    dev = _input(gu, _BF16, "gu")
    R, F2 = gu.shape
    if F2 % 2:
        raise FgbError(f"gu: expected an even width [G | U], got {F2}")
    F = F2 // 2
    ldgu = _mat(gu, _BF16, (R, F2), dev, "gu")
    if stash:
        q_gu = _new((R, F2), _U8, dev) if q_gu is None else q_gu
        s_gu = _new((_cdiv(F2, TILE), R), _F32, dev) if s_gu is None else s_gu
    q_h = _new((R, F), _U8, dev) if q_h is None else q_h
    s_h = _new((_cdiv(F, TILE), R), _F32, dev) if s_h is None else s_h
    if want_h and h is None:
        h = _new((R, F), _BF16, dev)
    ldq_gu = _mat(q_gu, _U8, (R, F2), dev, "q_gu") if q_gu is not None else 0
    lds_gu = _mat(s_gu, _F32, (_cdiv(F2, TILE), R), dev, "s_gu") if s_gu is not None else 0
    ldq_h = _mat(q_h, _U8, (R, F), dev, "q_h")
    lds_h = _mat(s_h, _F32, (_cdiv(F, TILE), R), dev, "s_h")
    ldh = _mat(h, _BF16, (R, F), dev, "h") if h is not None else 0
    _check(lib().fgb_swiglu_fwd_quant(_ptr(gu), R, F, ldgu, amax_floor, _ptr(q_gu), ldq_gu, _ptr(s_gu), lds_gu,
                                      _ptr(q_h), ldq_h, _ptr(s_h), lds_h, _ptr(h), ldh, _stream(gu)),
           "swiglu_fwd_quant")
    return q_gu, s_gu, q_h, s_h, h


def swiglu_bwd_quant(q_gu: torch.Tensor, s_gu: torch.Tensor, dh: torch.Tensor, amax_floor: float = 0.0,
                     want_dgu: bool = False, q=None, s=None, qT=None, sT=None, dgu=None):
    """[dG | dU] from the stash and dH, quantized both ways: returns (q, s, qT, sT, dgu)
    with (q, s) as quantize_1x128 and (qT, sT) as quantize_128x1 of [dG | dU]
    (dgu itself when want_dgu)."""
    dev = _input(q_gu, _U8, "q_gu")
    R, F2 = q_gu.shape
    if F2 % 2:
        raise FgbError(f"q_gu: expected an even width [G | U], got {F2}")
    F = F2 // 2
    Rp = _cdiv(R, TILE) * TILE
    ldq_gu = _mat(q_gu, _U8, (R, F2), dev, "q_gu")
    lds_gu = _mat(s_gu, _F32, (_cdiv(F2, TILE), R), dev, "s_gu")
    lddh = _mat(dh, _BF16, (R, F), dev, "dh")
    q = _new((R, F2), _U8, dev) if q is None else q
    s = _new((_cdiv(F2, TILE), R), _F32, dev) if s is None else s
    qT = _new((F2, Rp), _U8, dev) if qT is None else qT
    sT = _new((_cdiv(R, TILE), F2), _F32, dev) if sT is None else sT
    if want_dgu and dgu is None:
        dgu = _new((R, F2), _BF16, dev)
    ldq = _mat(q, _U8, (R, F2), dev, "q")
    lds = _mat(s, _F32, (_cdiv(F2, TILE), R), dev, "s")
    ldqT = _mat(qT, _U8, (F2, Rp), dev, "qT")
    ldsT = _mat(sT, _F32, (_cdiv(R, TILE), F2), dev, "sT")
    lddgu = _mat(dgu, _BF16, (R, F2), dev, "dgu") if dgu is not None else 0
    _check(lib().fgb_swiglu_bwd_quant(_ptr(q_gu), R, F, ldq_gu, _ptr(s_gu), lds_gu, _ptr(dh), lddh, amax_floor,
                                      _ptr(q), ldq, _ptr(s), lds, _ptr(qT), ldqT, _ptr(sT), ldsT,
                                      _ptr(dgu), lddgu, _stream(q_gu)), "swiglu_bwd_quant")
    return q, s, qT, sT, dgu


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def _weight_scales(sw, K, N, dev, name="sw"):
    _dense(sw, _F32, (_cdiv(K, TILE), _cdiv(N, TILE)), dev, name)


def gemm_fprop(qx, sx, qwT, sw, y=None, ue8m0: bool = False):
    """Y [M, N] bf16 = X W from qx [M, K] (1x128 scales sx [K/128, M]) and qwT [N, K]
    (W's transposed codes, 128x128 scales sw [K/128, N/128], contiguous)."""
    dev = _input(qx, _U8, "qx")
    M, K = qx.shape
    _input(qwT, _U8, "qwT")
    N = qwT.shape[0]
    ldqx = _mat(qx, _U8, (M, K), dev, "qx")
    ldsx = _mat(sx, _F32, (_cdiv(K, TILE), M), dev, "sx")
    ldqw = _mat(qwT, _U8, (N, K), dev, "qwT")
    _weight_scales(sw, K, N, dev)
    y = _new((M, N), _BF16, dev) if y is None else y
    ldy = _mat(y, _BF16, (M, N), dev, "y")
    _check(_fn("fgb_gemm_fprop", ue8m0)(M, N, K, _ptr(qx), ldqx, _ptr(sx), ldsx if K else M, _ptr(qwT), ldqw,
                                        _ptr(sw), _ptr(y), ldy, _stream(qx)), "gemm_fprop")
    return y


def gemm_dgrad(qdy, sdy, qw, sw, dx=None, ue8m0: bool = False):
    """dX [M, K] bf16 = dY W^T from qdy [M, N] (1x128 scales sdy [N/128, M]) and qw
    [K, N] (W's codes, 128x128 scales sw [K/128, N/128], contiguous)."""
    dev = _input(qdy, _U8, "qdy")
    M, N = qdy.shape
    _input(qw, _U8, "qw")
    K = qw.shape[0]
    ldqdy = _mat(qdy, _U8, (M, N), dev, "qdy")
    ldsdy = _mat(sdy, _F32, (_cdiv(N, TILE), M), dev, "sdy")
    ldqw = _mat(qw, _U8, (K, N), dev, "qw")
    _weight_scales(sw, K, N, dev)
    dx = _new((M, K), _BF16, dev) if dx is None else dx
    lddx = _mat(dx, _BF16, (M, K), dev, "dx")
    _check(_fn("fgb_gemm_dgrad", ue8m0)(M, K, N, _ptr(qdy), ldqdy, _ptr(sdy), ldsdy if N else M, _ptr(qw), ldqw,
                                        _ptr(sw), _ptr(dx), lddx, _stream(qdy)), "gemm_dgrad")
    return dx


def gemm_wgrad(qxT, sxT, qdyT, sdyT, M: int, dw=None, accumulate: bool = False, ue8m0: bool = False):
    """dW [K, N] fp32 = X^T dY over the first M tokens, from the 128x1 operands qxT
    [K, Mp], sxT [ceil(M/128), K] and qdyT [N, Mp], sdyT [ceil(M/128), N], Mp the
    operands' padded token count (>= roundup(M, 128), zero past M)."""
    dev = _input(qxT, _U8, "qxT")
    K, Mp = qxT.shape
    _input(qdyT, _U8, "qdyT")
    N = qdyT.shape[0]
    M = int(M)
    if M < 0 or Mp < _cdiv(M, TILE) * TILE:
        raise FgbError(f"gemm_wgrad: M = {M} needs operands of at least {_cdiv(M, TILE) * TILE} padded "
                       f"columns, got {Mp}")
    nb = _cdiv(M, TILE)
    ldqx = _mat(qxT, _U8, (K, Mp), dev, "qxT")
    ldqdy = _mat(qdyT, _U8, (N, Mp), dev, "qdyT")
    if sxT.dim() != 2 or sxT.shape[0] < nb or sdyT.dim() != 2 or sdyT.shape[0] < nb:
        raise FgbError(f"gemm_wgrad: sxT/sdyT need at least {nb} scale rows")
    ldsx = _mat(sxT, _F32, (sxT.shape[0], K), dev, "sxT")
    ldsdy = _mat(sdyT, _F32, (sdyT.shape[0], N), dev, "sdyT")
    dw = _new((K, N), _F32, dev) if dw is None else dw
    lddw = _mat(dw, _F32, (K, N), dev, "dw")
    _check(_fn("fgb_gemm_wgrad", ue8m0)(K, N, M, _ptr(qxT), ldqx, _ptr(sxT), ldsx if M else K, _ptr(qdyT), ldqdy,
                                        _ptr(sdyT), ldsdy if M else N, _ptr(dw), lddw, 1 if accumulate else 0,
                                        _stream(qxT)), "gemm_wgrad")
    return dw


def _offsets(offsets, dev):
    if not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int32 or offsets.dim() != 1 \
            or offsets.numel() < 1:
        raise FgbError("offsets: expected a 1-D int32 tensor of E+1 entries")
    if not offsets.is_cuda or offsets.device != dev:
        raise FgbError(f"offsets: expected a device tensor on {dev}, got one on {offsets.device}")
    if not offsets.is_contiguous():
        raise FgbError("offsets: expected a contiguous tensor")
    return offsets.numel() - 1


def gemm_fprop_grouped(offsets, qx, sx, qwT, sw, y=None, ue8m0: bool = False):
    """Per expert e: Y[o_e:o_{e+1}] = X[o_e:o_{e+1}] W_e.  qx [R_pad, K], sx [K/128,
    R_pad], qwT [E, N, K], sw [E, K/128, N/128], y [R_pad, N]; all contiguous."""
    dev = _input(qx, _U8, "qx")
    E = _offsets(offsets, dev)
    R_pad, K = qx.shape
    _input(qwT, _U8, "qwT", ndim=3)
    N = qwT.shape[1]
    _dense(qx, _U8, (R_pad, K), dev, "qx")
    _dense(sx, _F32, (_cdiv(K, TILE), R_pad), dev, "sx")
    _dense(qwT, _U8, (E, N, K), dev, "qwT")
    _dense(sw, _F32, (E, _cdiv(K, TILE), _cdiv(N, TILE)), dev, "sw")
    y = _new((R_pad, N), _BF16, dev) if y is None else y
    _dense(y, _BF16, (R_pad, N), dev, "y")
    _check(_fn("fgb_gemm_fprop_grouped", ue8m0)(E, _ptr(offsets), R_pad, N, K, _ptr(qx), _ptr(sx), _ptr(qwT),
                                                _ptr(sw), _ptr(y), _stream(qx)), "gemm_fprop_grouped")
    return y


def gemm_dgrad_grouped(offsets, qdy, sdy, qw, sw, dx=None, ue8m0: bool = False):
    """Per expert e: dX[o_e:o_{e+1}] = dY[o_e:o_{e+1}] W_e^T.  qdy [R_pad, N], sdy
    [N/128, R_pad], qw [E, K, N], sw [E, K/128, N/128], dx [R_pad, K]; all contiguous."""
    dev = _input(qdy, _U8, "qdy")
    E = _offsets(offsets, dev)
    R_pad, N = qdy.shape
    _input(qw, _U8, "qw", ndim=3)
    K = qw.shape[1]
    _dense(qdy, _U8, (R_pad, N), dev, "qdy")
    _dense(sdy, _F32, (_cdiv(N, TILE), R_pad), dev, "sdy")
    _dense(qw, _U8, (E, K, N), dev, "qw")
    _dense(sw, _F32, (E, _cdiv(K, TILE), _cdiv(N, TILE)), dev, "sw")
    dx = _new((R_pad, K), _BF16, dev) if dx is None else dx
    _dense(dx, _BF16, (R_pad, K), dev, "dx")
    _check(_fn("fgb_gemm_dgrad_grouped", ue8m0)(E, _ptr(offsets), R_pad, K, N, _ptr(qdy), _ptr(sdy), _ptr(qw),
                                                _ptr(sw), _ptr(dx), _stream(qdy)), "gemm_dgrad_grouped")
    return dx


def gemm_wgrad_grouped(offsets, qxT, sxT, qdyT, sdyT, dw=None, accumulate: bool = False, ue8m0: bool = False):
    """Per expert e: dW_e = X[o_e:o_{e+1}]^T dY[o_e:o_{e+1}].  qxT [K, R_pad], sxT
    [R_pad/128, K], qdyT [N, R_pad], sdyT [R_pad/128, N], dw [E, K, N]; all contiguous."""
    dev = _input(qxT, _U8, "qxT")
    E = _offsets(offsets, dev)
    K, R_pad = qxT.shape
    _input(qdyT, _U8, "qdyT")
    N = qdyT.shape[0]
    _dense(qxT, _U8, (K, R_pad), dev, "qxT")
    _dense(sxT, _F32, (_cdiv(R_pad, TILE), K), dev, "sxT")
    _dense(qdyT, _U8, (N, R_pad), dev, "qdyT")
    _dense(sdyT, _F32, (_cdiv(R_pad, TILE), N), dev, "sdyT")
    dw = _new((E, K, N), _F32, dev) if dw is None else dw
    _dense(dw, _F32, (E, K, N), dev, "dw")
    _check(_fn("fgb_gemm_wgrad_grouped", ue8m0)(E, _ptr(offsets), R_pad, K, N, _ptr(qxT), _ptr(sxT), _ptr(qdyT),
                                                _ptr(sdyT), _ptr(dw), 1 if accumulate else 0, _stream(qxT)),
           "gemm_wgrad_grouped")
    return dw
