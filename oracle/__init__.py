"""Plain CPU oracle for the fine-grained FP8 linear-layer path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``fine_grained_block_amd``) never imports it, and the two share no code.

The arithmetic lives in ``fgb_oracle.c`` (plain loops, fp64 where the method
leaves the precision free); this module only marshals numpy arrays.  What each
function computes, with the passage it follows:

* ``e4m3_decode`` / ``e4m3_encode`` -- the E4M3 element format.  prime-rl
  PR #4073, conventions table: scales divide by 448 and -0 (0x80) is kept apart
  from +0; "RN" cast.  Read as OCP E4M3FN with ties-to-even and saturation.
* ``quantize_1x128`` / ``quantize_128x128`` -- dynamic tile quantization with
  scale = tile absmax / 448.  "scratch: the backward pass, unrolled", section
  "What is asserted, and from where" (1x128 activation tiles, 128x128 weight
  tiles); partial-sum-drift notes, section 3, row (a) (per-block absmax scale,
  N_c = 128).
* ``quantize_128x1`` / ``requant_128x1`` -- the 128x1 re-tiling of Wgrad's
  transposed operands: same section of the "scratch" page (re-quantized 128x1
  from the saved tensors; backward casts emit both tile orientations).
* ``gemm_fprop`` / ``gemm_dgrad`` / ``gemm_wgrad`` -- block-scaled GEMM: each
  128-long contraction segment's partial sum times s_a*s_b, accumulated at high
  precision.  Partial-sum-drift notes, section 3 rows (a)-(b) and section 5;
  output dtypes from the "scratch" page (Fprop/Dgrad BF16, Wgrad FP32).
* ``*_grouped`` -- the same per expert over 128-aligned row segments (grouped
  expert GEMMs with empty experts, prime-rl PR #4073 "Validation completed").
* ``*_ue8m0`` quantizers -- power-of-two scales stored as E8M0 bytes (prime-rl
  PR #4073 "Results": the power-of-two scale format); the GEMMs take them as
  fp32 scales through ``e8m0_decode``.
* ``swiglu_*`` -- SwiGLU with its casts fused into the producer kernels ("scratch"
  page, same section: the SwiGLU input saved as E4M3, backward casts emitting
  both orientations, backward computing in BF16 from the dequantized input).
* ``*_sr`` quantizers, ``philox4x32_10``, ``e4m3_encode_sr`` -- stochastic
  rounding of the cast (prime-rl PR #4073 conventions row "SR agreement":
  stateless seed/salt/counter words from Philox, lower/upper-magnitude
  neighbour); Philox4x32-10 as published by Salmon et al. (SC'11).

The GEMM functions return the exact-to-fp64 value ``r`` and the absolute sum
``aabs`` (sum of |terms|), not a rounded output; callers compare the GPU's
BF16/FP32 output against ``r``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fgb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# the mutation tests load a deliberately broken build of the same source from here
_LIB_OVERRIDE = os.environ.get("FGB_ORACLE_LIB")
TILE = 128

_lib = None


def compile_oracle(src: str, out: str) -> str:
    """gcc with IEEE arithmetic: no fast-math, no FMA contraction."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle in place (oracle/liboracle.so)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_oracle(_SRC, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        # (re)build when the library is missing or older than its source
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [F]
    lib.orc_bf16_round.restype = ctypes.c_uint16
    lib.orc_bf16_round.argtypes = [ctypes.c_double]
    lib.orc_quantize_1x128.argtypes = [P, I64, I64, I64, F, P, I64, P, I64]
    lib.orc_quantize_128x1.argtypes = [P, I64, I64, I64, F, P, I64, P, I64]
    lib.orc_quantize_128x128.argtypes = [P, I64, I64, I64, F, P, I64, P, I64, P]
    lib.orc_requant_128x1.argtypes = [P, I64, I64, I64, P, I64, P, I64, P, I64]
    lib.orc_e8m0_decode.restype = ctypes.c_double
    lib.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.orc_quantize_1x128_ue8m0.argtypes = [P, I64, I64, I64, F, P, I64, P, I64]
    lib.orc_quantize_128x1_ue8m0.argtypes = [P, I64, I64, I64, F, P, I64, P, I64]
    lib.orc_quantize_128x128_ue8m0.argtypes = [P, I64, I64, I64, F, P, I64, P, I64, P]
    lib.orc_requant_128x1_ue8m0.argtypes = [P, I64, I64, I64, P, I64, P, I64, P, I64]
    lib.orc_requant_128x128_ue8m0.argtypes = [P, I64, I64, I64, P, F, P, I64, P, I64, P]
    lib.orc_gemm_block_scaled.argtypes = [I64, P, I64, P, I64, I64, I64,
                                          P, I64, P, I64, I64, I64,
                                          P, I64, P, I64, P, P]
    lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
    lib.orc_e4m3_encode_bits_range.argtypes = [ctypes.c_uint32, I64, P]
    lib.orc_e4m3_decode_array.argtypes = [P, I64, P]
    lib.orc_bf16_round_array.argtypes = [P, I64, P]
    U64, U32 = ctypes.c_uint64, ctypes.c_uint32
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_sr_word.restype = ctypes.c_uint32
    lib.orc_sr_word.argtypes = [U64, U32, I64, I64]
    lib.orc_e4m3_encode_sr.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_sr.argtypes = [F, U32]
    lib.orc_e4m3_encode_sr_array.argtypes = [P, P, I64, P]
    lib.orc_sr_words.argtypes = [U64, U32, I64, I64, I64, I64, P]
    lib.orc_quantize_1x128_sr.argtypes = [P, I64, I64, I64, F, P, I64, P, I64, U64, U32]
    lib.orc_quantize_128x1_sr.argtypes = [P, I64, I64, I64, F, P, I64, P, I64, U64, U32]
    lib.orc_quantize_128x128_sr.argtypes = [P, I64, I64, I64, F, P, I64, P, I64, P, U64, U32]
    lib.orc_swiglu_h.argtypes = [P, I64, I64, I64, P, I64]
    lib.orc_swiglu_dgu.argtypes = [P, I64, I64, I64, P, I64, P, I64, P, I64]
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops from now on (timing only)."""
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().orc_e4m3_decode_array(_ptr(codes), codes.size, _ptr(out))
    return out


def e4m3_encode(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(f), f.size, _ptr(out))
    return out


def e4m3_encode_bits_range(start: int, n: int) -> np.ndarray:
    """Encode the fp32 values with bit patterns start .. start+n-1."""
    out = np.empty(n, np.uint8)
    _load().orc_e4m3_encode_bits_range(ctypes.c_uint32(start), n, _ptr(out))
    return out


def bf16_round(r) -> np.ndarray:
    """Round float64 values to bfloat16 (RNE, one rounding); returns uint16 bits."""
    r = _c(r, np.float64)
    out = np.empty(r.shape, np.uint16)
    _load().orc_bf16_round_array(_ptr(r), r.size, _ptr(out))
    return out


def bf16_to_float(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def quantize_1x128(x_bits, amax_floor: float = 0.0):
    """x_bits: bf16 bit patterns [R, C].  Returns (q [R, C] uint8, s [ceil(C/128), R] float32)."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty((_cdiv(C, TILE), R), np.float32)
    _load().orc_quantize_1x128(_ptr(x), R, C, C, ctypes.c_float(amax_floor),
                               _ptr(q), C, _ptr(s), R)
    return q, s


def quantize_128x1(x_bits, amax_floor: float = 0.0):
    """x_bits [R, C] -> (qT [C, roundup(R,128)] uint8 zero-padded, sT [ceil(R/128), C] float32)."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    Rp = _cdiv(R, TILE) * TILE
    qT = np.empty((C, Rp), np.uint8)
    sT = np.empty((_cdiv(R, TILE), C), np.float32)
    _load().orc_quantize_128x1(_ptr(x), R, C, C, ctypes.c_float(amax_floor),
                               _ptr(qT), Rp, _ptr(sT), C)
    return qT, sT


def quantize_128x128(w_bits, amax_floor: float = 0.0):
    """w_bits [K, N] -> (q [K, N], qT [N, K], s [ceil(K/128), ceil(N/128)] float32)."""
    w = _c(w_bits, np.uint16)
    K, N = w.shape
    q = np.empty((K, N), np.uint8)
    qT = np.empty((N, K), np.uint8)
    s = np.empty((_cdiv(K, TILE), _cdiv(N, TILE)), np.float32)
    _load().orc_quantize_128x128(_ptr(w), K, N, N, ctypes.c_float(amax_floor),
                                 _ptr(q), N, _ptr(qT), K, _ptr(s))
    return q, qT, s


def requant_128x1(q, s):
    """1x128 codes q [R, C] with scales s [ceil(C/128), R] -> (qT [C, roundup(R,128)], sT [ceil(R/128), C])."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    R, C = q.shape
    assert s.shape == (_cdiv(C, TILE), R)
    Rp = _cdiv(R, TILE) * TILE
    qT = np.empty((C, Rp), np.uint8)
    sT = np.empty((_cdiv(R, TILE), C), np.float32)
    _load().orc_requant_128x1(_ptr(q), R, C, C, _ptr(s), R, _ptr(qT), Rp, _ptr(sT), C)
    return qT, sT


# --------------------------------------------------------------------------
# Power-of-two (UE8M0) scales: the same tilings, each scale 2^e stored as the
# E8M0 byte e + 127, e the smallest integer with 448 * 2^e >= absmax
# (prime-rl PR #4073 "Results": power-of-two scales; rounding up is a reading).
# --------------------------------------------------------------------------

def e8m0_decode(e) -> np.ndarray:
    """E8M0 bytes -> float64 scales 2^(byte - 127) (0xFF -> NaN)."""
    e = np.asarray(e, np.uint8)
    lib = _load()
    table = np.array([lib.orc_e8m0_decode(u) for u in range(256)])
    return table[e]


def quantize_1x128_ue8m0(x_bits, amax_floor: float = 0.0):
    """bf16 bits [R, C] -> (q [R, C] uint8, e [ceil(C/128), R] uint8)."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    e = np.empty((_cdiv(C, TILE), R), np.uint8)
    _load().orc_quantize_1x128_ue8m0(_ptr(x), R, C, C, amax_floor, _ptr(q), C, _ptr(e), R)
    return q, e


def quantize_128x1_ue8m0(x_bits, amax_floor: float = 0.0):
    """bf16 bits [R, C] -> (qT [C, roundup(R,128)] zero padded, eT [ceil(R/128), C])."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    Rp = _cdiv(R, TILE) * TILE
    qT = np.empty((C, Rp), np.uint8)
    eT = np.empty((_cdiv(R, TILE), C), np.uint8)
    _load().orc_quantize_128x1_ue8m0(_ptr(x), R, C, C, amax_floor, _ptr(qT), Rp, _ptr(eT), C)
    return qT, eT


def quantize_128x128_ue8m0(w_bits, amax_floor: float = 0.0):
    """bf16 bits [K, N] -> (q [K, N], qT [N, K], e [ceil(K/128), ceil(N/128)])."""
    w = _c(w_bits, np.uint16)
    K, N = w.shape
    q = np.empty((K, N), np.uint8)
    qT = np.empty((N, K), np.uint8)
    e = np.empty((_cdiv(K, TILE), _cdiv(N, TILE)), np.uint8)
    _load().orc_quantize_128x128_ue8m0(_ptr(w), K, N, N, amax_floor, _ptr(q), N, _ptr(qT), K, _ptr(e))
    return q, qT, e


def requant_128x1_ue8m0(q, e):
    """UE8M0 1x128 codes q [R, C] with bytes e [ceil(C/128), R] -> (qT, eT) as quantize_128x1_ue8m0."""
    q = _c(q, np.uint8)
    e = _c(e, np.uint8)
    R, C = q.shape
    assert e.shape == (_cdiv(C, TILE), R)
    Rp = _cdiv(R, TILE) * TILE
    qT = np.empty((C, Rp), np.uint8)
    eT = np.empty((_cdiv(R, TILE), C), np.uint8)
    _load().orc_requant_128x1_ue8m0(_ptr(q), R, C, C, _ptr(e), R, _ptr(qT), Rp, _ptr(eT), C)
    return qT, eT


def requant_128x128_ue8m0(q, s, amax_floor: float = 0.0):
    """Second stage of the two-stage weight cast: 128x128 E4M3 codes q [K, N]
    with fp32 tile scales s [ceil(K/128), ceil(N/128)] (as quantize_128x128
    returns them) -> (q2 [K, N], q2T [N, K], e [ceil(K/128), ceil(N/128)]):
    v = fl32(dec(q) * s), then the UE8M0 128x128 rule on v."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    K, N = q.shape
    assert s.shape == (_cdiv(K, TILE), _cdiv(N, TILE))
    q2 = np.empty((K, N), np.uint8)
    q2T = np.empty((N, K), np.uint8)
    e = np.empty((_cdiv(K, TILE), _cdiv(N, TILE)), np.uint8)
    _load().orc_requant_128x128_ue8m0(_ptr(q), K, N, N, _ptr(s), amax_floor, _ptr(q2), N, _ptr(q2T), K, _ptr(e))
    return q2, q2T, e


# --------------------------------------------------------------------------
# Stochastic rounding: the same tile scales, the cast picks the lower or upper
# E4M3 magnitude neighbour with a Philox4x32-10 word per element (prime-rl
# PR #4073 conventions row "SR agreement": stateless seed/salt/counter, Philox,
# lower/upper-magnitude rule; the word layout is a reading, see fgb_oracle.c).
# --------------------------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    """One Philox4x32-10 block: ctr 4 x uint32, key 2 x uint32 -> 4 x uint32."""
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.empty(4, np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_words(seed: int, salt: int, r0: int, R: int, c0: int, C: int) -> np.ndarray:
    """The random words of elements (r0..r0+R-1) x (c0..c0+C-1) -> uint32 [R, C]."""
    out = np.empty((R, C), np.uint32)
    _load().orc_sr_words(seed, salt, r0, R, c0, C, _ptr(out))
    return out


def e4m3_encode_sr(v, u) -> np.ndarray:
    """SR codes of fp32 values v with 32-bit words u (same shape)."""
    v = _c(v, np.float32)
    u = _c(u, np.uint32)
    assert v.shape == u.shape
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_encode_sr_array(_ptr(v), _ptr(u), v.size, _ptr(out))
    return out


def quantize_1x128_sr(x_bits, seed: int, salt: int, amax_floor: float = 0.0):
    """As quantize_1x128 with the SR cast."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty((_cdiv(C, TILE), R), np.float32)
    _load().orc_quantize_1x128_sr(_ptr(x), R, C, C, ctypes.c_float(amax_floor), _ptr(q), C, _ptr(s), R,
                                  seed, salt)
    return q, s


def quantize_128x1_sr(x_bits, seed: int, salt: int, amax_floor: float = 0.0):
    """As quantize_128x1 with the SR cast (element (r, c) of x draws word (r, c))."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    Rp = _cdiv(R, TILE) * TILE
    qT = np.empty((C, Rp), np.uint8)
    sT = np.empty((_cdiv(R, TILE), C), np.float32)
    _load().orc_quantize_128x1_sr(_ptr(x), R, C, C, ctypes.c_float(amax_floor), _ptr(qT), Rp, _ptr(sT), C,
                                  seed, salt)
    return qT, sT


def quantize_128x128_sr(w_bits, seed: int, salt: int, amax_floor: float = 0.0):
    """As quantize_128x128 with the SR cast (q and qT hold the same codes)."""
    w = _c(w_bits, np.uint16)
    K, N = w.shape
    q = np.empty((K, N), np.uint8)
    qT = np.empty((N, K), np.uint8)
    s = np.empty((_cdiv(K, TILE), _cdiv(N, TILE)), np.float32)
    _load().orc_quantize_128x128_sr(_ptr(w), K, N, N, ctypes.c_float(amax_floor), _ptr(q), N, _ptr(qT), K,
                                    _ptr(s), seed, salt)
    return q, qT, s


# --------------------------------------------------------------------------
# SwiGLU with its casts fused ("scratch" page, section "What is asserted, and
# from where": the SwiGLU input saved as E4M3, the forward emitting the next
# GEMM's E4M3 operand, the backward emitting both tile orientations and
# computing in BF16 from the dequantized input).  [G | U] is one [R, 2F]
# tensor; the exact values are rounded once to BF16 (see fgb_oracle.c).
# --------------------------------------------------------------------------

def swiglu_h(gu_bits):
    """H = bf16(silu(G) * U) for GU [R, 2F] bf16 bits -> bf16 bits [R, F]."""
    gu = _c(gu_bits, np.uint16)
    R, F2 = gu.shape
    assert F2 % 2 == 0
    F = F2 // 2
    h = np.empty((R, F), np.uint16)
    _load().orc_swiglu_h(_ptr(gu), R, F, F2, _ptr(h), F)
    return h


def swiglu_dgu(q_gu, s_gu, dh_bits):
    """[dG | dU] bf16 bits [R, 2F] from the 1x128 stash (q_gu [R, 2F], s_gu
    [2F/128, R]) and dH [R, F] bf16 bits."""
    q = _c(q_gu, np.uint8)
    s = _c(s_gu, np.float32)
    dh = _c(dh_bits, np.uint16)
    R, F2 = q.shape
    F = F2 // 2
    assert dh.shape == (R, F) and s.shape == (_cdiv(F2, TILE), R)
    out = np.empty((R, F2), np.uint16)
    _load().orc_swiglu_dgu(_ptr(q), R, F, F2, _ptr(s), R, _ptr(dh), F, _ptr(out), F2)
    return out


def swiglu_fwd_quant(gu_bits, amax_floor: float = 0.0):
    """The fused forward: (q_gu, s_gu) = 1x128 stash of [G | U]; (q_h, s_h) = 1x128
    of H; h = H's bf16 bits."""
    q_gu, s_gu = quantize_1x128(gu_bits, amax_floor)
    h = swiglu_h(gu_bits)
    q_h, s_h = quantize_1x128(h, amax_floor)
    return q_gu, s_gu, q_h, s_h, h


def swiglu_bwd_quant(q_gu, s_gu, dh_bits, amax_floor: float = 0.0):
    """The fused backward: dgu = [dG | dU] bf16 bits, then both tile orientations
    (q, s) = 1x128 and (qT, sT) = 128x1 of it."""
    dgu = swiglu_dgu(q_gu, s_gu, dh_bits)
    q, s = quantize_1x128(dgu, amax_floor)
    qT, sT = quantize_128x1(dgu, amax_floor)
    return dgu, q, s, qT, sT


# --------------------------------------------------------------------------
# Block-scaled GEMMs
# --------------------------------------------------------------------------

def _sel(idx, n):
    if idx is None:
        return np.arange(n, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.ndim == 1 and (idx.size == 0 or (idx.min() >= 0 and idx.max() < n))
    return idx


def _gemm(Kc, A, sa, sa_sb, sa_si, sa_group, B, sb, sb_sb, sb_sj, sb_group, rows, cols):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[0])
    out = np.empty((rows.size, cols.size), np.float64)
    aabs = np.empty((rows.size, cols.size), np.float64)
    if rows.size and cols.size:
        _load().orc_gemm_block_scaled(Kc, _ptr(A), A.shape[1], _ptr(sa), sa_sb, sa_si, sa_group,
                                      _ptr(B), B.shape[1], _ptr(sb), sb_sb, sb_sj, sb_group,
                                      _ptr(rows), rows.size, _ptr(cols), cols.size,
                                      _ptr(out), _ptr(aabs))
    return out, aabs


def gemm_fprop(qx, sx, qwT, sw, rows=None, cols=None):
    """Y = X W.  qx [M, K] (1x128 scales sx [K/128, M]); qwT [N, K] (W's codes
    transposed, 128x128 scales sw [K/128, N/128]).  Returns (r [m, n], aabs)."""
    M, K = qx.shape
    N = qwT.shape[0]
    assert qwT.shape[1] == K and K % TILE == 0 and N % TILE == 0
    assert sx.shape == (K // TILE, M) and sw.shape == (K // TILE, N // TILE)
    return _gemm(K, qx, sx, M, 1, 1, qwT, sw, N // TILE, 1, TILE, rows, cols)


def gemm_dgrad(qdy, sdy, qw, sw, rows=None, cols=None):
    """dX = dY W^T.  qdy [M, N] (1x128 scales sdy [N/128, M]); qw [K, N] (W's
    codes, scales sw [K/128, N/128]).  Returns (r [m, k], aabs)."""
    M, N = qdy.shape
    K = qw.shape[0]
    assert qw.shape[1] == N and K % TILE == 0 and N % TILE == 0
    assert sdy.shape == (N // TILE, M) and sw.shape == (K // TILE, N // TILE)
    return _gemm(N, qdy, sdy, M, 1, 1, qw, sw, 1, N // TILE, TILE, rows, cols)


def gemm_wgrad(qxT, sxT, qdyT, sdyT, M, rows=None, cols=None):
    """dW = X^T dY in W's [K, N] shape.  qxT [K, Mp], sxT [ceil(M/128), K];
    qdyT [N, Mp], sdyT [ceil(M/128), N]; contraction over the first M of Mp
    columns (the rest is zero padding).  Returns (r [k, n], aabs)."""
    K, Mp = qxT.shape
    N = qdyT.shape[0]
    assert qdyT.shape[1] == Mp and M <= Mp
    nb = _cdiv(M, TILE)
    assert sxT.shape[0] >= nb and sdyT.shape[0] >= nb
    return _gemm(M, qxT, sxT, sxT.shape[1], 1, 1, qdyT, sdyT, sdyT.shape[1], 1, 1, rows, cols)


# --------------------------------------------------------------------------
# Grouped (MoE expert) GEMMs: the dense oracle applied per expert segment
# --------------------------------------------------------------------------

def _segments(offsets):
    offsets = np.asarray(offsets, dtype=np.int64)
    return [(int(offsets[e]), int(offsets[e + 1])) for e in range(offsets.size - 1)]


def gemm_fprop_grouped(offsets, qx, sx, qwT, sw, rows=None, cols=None):
    """Per expert e: Y[o_e:o_{e+1}] = X[o_e:o_{e+1}] W_e.  qwT [E, N, K], sw [E, K/128, N/128].
    Rows outside every segment give r = 0."""
    R, K = qx.shape
    N = qwT.shape[1]
    rows = _sel(rows, R)
    cols = _sel(cols, N)
    out = np.zeros((rows.size, cols.size))
    aabs = np.zeros((rows.size, cols.size))
    for e, (a, b) in enumerate(_segments(offsets)):
        pick = np.nonzero((rows >= a) & (rows < b))[0]
        if pick.size == 0:
            continue
        r, aa = gemm_fprop(qx[a:b], sx[:, a:b], qwT[e], sw[e], rows[pick] - a, cols)
        out[pick] = r
        aabs[pick] = aa
    return out, aabs


def gemm_dgrad_grouped(offsets, qdy, sdy, qw, sw, rows=None, cols=None):
    """Per expert e: dX[o_e:o_{e+1}] = dY[o_e:o_{e+1}] W_e^T.  qw [E, K, N], sw [E, K/128, N/128]."""
    R, N = qdy.shape
    K = qw.shape[1]
    rows = _sel(rows, R)
    cols = _sel(cols, K)
    out = np.zeros((rows.size, cols.size))
    aabs = np.zeros((rows.size, cols.size))
    for e, (a, b) in enumerate(_segments(offsets)):
        pick = np.nonzero((rows >= a) & (rows < b))[0]
        if pick.size == 0:
            continue
        r, aa = gemm_dgrad(qdy[a:b], sdy[:, a:b], qw[e], sw[e], rows[pick] - a, cols)
        out[pick] = r
        aabs[pick] = aa
    return out, aabs


def gemm_wgrad_grouped(offsets, qxT, sxT, qdyT, sdyT, experts=None, rows=None, cols=None):
    """Per expert e: dW_e = X_e^T dY_e over the segment's rows (128-aligned, zero padded).
    qxT [K, R_pad], sxT [R_pad/128, K], qdyT [N, R_pad], sdyT [R_pad/128, N].
    Returns (r [len(experts), k, n], aabs); an empty expert gives zeros."""
    K = qxT.shape[0]
    N = qdyT.shape[0]
    segs = _segments(offsets)
    experts = range(len(segs)) if experts is None else experts
    rows = _sel(rows, K)
    cols = _sel(cols, N)
    out = np.zeros((len(experts), rows.size, cols.size))
    aabs = np.zeros_like(out)
    for i, e in enumerate(experts):
        a, b = segs[e]
        if b == a:
            continue
        assert a % TILE == 0 and b % TILE == 0
        r, aa = gemm_wgrad(qxT[:, a:b], sxT[a // TILE:b // TILE], qdyT[:, a:b],
                           sdyT[a // TILE:b // TILE], b - a, rows, cols)
        out[i] = r
        aabs[i] = aa
    return out, aabs
