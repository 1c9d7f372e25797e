// Device helpers shared by the quantization and GEMM kernels of libfgb (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgb {

constexpr int kTile = 128;          // quantization tile / GEMM contraction block
constexpr float kE4M3Max = 448.0f;  // largest finite OCP E4M3FN value

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite or +-inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 values rounded to nearest even bf16 by the hardware converter
// (v_cvt_pk_bf16_f32), a in the low half: one instruction where the integer
// form above takes three per value.  Equal to it for every non-NaN input.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_hw v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// ---------------------------------------------------------------------------
// E4M3FN codec on the hardware converters.
// v_cvt_pk_fp8_f32 rounds to nearest even; the operands are clamped to +-448
// first, which is the saturating rule for every finite input.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max); }

// Four fp32 values -> four E4M3 codes, byte i of the result = code of value i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
}

// The same without the clamp, for values known to be finite with |v| at most
// 448 up to the rounding of a cast multiplier (x * fl32(448/a) for |x| <= a).
// The converter rounds to nearest even within the format and gives the NaN
// code only past 464, the midpoint above 448 (measured on gfx950 for every
// fp32 value in [440, 500) and its negation: all equal the saturating
// conversion up to 464).
__device__ __forceinline__ uint32_t e4m3x4_inrange(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
// FIX: the general cast (clamp, then the fix-ups of fix_codes by the caller);
// otherwise the in-range cast for finite nonzero multipliers.
template <bool FIX>
__device__ __forceinline__ uint32_t e4m3x4_t(float a, float b, float c, float d) {
    if constexpr (FIX) return e4m3x4(a, b, c, d);
    else return e4m3x4_inrange(a, b, c, d);
}

// Codes in byte 0,1 (HI = false) or byte 2,3 (HI = true) of w -> two fp32 values (exact).
template <bool HI>
__device__ __forceinline__ float2 e4m3x2_decode(uint32_t w) {
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    return make_float2(v[0], v[1]);
}

// ---------------------------------------------------------------------------
// Tile scale and inverse from the absmax a (>= 0, finite or +inf):
//   s = fl32(a / 448), inv = a == 0 ? 0 : min(fl32(448 / a), FLT_MAX).
// Both are IEEE divisions (HIP's default correctly rounded fp32 divide).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_scale(float a, float& s, float& inv) {
    if (a != a) {                   // a NaN in the tile: NaN scale and multiplier
        s = inv = __uint_as_float(0x7FC00000u);
        return;
    }
    s = a / kE4M3Max;
    inv = (a == 0.0f) ? 0.0f : fminf(kE4M3Max / a, 3.40282346638528859812e+38f);
}

// ---------------------------------------------------------------------------
// NaN tiles.  The absmax is an integer max over magnitude bits, and a NaN's
// bits exceed +inf's, so one NaN element makes the tile's absmax NaN; the
// floor (>= 0, finite) is applied the same way so that it cannot drop it.  A
// NaN tile gets a NaN scale (the canonical quiet NaN; E8M0 byte 0xFF for
// power-of-two scales) and the E4M3 NaN code 0x7F for every element, so the
// NaN reaches every GEMM output the tile feeds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float floored_absmax(uint32_t abs_bits, float amax_floor) {
    return __uint_as_float(max(abs_bits, __float_as_uint(amax_floor)));
}
// A tile whose multiplier is 0 (an all-zero tile, or an infinite absmax: 448/Inf)
// casts Inf * 0 = NaN for its infinite elements; the clamp to +-448 before the
// cast would turn that NaN into -448, so such products get the NaN code 0x7F.
__device__ __forceinline__ uint32_t nan_products(uint32_t codes, float p0, float p1, float p2, float p3) {
    const uint32_t nan = (p0 != p0 ? 0x000000FFu : 0u) | (p1 != p1 ? 0x0000FF00u : 0u) |
                         (p2 != p2 ? 0x00FF0000u : 0u) | (p3 != p3 ? 0xFF000000u : 0u);
    return (codes & ~nan) | (0x7F7F7F7Fu & nan);
}
// Four codes of one tile with cast multiplier `mul` and products p_i = x_i * mul:
// a NaN tile gives 0x7F in every byte, a zero multiplier the NaN code for NaN
// products; otherwise the codes are returned unchanged.  Both cases are rare
// and branch around the common path.
__device__ __forceinline__ uint32_t fix_codes(uint32_t codes, float mul, float p0, float p1, float p2, float p3) {
    if (__builtin_expect(mul != mul, 0)) return 0x7F7F7F7Fu;
    if (__builtin_expect(mul == 0.0f, 0)) return nan_products(codes, p0, p1, p2, p3);
    return codes;
}
// A cast multiplier that needs no fix-up of its codes: finite and nonzero (the
// common case, where no product can be NaN).  Callers test it once for all the
// multipliers a thread uses and branch to a path without fix_codes.
__device__ __forceinline__ bool plain_mul(float m) { return m == m && m != 0.0f; }
// For power-of-two scales the multiplier 2^-e stays finite and nonzero even for
// an infinite tile (e clamps at 127, reached only by an infinite absmax): such
// a tile's products are infinite and need the clamp, so 2^-127 is not plain.
template <bool PO2>
__device__ __forceinline__ bool plain_mul_t(float m) {
    if constexpr (PO2) return plain_mul(m) && m > 0x1p-127f;
    else return plain_mul(m);
}
template <bool FIX>
__device__ __forceinline__ uint32_t fix_codes_if(uint32_t codes, float mul, float p0, float p1, float p2, float p3) {
    if constexpr (FIX) return fix_codes(codes, mul, p0, p1, p2, p3);
    else return codes;
}
// The same for four codes of four different tiles (byte i: multiplier m_i, product p_i).
__device__ __forceinline__ uint32_t fix_codes4(uint32_t codes, float m0, float m1, float m2, float m3,
                                               float p0, float p1, float p2, float p3) {
    const uint32_t tile = (m0 != m0 ? 0x000000FFu : 0u) | (m1 != m1 ? 0x0000FF00u : 0u) |
                          (m2 != m2 ? 0x00FF0000u : 0u) | (m3 != m3 ? 0xFF000000u : 0u);
    codes = nan_products(codes, p0, p1, p2, p3);
    return (codes & ~tile) | (0x7F7F7F7Fu & tile);
}
// Byte mask of the valid rows among 8 consecutive rows of which `nv` exist
// (lo: rows 0..3, hi: rows 4..7): padding rows of transposed codes stay 0x00.
__device__ __forceinline__ uint32_t rows_mask_lo(int nv) {
    return nv >= 4 ? 0xFFFFFFFFu : (nv <= 0 ? 0u : (1u << (8 * nv)) - 1u);
}
__device__ __forceinline__ uint32_t rows_mask_hi(int nv) {
    return nv >= 8 ? 0xFFFFFFFFu : (nv <= 4 ? 0u : (1u << (8 * (nv - 4))) - 1u);
}

// ---------------------------------------------------------------------------
// Power-of-two (UE8M0) tile scale from the absmax a (>= 0): e is the smallest
// integer with 448 * 2^e >= a, clamped to [-127, 127] (zero and fp32-subnormal
// absmaxes give -127, +inf gives 127); byte = e + 127 is its E8M0 encoding and
// mul = 2^-e (exact).  NaN gives the E8M0 NaN byte 0xFF and mul = NaN.
// With a = (1 + m/2^23) 2^(E-127) and 448 = 1.75 * 2^8: e = E - 135 when the
// significand is at most 1.75 (m <= 0x600000), else E - 134.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_scale_ue8m0(float a, uint32_t& byte, float& mul) {
    const uint32_t u = __float_as_uint(a);
    const int E = (int)(u >> 23);
    const uint32_t m = u & 0x7FFFFFu;
    if (E == 255 && m != 0) {
        byte = 0xFFu;
        mul = __uint_as_float(0x7FC00000u);
        return;
    }
    int e = (E == 0) ? -127 : (E == 255 ? 127 : (m <= 0x600000u ? E - 135 : E - 134));
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    byte = (uint32_t)(e + 127);
    mul = e <= 126 ? __uint_as_float((uint32_t)(127 - e) << 23) : __uint_as_float(0x00400000u);
}

// E8M0 byte -> 2^(byte - 127) as fp32 (byte 0 is the subnormal 2^-127; 0xFF is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
    return byte == 0xFFu ? __uint_as_float(0x7FC00000u)
         : (byte == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(byte << 23));
}

// ---------------------------------------------------------------------------
// Stochastic rounding (prime-rl PR #4073, conventions row "SR agreement": a
// stateless seed / salt / counter Philox word per element, and the lower- or
// upper-magnitude E4M3 neighbour).
//
// philox4x32_10: the Philox4x32 generator with 10 rounds (Salmon, Moraes,
// Dror, Shaw, SC'11).  Element (r, c) of the tensor being quantized takes
// word c % 4 of the block at counter (c / 4, r, salt, 0), key (seed low,
// seed high); the key is wave-uniform.
// ---------------------------------------------------------------------------
struct SrArgs {
    uint32_t k0 = 0, k1 = 0;      // seed, low and high 32 bits
    uint32_t salt = 0;
};

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// Words of the 8 consecutive elements (r, c .. c+7), c a multiple of 8.
__device__ __forceinline__ void sr_words8(const SrArgs& a, int64_t r, int64_t c, uint32_t (&u)[8]) {
    uint32_t w0[4], w1[4];
    philox4x32_10((uint32_t)(c >> 2), (uint32_t)r, a.salt, 0u, a.k0, a.k1, w0);
    philox4x32_10((uint32_t)(c >> 2) + 1u, (uint32_t)r, a.salt, 0u, a.k0, a.k1, w1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { u[i] = w0[i]; u[4 + i] = w1[i]; }
}

// The E4M3 value that stochastic rounding of v with word u selects (an exact
// grid value, sign kept, |v| >= 448 -> 448; NaN passes through): with m = |v|,
// lo/hi its lower/upper grid neighbours, hi when u < (m - lo)/(hi - lo) * 2^32.
//   m >= 2^-6 (E4M3 normals): the grid keeps 3 of the 23 fp32 mantissa bits;
//     (m - lo)/(hi - lo) = D / 2^20 for D the 20 dropped bits, so hi iff
//     (u >> 12) < D, and hi = lo + one unit of the kept mantissa (IEEE carry).
//   m < 2^-6: spacing 2^-9; t = 512 m is exact, frac = t - floor(t) exact,
//     frac * 2^32 exact, and u < frac * 2^32 iff u < ceil(frac * 2^32); frac
//     has at most 24 significant bits, so ceil(frac * 2^32) <= 2^32 - 2^8 fits
//     in 32 bits.
__device__ __forceinline__ float e4m3_sr_value(float v, uint32_t u) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t mb = b & 0x7FFFFFFFu;
    if (mb > 0x7F800000u) return v;                       // NaN
    if (mb >= 0x43E00000u) return __uint_as_float((b & 0x80000000u) | 0x43E00000u);   // >= 448
    float mag;
    if (mb >= 0x3C800000u) {                              // >= 2^-6
        const uint32_t d = mb & 0xFFFFFu;
        const uint32_t up = (u >> 12) < d ? 1u : 0u;
        mag = __uint_as_float((mb & ~0xFFFFFu) + (up << 20));
    } else {
        const float t = __uint_as_float(mb) * 512.0f;
        const float fl = floorf(t);
        const float thr = (t - fl) * 4294967296.0f;
        const uint32_t tc = (uint32_t)ceilf(thr);
        const float up = u < tc ? 1.0f : 0.0f;
        mag = (fl + up) * 0.001953125f;                   // (fl + up) * 2^-9, exact
    }
    return __uint_as_float(__float_as_uint(mag) | (b & 0x80000000u));
}

// Four SR codes (byte i = code of value i).
__device__ __forceinline__ uint32_t e4m3x4_sr(float a, float b, float c, float d,
                                              uint32_t ua, uint32_t ub, uint32_t uc, uint32_t ud) {
    return e4m3x4(e4m3_sr_value(a, ua), e4m3_sr_value(b, ub), e4m3_sr_value(c, uc), e4m3_sr_value(d, ud));
}

// ---------------------------------------------------------------------------
// Cross-lane unsigned max.  DPP within a row of 16 lanes, then swizzles.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max over each aligned group of 16 lanes (every lane of the group gets it)
__device__ __forceinline__ uint32_t max16(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
    v = max(v, dpp_u32<0x140>(v));  // row_mirror
    return v;
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) {
    return (uint32_t)__shfl_xor((int)v, m, 64);
}

// ---------------------------------------------------------------------------
// Vector global memory access
// ---------------------------------------------------------------------------
// Blocks of a grid of nrb row blocks x ncb column blocks, launched as one
// dimension.  cols_fast: the column blocks vary fastest, so the blocks resident
// together cover whole rows of the tensor, whose bytes spread over every HBM
// channel; ordered row blocks first, they read one column band of many rows, at
// addresses that repeat with the row pitch -- for a pitch that is a multiple of
// 8 KB on a few channels only (MoE weight cast, pitch 8 KB: 11% faster cold;
// 1x128 cast 5-7%).  With the row blocks fastest, consecutive blocks extend the
// same transposed output rows, which kernels with a transposed output prefer
// at other pitches (128x128 cast at a 14 KB pitch 5% faster cold; the 128x1
// cast and the requant 7-8% faster).
struct BlockRC { int64_t r, c; };
__device__ __forceinline__ BlockRC block_rc(bool cols_fast, int64_t nrb, int64_t ncb) {
    const uint32_t b = blockIdx.x;
    if (cols_fast) return {(int64_t)(b / (uint32_t)ncb), (int64_t)(b % (uint32_t)ncb)};
    return {(int64_t)(b % (uint32_t)nrb), (int64_t)(b / (uint32_t)nrb)};
}
// The one-dimensional grid for nrb x ncb blocks; 0 when it exceeds the launch limit.
inline unsigned grid_rc(int64_t nrb, int64_t ncb) {
    const int64_t n = nrb * ncb;
    return (nrb > 0 && ncb > 0 && n <= 0x7FFFFFFF) ? (unsigned)n : 0u;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Non-temporal 16-byte load, for an input read once: its lines are not kept in
// L2 / the MALL, which stay with the outputs that the next kernel reads.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    return make_uint4(__builtin_nontemporal_load(&q->x), __builtin_nontemporal_load(&q->y),
                      __builtin_nontemporal_load(&q->z), __builtin_nontemporal_load(&q->w));
}
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
// Non-temporal 16-byte store, for a large output that no later part of the
// same kernel reads: its lines are not kept in L2 / the MALL, where they would
// evict the operand lines that the kernel's remaining tiles re-read.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_stream(void* p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace fgb
