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
    s = a / kE4M3Max;
    inv = (a == 0.0f) ? 0.0f : fminf(kE4M3Max / a, 3.40282346638528859812e+38f);
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
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

}  // namespace fgb
