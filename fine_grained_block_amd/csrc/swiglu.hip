// SwiGLU with its E4M3 casts fused into the producer kernels, for gfx950.
//
// "scratch: the backward pass, unrolled", section "What is asserted, and from
// where": the SwiGLU input is saved as E4M3; a cast rides the nearest vector
// kernel, so the SwiGLU forward emits the down projection's E4M3 operand and
// the SwiGLU backward emits the gate/up projection's dgrad and wgrad operands
// in both tile orientations; the backward computes in BF16 from the
// dequantized E4M3 input.
//
// The gate/up output is one tensor [G | U] of shape [R][2F] (G = columns
// 0..F-1, U = F..2F-1).  Values:
//   forward   H  = bf16(silu(G) * U)                          (one rounding of the exact value)
//   backward  G~ = bf16(fl32(dec(q_g) * s_g)), U~ likewise     (dequantize, then the BF16 dtype)
//             dG = bf16(dH * U~ * silu'(G~)), dU = bf16(dH * silu(G~))
// and the casts are the 1x128 / 128x1 tile quantizers of quant.hip applied to
// [G | U] (the stash), H, and [dG | dU].
//
// Exact rounding.  Each value is first formed in fp32 (expf, IEEE division).
// Its relative error is a few fp32 ulps (the expf error plus four roundings;
// for silu' the cancellation in 1 + g (1 - sigma) is carried in a per-element
// bound).  When the fp32 value lies farther than that bound from every bf16
// rounding midpoint, its bf16 rounding is the exact value's.  Otherwise, and
// for |g| > 80, the value is recomputed in fp64, where an exact product on a
// midpoint (g*u/2 for tiny g, g*u or f for a saturated sigmoid) is moved off
// it by the sign of the exact correction.

#include "device_common.hpp"
#include "fgb_internal.hpp"

namespace fgb {

namespace {

// One RNE rounding of a finite double (|v| < 2^128) to bf16 bits: round to
// fp32 with round-to-odd (truncate, set the last bit when inexact), then RNE
// to bf16 -- round-to-odd with >= 2 extra bits makes the second rounding exact.
__device__ uint32_t bf16_rne_f64(double v) {
    float f = (float)v;
    const double back = (double)f;
    if (back != v) {
        uint32_t b = __float_as_uint(f);
        if (fabs(back) > fabs(v)) b -= 1u;          // the magnitude was rounded up: step back
        f = __uint_as_float(b | 1u);
    }
    return f32_to_bf16_rne(f) & 0xFFFFu;
}

// bf16 bits of the exact hi * (1 + c): hi has at most 17 significant bits,
// |c| <= 2^-10 with sign c_sign (0: c is exactly 0; c may underflow to 0 for
// a huge gate).  A 17-bit value that is not a bf16 midpoint lies >= 2^-17 |hi|
// from every midpoint, so below |c| = 2^-36 the correction only breaks a tie;
// above it hi + hi*c keeps the correction in fp64 (17 + 36 = 53 bits).
__device__ uint32_t bf16_scaled_f64(double hi, double c, int c_sign) {
    // a zero product keeps its sign (hi * (1 + c), 1 + c > 0); hi + hi*c would
    // turn -0 into +0 where hi*c is +0
    if (hi == 0.0) return bf16_rne_f64(hi);
    if (fabs(c) >= 0x1p-36) return bf16_rne_f64(hi + hi * c);
    if (c_sign == 0) return bf16_rne_f64(hi);
    int ex;
    frexp(fabs(hi), &ex);
    ex -= 1;                                        // |hi| in [2^ex, 2^(ex+1))
    if (ex < -126) ex = -126;                       // bf16 subnormal quantum 2^-133
    const double q = ldexp(fabs(hi), 7 - ex);       // exact
    const double fl = floor(q);
    if (q - fl != 0.5) return bf16_rne_f64(hi);
    const double m = c_sign > 0 ? fl + 1.0 : fl;    // the tie goes the correction's way
    const float r = (float)ldexp(m, ex - 7);        // exact
    return (__float_as_uint(r) >> 16) | (signbit(hi) ? 0x8000u : 0u);
}

// sigma(g) and 1 - sigma(g) in fp64, each without cancellation.
__device__ void sigma_f64(double g, double& sig, double& om) {
    if (g >= 0.0) {
        const double e = exp(-g);
        sig = 1.0 / (1.0 + e);
        om = e / (1.0 + e);
    } else {
        const double e = exp(g);
        sig = e / (1.0 + e);
        om = 1.0 / (1.0 + e);
    }
}

// bf16(silu(g) * f) in fp64 (f exact: a bf16 value).
//   silu(g) = (g/2)(1 + tanh(g/2)), split off for |g| < 2^-10;
//           = g (1 - (1 - sigma)), split off where 1 - sigma < 2^-10.
__device__ __noinline__ uint32_t silu_times_f64(float gf, float ff) {
    const double g = gf, f = ff;
    if (fabs(g) < 0x1p-10)
        return bf16_scaled_f64(g * f * 0.5, tanh(0.5 * g), g > 0.0 ? 1 : (g < 0.0 ? -1 : 0));
    double sig, om;
    sigma_f64(g, sig, om);
    if (om < 0x1p-10) return bf16_scaled_f64(g * f, -om, -1);
    return bf16_rne_f64(g * f * sig);
}

// bf16(silu'(g) * d * u) in fp64 (d * u exact there: two bf16 values).
//   silu'(g) = (1/2)(1 + tanh(g/2) + g / (2 cosh^2(g/2))), split off for |g| < 2^-10;
//            = 1 + (1 - sigma)(g sigma - 1), split off where that term is < 2^-10 (g > 2).
__device__ __noinline__ uint32_t dsilu_times_f64(float gf, float df, float uf) {
    const double g = gf, f = (double)df * (double)uf;
    if (fabs(g) < 0x1p-10) {
        const double ch = cosh(0.5 * g);
        return bf16_scaled_f64(f * 0.5, tanh(0.5 * g) + g / (2.0 * ch * ch), g > 0.0 ? 1 : (g < 0.0 ? -1 : 0));
    }
    double sig, om;
    sigma_f64(g, sig, om);
    const double c = om * (g * sig - 1.0);
    if (g > 2.0 && fabs(c) < 0x1p-10) return bf16_scaled_f64(f, c, 1);
    return bf16_rne_f64(f * (sig * (1.0 + g * om)));
}

// Distance, in fp32 ulps, from v to the nearest bf16 rounding midpoint: the
// bits below the bf16 mantissa against 0x8000.
__device__ __forceinline__ float midpoint_distance(float v) {
    const uint32_t low = __float_as_uint(v) & 0xFFFFu;
    return (float)(low > 0x8000u ? low - 0x8000u : 0x8000u - low);
}

// fp32 fast paths.  Errors in units of 2^-23 relative (one fp32 ulp at most):
// expf <= 2 (its documented bound is 1), v_rcp_f32 <= 1, each IEEE add or
// multiply <= 1/2.  A result is accepted when its distance to the nearest bf16
// midpoint, in fp32 ulps of the result (at most 2^24 per unit relative error),
// exceeds twice its error bound; otherwise the fp64 path decides.

// silu(g) * f: e (2) -> 1 + e (2.5) -> rcp (3.5) -> * g (4) -> * f (4.5 units
// = 9 ulps of the result); accepted beyond 24 ulps.
// e = expf(-g) and sig = rcp(1 + e) are passed in, so that silu and silu' of
// one gate share them (for |g| > 80 they are discarded unused).
// The fast paths return the fp32 value and whether its bf16 rounding is
// decided by it; undecided values go to the fp64 forms.
__device__ __forceinline__ float silu_times_fast_v(float g, float f, float sig, bool& ok) {
    const float v = (g * sig) * f;
    ok = fabsf(g) <= 80.0f && midpoint_distance(v) > 24.0f;
    return v;
}

// silu'(g) * d * u = sigma (1 + t) f, t = g e sigma, f = d u (exact in fp32 for
// |f| >= 2^-134: 16 significant bits).  t carries <= 5 units, so 1 + t has an
// absolute error <= 5 |t| + 1/2 units and the result a relative error
// <= 8 (1 + |t| / |1 + t|) units (<= 2^-20 (1 + |t|/|1+t|)); accepted beyond
// twice that in ulps, plus 8.
__device__ __forceinline__ float dsilu_times_fast_v(float g, float d, float u, float e, float sig, bool& ok) {
    const float f = d * u;
    const float t = g * (e * sig);
    const float s1 = 1.0f + t;
    const float v = (sig * s1) * f;
    const float ratio = fabsf(t) * __builtin_amdgcn_rcpf(fabsf(s1)) * 1.0001f;
    const float margin = 2.0f * 0x1p-20f * (1.0f + ratio) * 0x1p24f + 8.0f;
    ok = fabsf(g) <= 80.0f && (f == 0.0f || fabsf(f) >= 0x1p-134f) && ratio < 1024.0f &&
         midpoint_distance(v) > margin;
    return v;
}

// the sigmoid pieces of the fast paths: e = expf(-g), sig = rcp(1 + e)
__device__ __forceinline__ void sigmoid_pieces(float g, float& e, float& sig) {
    e = expf(-g);
    sig = __builtin_amdgcn_rcpf(1.0f + e);
}


__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// E4M3 code -> its value (exact).
__device__ __forceinline__ float e4m3_decode1(uint8_t code) { return e4m3x2_decode<false>((uint32_t)code).x; }

// RN codes of four values times inv (the quantizers' cast); a finite nonzero
// multiplier needs neither the clamp nor the NaN fix-ups.
__device__ __forceinline__ uint32_t codes4(const float* v, float inv) {
    if (__builtin_expect(plain_mul(inv), 1))
        return e4m3x4_inrange(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    return fix_codes(e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv), inv,
                     v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
}

}  // namespace

// ---------------------------------------------------------------------------
// Forward.  A block of 256 threads covers 64 rows and one 128-column tile b of
// H (G tile b, U tile F/128 + b); 16 lanes per row, 8 columns per lane, so a
// row's three 1x128 tiles (G, U, H) each reduce with one DPP max over 16 lanes.
// ---------------------------------------------------------------------------
constexpr int kSwRows = 64;

__global__ __launch_bounds__(256) void k_swiglu_fwd(
    const uint16_t* __restrict__ gu, int64_t R, int64_t F, int64_t ldgu, float amax_floor,
    uint8_t* __restrict__ q_gu, int64_t ldq_gu, float* __restrict__ s_gu, int64_t lds_gu,
    uint8_t* __restrict__ q_h, int64_t ldq_h, float* __restrict__ s_h, int64_t lds_h,
    uint16_t* __restrict__ h_out, int64_t ldh)
{
    const int lane16 = threadIdx.x & 15;
    const int grp = threadIdx.x >> 4;
    const int64_t nb = F / kTile;
    const BlockRC bl = block_rc(true, (R + kSwRows - 1) / kSwRows, nb);
    const int64_t b = bl.c;
    const int64_t c = b * kTile + lane16 * 8;          // column in H and G; U at F + c
    for (int it = 0; it < 4; ++it) {
        const int64_t r = bl.r * kSwRows + grp + 16 * it;
        const bool ok = r < R;
        // [G | U] is read once: non-temporal loads (see ld16_stream)
        const uint4 wg = ok ? ld16_stream(gu + r * ldgu + c) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 wu = ok ? ld16_stream(gu + r * ldgu + F + c) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t g2[4] = {wg.x, wg.y, wg.z, wg.w}, u2[4] = {wu.x, wu.y, wu.z, wu.w};
        float g[8], u[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            g[2 * k] = bf16_lo(g2[k]); g[2 * k + 1] = bf16_hi(g2[k]);
            u[2 * k] = bf16_lo(u2[k]); u[2 * k + 1] = bf16_hi(u2[k]);
        }
        // the stash: 1x128 tiles b (G) and nb + b (U) of [G | U]
        if (q_gu != nullptr) {
            uint32_t mg = 0, mu = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mg = max(mg, __float_as_uint(g[k]) & 0x7FFFFFFFu);
                mu = max(mu, __float_as_uint(u[k]) & 0x7FFFFFFFu);
            }
            mg = max16(mg);
            mu = max16(mu);
            float sg, ig, su, iu;
            tile_scale(floored_absmax(mg, amax_floor), sg, ig);
            tile_scale(floored_absmax(mu, amax_floor), su, iu);
            if (ok) {
                st8(q_gu + r * ldq_gu + c, make_uint2(codes4(g, ig), codes4(g + 4, ig)));
                st8(q_gu + r * ldq_gu + F + c, make_uint2(codes4(u, iu), codes4(u + 4, iu)));
                if (lane16 == 0) {
                    s_gu[b * lds_gu + r] = sg;
                    s_gu[(nb + b) * lds_gu + r] = su;
                }
            }
        }
        // H = bf16(silu(G) U), then its 1x128 tile b
        // (decided values rounded two at a time by the hardware converter -- the
        // same RNE as the integer form for finite values; the others in fp64)
        float vh[8];
        bool okh[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float e, sig;
            sigmoid_pieces(g[k], e, sig);
            vh[k] = silu_times_fast_v(g[k], u[k], sig, okh[k]);
        }
        uint32_t hw[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) hw[k2] = cvt_pk_bf16(vh[2 * k2], vh[2 * k2 + 1]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (!okh[k]) {
                const uint32_t v = silu_times_f64(g[k], u[k]);
                hw[k >> 1] = (k & 1) ? ((hw[k >> 1] & 0xFFFFu) | (v << 16)) : ((hw[k >> 1] & 0xFFFF0000u) | v);
            }
        }
        float hv[8];
        uint32_t mh = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            hv[k] = (k & 1) ? bf16_hi(hw[k >> 1]) : bf16_lo(hw[k >> 1]);
            mh = max(mh, __float_as_uint(hv[k]) & 0x7FFFFFFFu);
        }
        mh = max16(mh);
        float sh, ih;
        tile_scale(floored_absmax(mh, amax_floor), sh, ih);
        if (ok) {
            st8(q_h + r * ldq_h + c, make_uint2(codes4(hv, ih), codes4(hv + 4, ih)));
            if (lane16 == 0) s_h[b * lds_h + r] = sh;
            if (h_out != nullptr)
                st16(h_out + r * ldh + c, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// Backward.  A block of 256 threads covers 128 rows and one 128-column gate
// tile j and produces two output tiles, dG (columns 128j..) and dU
// (F + 128j..).  Phase 1 forms both tiles' bf16 values row by row (thread t:
// rows r0 + 8*(t/16) + i, columns 8*(t%16) ..+8; dG and dU of an element share
// its sigmoid) into two 128 x 128 bf16 tiles in LDS.  Phase 2, once per tile,
// reads back the thread's 8 x 8 patch and quantizes it both ways: 1x128 (row
// maxima: one DPP max per 16-lane row group) and 128x1 (column maxima: lane
// swizzles plus LDS; codes transposed through LDS, over the dG tile once it
// has been read, so every qT store is a 16-byte piece of a 128-byte row).
// Phase 1 keeps only four rows of inputs live, so the fp64 fallback can be a
// call.
// ---------------------------------------------------------------------------
constexpr int kSwTr = 136;   // bytes per staged qT row

__global__ __launch_bounds__(256, 2) void k_swiglu_bwd(
    const uint8_t* __restrict__ q_gu, int64_t R, int64_t F, int64_t ldq_gu,
    const float* __restrict__ s_gu, int64_t lds_gu,
    const uint16_t* __restrict__ dh, int64_t lddh, float amax_floor,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ sT, int64_t ldsT,
    uint16_t* __restrict__ dgu, int64_t lddgu)
{
    __shared__ uint32_t red[4][kTile];
    __shared__ float col_mul[kTile];
    // both output tiles' bf16 values (dG in vt[0], dU in vt[1]); the staged
    // transposed codes reuse vt[0] once its values have been read
    __shared__ __attribute__((aligned(16))) uint16_t vt[2][kTile * kTile];
    uint8_t* const tr = reinterpret_cast<uint8_t*>(&vt[0][0]);
    static_assert(kTile * kSwTr <= (int)sizeof(vt[0]), "staged codes fit one value tile");
    // values the fp32 path leaves undecided: (tile << 14) | (row << 7) | column
    constexpr int kFbMax = 1024;
    __shared__ uint16_t fb_list[kFbMax];
    __shared__ uint32_t fb_count;

    const int t = threadIdx.x;
    const int cg = t & 15, rg = t >> 4, wave = t >> 6;
    const int64_t nb = F / kTile;
    const BlockRC bl = block_rc(true, (R + kTile - 1) / kTile, nb);
    const int64_t r0 = bl.r * kTile;
    const int64_t j = bl.c;
    const int64_t cc = j * kTile + cg * 8;             // gate column; up column F + cc

    // phase 1: G~ = bf16(fl32(dec(q) s)), U~ likewise, dH; both tiles' values
    // from one pass (dG and dU of an element share its sigmoid).  1a: four rows
    // at a time, their raw inputs first, then every value whose fp32 form
    // decides its bf16 rounding; need[h] marks the others (bit 8 i + k).
    uint64_t need[2] = {0, 0};
    if (t == 0) fb_count = 0;
    __syncthreads();                                     // the count is zero before any thread adds to it
#pragma unroll 1
    for (int i0 = 0; i0 < 8; i0 += 4) {
        uint2 cgw[4], cuw[4];
        uint4 dw[4];
        float sg[4], su[4];
        // the thread's first patch row; rows are whole leading dimensions apart
        const int64_t rp = r0 + rg * 8;
        const uint8_t* pq = q_gu + rp * ldq_gu + cc;
        const uint16_t* pd = dh + rp * lddh + cc;
        const float* ps = s_gu + j * lds_gu + rp;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = i0 + ii;
            const bool ok = rp + i < R;
            cgw[ii] = ok ? ld8(pq + i * ldq_gu) : make_uint2(0u, 0u);
            dw[ii] = ok ? ld16(pd + i * lddh) : make_uint4(0u, 0u, 0u, 0u);
            sg[ii] = ok ? ps[i] : 0.0f;
            cuw[ii] = ok ? ld8(pq + i * ldq_gu + F) : make_uint2(0u, 0u);
            su[ii] = ok ? ps[nb * lds_gu + i] : 0.0f;
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = i0 + ii;
            const float2 g0 = e4m3x2_decode<false>(cgw[ii].x), g1 = e4m3x2_decode<true>(cgw[ii].x);
            const float2 g2 = e4m3x2_decode<false>(cgw[ii].y), g3 = e4m3x2_decode<true>(cgw[ii].y);
            const float gd[8] = {g0.x, g0.y, g1.x, g1.y, g2.x, g2.y, g3.x, g3.y};
            const float2 u0 = e4m3x2_decode<false>(cuw[ii].x), u1 = e4m3x2_decode<true>(cuw[ii].x);
            const float2 u2 = e4m3x2_decode<false>(cuw[ii].y), u3 = e4m3x2_decode<true>(cuw[ii].y);
            const float ud[8] = {u0.x, u0.y, u1.x, u1.y, u2.x, u2.y, u3.x, u3.y};
            const uint32_t dd[4] = {dw[ii].x, dw[ii].y, dw[ii].z, dw[ii].w};
            // G~ and U~ of the row's 8 columns, rounded to bf16 two at a time by
            // the hardware converter (finite values: the same RNE as the integer form)
            uint32_t gb[4], ub[4];
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                gb[k2] = cvt_pk_bf16(gd[2 * k2] * sg[ii], gd[2 * k2 + 1] * sg[ii]);
                ub[k2] = cvt_pk_bf16(ud[2 * k2] * su[ii], ud[2 * k2 + 1] * su[ii]);
            }
            uint32_t wg[4], wu[4];
            float vg[8], vu[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float g = (k & 1) ? bf16_hi(gb[k >> 1]) : bf16_lo(gb[k >> 1]);
                const float u = (k & 1) ? bf16_hi(ub[k >> 1]) : bf16_lo(ub[k >> 1]);
                const float d = (k & 1) ? bf16_hi(dd[k >> 1]) : bf16_lo(dd[k >> 1]);
                float e, sig;
                sigmoid_pieces(g, e, sig);
                bool okg, oku;
                vg[k] = dsilu_times_fast_v(g, d, u, e, sig, okg);
                vu[k] = silu_times_fast_v(g, d, sig, oku);
                if (!okg) need[0] |= 1ull << (8 * i + k);
                if (!oku) need[1] |= 1ull << (8 * i + k);
            }
            // decided values rounded two at a time by the hardware converter (the
            // same RNE as the integer form for finite values); the others stay 0
            // for the fp64 pass
            const uint32_t mg = (uint32_t)(need[0] >> (8 * i)) & 0xFFu, mu = (uint32_t)(need[1] >> (8 * i)) & 0xFFu;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const uint32_t keep_g = ((mg >> (2 * k2)) & 1u ? 0u : 0x0000FFFFu) | ((mg >> (2 * k2 + 1)) & 1u ? 0u : 0xFFFF0000u);
                const uint32_t keep_u = ((mu >> (2 * k2)) & 1u ? 0u : 0x0000FFFFu) | ((mu >> (2 * k2 + 1)) & 1u ? 0u : 0xFFFF0000u);
                wg[k2] = cvt_pk_bf16(vg[2 * k2], vg[2 * k2 + 1]) & keep_g;
                wu[k2] = cvt_pk_bf16(vu[2 * k2], vu[2 * k2 + 1]) & keep_u;
            }
            *reinterpret_cast<uint4*>(&vt[0][(rg * 8 + i) * kTile + cg * 8]) = make_uint4(wg[0], wg[1], wg[2], wg[3]);
            *reinterpret_cast<uint4*>(&vt[1][(rg * 8 + i) * kTile + cg * 8]) = make_uint4(wu[0], wu[1], wu[2], wu[3]);
        }
    }
    // 1b: the marked values in fp64.  They are rare but scattered, so a lane
    // would serialize its wave on them: the block gathers them into one list
    // and spreads it over all threads.  Marks beyond the list's room stay with
    // their thread.
    auto fallback = [&](int h, int row, int col) __attribute__((always_inline)) {
        const int64_t r = r0 + row;                      // marked values lie in valid rows
        const int64_t c = j * kTile + col;
        const float g = bf16_value(f32_to_bf16_rne(e4m3_decode1(q_gu[r * ldq_gu + c]) * s_gu[j * lds_gu + r]));
        const float d = bf16_value(dh[r * lddh + c]);
        uint32_t v;
        if (h == 0) {
            const float u = bf16_value(f32_to_bf16_rne(e4m3_decode1(q_gu[r * ldq_gu + F + c]) *
                                                       s_gu[(nb + j) * lds_gu + r]));
            v = dsilu_times_f64(g, d, u);
        } else {
            v = silu_times_f64(g, d);
        }
        vt[h][row * kTile + col] = (uint16_t)v;
    };
    {
        const uint32_t cnt = (uint32_t)(__builtin_popcountll(need[0]) + __builtin_popcountll(need[1]));
        uint32_t at = cnt ? atomicAdd(&fb_count, cnt) : 0u;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            uint64_t m = need[h];
            while (m != 0 && at < (uint32_t)kFbMax) {
                const int idx = __builtin_ctzll(m);
                m &= m - 1;
                fb_list[at++] = (uint16_t)((h << 14) | ((rg * 8 + (idx >> 3)) << 7) | (cg * 8 + (idx & 7)));
            }
            need[h] = m;                                 // what did not fit
        }
    }
    __syncthreads();
    {
        const uint32_t n = fb_count < (uint32_t)kFbMax ? fb_count : (uint32_t)kFbMax;
#pragma unroll 1
        for (uint32_t e = (uint32_t)t; e < n; e += 256u) {
            const uint32_t code = fb_list[e];
            fallback((int)(code >> 14), (int)((code >> 7) & 127u), (int)(code & 127u));
        }
    }
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        while (need[h] != 0) {
            const int idx = __builtin_ctzll(need[h]);
            need[h] &= need[h] - 1;
            fallback(h, rg * 8 + (idx >> 3), cg * 8 + (idx & 7));
        }
    }
    __syncthreads();

    for (int half = 0; half < 2; ++half) {
        const int64_t oc0 = (half == 0 ? 0 : F) + j * kTile;      // first output column of the tile
        const int64_t tile = (half == 0 ? 0 : nb) + j;            // its 1x128 block index
        const uint16_t* vh = vt[half];
        if (dgu != nullptr) {
            uint16_t* po = dgu + (r0 + rg * 8) * lddgu + oc0 + cg * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t r = r0 + rg * 8 + i;
                const uint4 w = *reinterpret_cast<const uint4*>(&vh[(rg * 8 + i) * kTile + cg * 8]);
                if (r < R) st16(po + i * lddgu, w);
            }
        }

        // phase 2: the thread's patch back from LDS, quantized both ways.  Each
        // part reads the patch again rather than keeping it in registers across
        // the barriers of the column scales.
        auto patch = [&](float (&v)[8][8]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 w = *reinterpret_cast<const uint4*>(&vh[(rg * 8 + i) * kTile + cg * 8]);
                v[i][0] = bf16_lo(w.x); v[i][1] = bf16_hi(w.x); v[i][2] = bf16_lo(w.y); v[i][3] = bf16_hi(w.y);
                v[i][4] = bf16_lo(w.z); v[i][5] = bf16_hi(w.z); v[i][6] = bf16_lo(w.w); v[i][7] = bf16_hi(w.w);
            }
        };
        float s_own;
        {
            float v[8][8];
            patch(v);
            // 1x128 first (it needs no other thread's values): each row's tile is
            // the block's 128 columns of that row; lane cg = i of the 16-lane row
            // group computes row i's scale, the others fetch its multiplier with
            // a lane shuffle
            float a_own = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(v[i][k]) & 0x7FFFFFFFu);
                m = max16(m);
                if (cg == i) a_own = floored_absmax(m, amax_floor);
            }
            float iv_own;
            tile_scale(a_own, s_own, iv_own);
            const int lane = t & 63;
            uint8_t* pq8 = q + (r0 + rg * 8) * ldq + oc0 + cg * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float iv = __shfl(iv_own, (lane & 48) | i, 64);
                const int64_t r = r0 + rg * 8 + i;
                if (r < R) st8(pq8 + i * ldq, make_uint2(codes4(v[i], iv), codes4(v[i] + 4, iv)));
            }
        }
        // 128x1: column maxima over the block's 128 rows
        uint32_t mc[8];
        {
            float v[8][8];
            patch(v);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i][k]) & 0x7FFFFFFFu);
                m = max(m, shfl_xor_u32(m, 16));
                m = max(m, shfl_xor_u32(m, 32));
                mc[k] = m;
            }
        }
        if ((t & 63) < 16) {
#pragma unroll
            for (int k = 0; k < 8; ++k) red[wave][cg * 8 + k] = mc[k];
        }
        __syncthreads();
        // thread c < 128 computes column c's scale once and shares its multiplier
        if (t < kTile) {
            const uint32_t m = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
            float sc, iv;
            tile_scale(floored_absmax(m, amax_floor), sc, iv);
            col_mul[t] = iv;
            sT[bl.r * ldsT + oc0 + t] = sc;
        }
        __syncthreads();                                   // col_mul written
        float inv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) inv[k] = col_mul[cg * 8 + k];
        {
            const int64_t rr = r0 + rg * 8 + cg;
            if (cg < 8 && rr < R) s[tile * lds + rr] = s_own;
        }
        // transposed codes through LDS: column k of the patch -> 8 row bytes.  The
        // staged codes overlay vt[0]: for the first tile every thread reads its
        // patch before any thread writes there.
        {
            float v[8][8];
            patch(v);
            if (half == 0) __syncthreads();
            // rows past R are the zero padding of the transposed codes
            const int nv = (int)(R - (r0 + rg * 8) < 8 ? (R - (r0 + rg * 8) < 0 ? 0 : R - (r0 + rg * 8)) : 8);
            const uint32_t vlo = rows_mask_lo(nv), vhi = rows_mask_hi(nv);
            auto emit = [&](auto fix) __attribute__((always_inline)) {
                constexpr bool FIX = decltype(fix)::value;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t lo = fix_codes_if<FIX>(
                        e4m3x4_t<FIX>(v[0][k] * inv[k], v[1][k] * inv[k], v[2][k] * inv[k], v[3][k] * inv[k]),
                        inv[k], v[0][k] * inv[k], v[1][k] * inv[k], v[2][k] * inv[k], v[3][k] * inv[k]) & vlo;
                    const uint32_t hi = fix_codes_if<FIX>(
                        e4m3x4_t<FIX>(v[4][k] * inv[k], v[5][k] * inv[k], v[6][k] * inv[k], v[7][k] * inv[k]),
                        inv[k], v[4][k] * inv[k], v[5][k] * inv[k], v[6][k] * inv[k], v[7][k] * inv[k]) & vhi;
                    *reinterpret_cast<uint2*>(&tr[(cg * 8 + k) * kSwTr + rg * 8]) = make_uint2(lo, hi);
                }
            };
            // one test for all eight column multipliers: finite nonzero ones need no fix-ups
            bool plain = true;
#pragma unroll
            for (int k = 0; k < 8; ++k) plain = plain && plain_mul(inv[k]);
            if (plain) emit(std::false_type{});
            else emit(std::true_type{});
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = p * 32 + (t >> 3);
            const int seg = t & 7;
            const uint2 a = *reinterpret_cast<const uint2*>(&tr[row * kSwTr + seg * 16]);
            const uint2 bq = *reinterpret_cast<const uint2*>(&tr[row * kSwTr + seg * 16 + 8]);
            st16(qT + (oc0 + row) * ldqT + r0 + seg * 16, make_uint4(a.x, a.y, bq.x, bq.y));
        }
        __syncthreads();                                   // red and tr are reused by the second tile
    }
}

hipError_t launch_swiglu_fwd(const uint16_t* gu, int64_t R, int64_t F, int64_t ldgu, float amax_floor,
                             uint8_t* q_gu, int64_t ldq_gu, float* s_gu, int64_t lds_gu,
                             uint8_t* q_h, int64_t ldq_h, float* s_h, int64_t lds_h,
                             uint16_t* h, int64_t ldh, hipStream_t stream)
{
    const dim3 grid(grid_rc((R + kSwRows - 1) / kSwRows, F / kTile));
    if (grid.x == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_swiglu_fwd, grid, dim3(256), 0, stream, gu, R, F, ldgu, amax_floor,
                       q_gu, ldq_gu, s_gu, lds_gu, q_h, ldq_h, s_h, lds_h, h, ldh);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint8_t* q_gu, int64_t R, int64_t F, int64_t ldq_gu,
                             const float* s_gu, int64_t lds_gu, const uint16_t* dh, int64_t lddh,
                             float amax_floor, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             uint16_t* dgu, int64_t lddgu, hipStream_t stream)
{
    const dim3 grid(grid_rc((R + kTile - 1) / kTile, F / kTile));
    if (grid.x == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_swiglu_bwd, grid, dim3(256), 0, stream, q_gu, R, F, ldq_gu, s_gu, lds_gu,
                       dh, lddh, amax_floor, q, ldq, s, lds, qT, ldqT, sT, ldsT, dgu, lddgu);
    return hipGetLastError();
}

}  // namespace fgb
