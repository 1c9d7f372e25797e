// Dynamic E4M3 tile quantization kernels for gfx950.
//
// Tile rule ("scratch: the backward pass, unrolled", section "What is asserted,
// and from where": 1x128 activation tiles, 128x128 weight tiles, Wgrad
// operands re-tiled 128x1; partial-sum-drift notes, section 3 row (a): scale
// from the in-block absmax; prime-rl PR #4073 conventions table: /448, -0):
//   a = max(absmax(tile), floor); s = fl32(a/448); inv = a ? min(fl32(448/a), FLT_MAX) : 0
//   q = e4m3_rne_sat(fl32(x * inv))
//
// All kernels are HBM-bound; they read their bf16 inputs with non-temporal loads
// (read once: the next GEMM's operands, the codes written here, keep the caches;
// in the linear step the 1x128 cast of X runs 24% faster, the step 2%).  The
// absmax is an integer max over |bits|
// (exact, independent of denormal modes); scale and inverse are IEEE fp32
// divisions, one pair per tile; the cast is the hardware v_cvt_pk_fp8_f32.

#include "device_common.hpp"
#include "fgb_internal.hpp"

namespace fgb {

// ---------------------------------------------------------------------------
// 1x128.  A block of 256 threads covers 64 rows of one 128-column block; each
// group of 16 lanes owns one row at a time (8 bf16 = 16 B per lane, so a
// group reads the tile's 256 contiguous bytes) and reduces its absmax with
// DPP inside the 16-lane row.
// ---------------------------------------------------------------------------
constexpr int kQ1Per = 4;                       // rows per 16-lane group
constexpr int kQ1Rows = 16 * kQ1Per;

// PO2: power-of-two scales (the UE8M0 values, held in fp32); otherwise absmax/448.
// SR: stochastic rounding of the cast with the words of `sr` (absmax/448 scales).
template <bool PO2, bool SR>
__global__ __launch_bounds__(256) void k_quantize_1x128(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds, SrArgs sr)
{
    static_assert(!(PO2 && SR), "stochastic rounding uses absmax/448 scales");
    const int lane16 = threadIdx.x & 15;
    const int grp = threadIdx.x >> 4;
    const BlockRC bl = block_rc(true, (R + kQ1Rows - 1) / kQ1Rows, (C + kTile - 1) / kTile);
    const int64_t rb = bl.r * kQ1Rows;
    const int64_t j = bl.c;
    const int64_t c = j * kTile + lane16 * 8;
    const bool cok = c < C;
    // all kQ1Rows rows and the whole 128-column block inside the tensor
    // (block-uniform): no checks, rows addressed from one 64-bit pointer
    const bool full = rb + kQ1Rows <= R && (j + 1) * kTile <= C;
    const uint16_t* const xrow = x + (rb + grp) * ldx + c;

    uint4 v[kQ1Per];
#pragma unroll
    for (int it = 0; it < kQ1Per; ++it) {
        const bool ok = full || (cok && rb + grp + 16 * it < R);
        v[it] = ok ? ld16_stream(xrow + 16 * it * ldx) : make_uint4(0u, 0u, 0u, 0u);
    }
    // the 4 row maxima; lane it of the 16-lane row group then computes row it's
    // scale (one pair of divisions per wave) and every lane fetches the
    // multiplier of row it from that lane
    float a_own = 0.0f;
#pragma unroll
    for (int it = 0; it < kQ1Per; ++it) {
        const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
        u16x2 m2 = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int k = 1; k < 4; ++k)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
        uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]);
        m = max16(m);
        if (lane16 == it) a_own = floored_absmax(m << 16, amax_floor);
    }
    float sc_own = 0.0f, inv_own;
    uint32_t eb_own = 0;
    if constexpr (PO2) tile_scale_ue8m0(a_own, eb_own, inv_own);
    else tile_scale(a_own, sc_own, inv_own);
    const int lane = threadIdx.x & 63;
    uint8_t* const qrow = q + (rb + grp) * ldq + c;
    float invs[kQ1Per];
    bool plain = true;
#pragma unroll
    for (int it = 0; it < kQ1Per; ++it) {
        invs[it] = __shfl(inv_own, (lane & 48) | it, 64);
        plain = plain && plain_mul_t<PO2>(invs[it]);
    }
    auto emit = [&](auto fix) __attribute__((always_inline)) {
        constexpr bool FIX = decltype(fix)::value;
#pragma unroll
        for (int it = 0; it < kQ1Per; ++it) {
            const int64_t r = rb + grp + 16 * it;
            const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
            const float inv = invs[it];
            uint32_t o0, o1;
            if constexpr (SR) {
                uint32_t u[8];
                sr_words8(sr, r, c, u);
                o0 = e4m3x4_sr(bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, bf16_lo(w[1]) * inv, bf16_hi(w[1]) * inv,
                               u[0], u[1], u[2], u[3]);
                o1 = e4m3x4_sr(bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, bf16_lo(w[3]) * inv, bf16_hi(w[3]) * inv,
                               u[4], u[5], u[6], u[7]);
            } else {
                o0 = e4m3x4_t<FIX>(bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, bf16_lo(w[1]) * inv, bf16_hi(w[1]) * inv);
                o1 = e4m3x4_t<FIX>(bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, bf16_lo(w[3]) * inv, bf16_hi(w[3]) * inv);
            }
            o0 = fix_codes_if<FIX>(o0, inv, bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, bf16_lo(w[1]) * inv,
                                   bf16_hi(w[1]) * inv);
            o1 = fix_codes_if<FIX>(o1, inv, bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, bf16_lo(w[3]) * inv,
                                   bf16_hi(w[3]) * inv);
            if (full || (cok && r < R)) st8(qrow + 16 * it * ldq, make_uint2(o0, o1));
        }
    };
    // finite nonzero multipliers (the common case): no product is NaN, no fix-up
    if (plain) emit(std::false_type{});
    else emit(std::true_type{});
    if (lane16 < kQ1Per) {     // the block's segment j exists (grid = ceil(C/128)): only rows can be past the end
        const int64_t r = rb + grp + 16 * lane16;
        if (r < R) s[j * lds + r] = PO2 ? e8m0_to_f32(eb_own) : sc_own;
    }
}

static SrArgs sr_args(const SrParams* sr)
{
    SrArgs a;
    if (sr) {
        a.k0 = (uint32_t)sr->seed;
        a.k1 = (uint32_t)(sr->seed >> 32);
        a.salt = sr->salt;
    }
    return a;
}

hipError_t launch_quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                                 float amax_floor, uint8_t* q, int64_t ldq,
                                 float* s, int64_t lds, bool po2, hipStream_t stream, const SrParams* sr)
{
    if (po2 && sr) return hipErrorInvalidValue;
    const dim3 grid(grid_rc((R + kQ1Rows - 1) / kQ1Rows, (C + kTile - 1) / kTile));
    if (grid.x == 0) return hipErrorInvalidValue;
    const SrArgs a = sr_args(sr);
    if (po2)
        hipLaunchKernelGGL((k_quantize_1x128<true, false>), grid, dim3(256), 0, stream,
                           x, R, C, ldx, amax_floor, q, ldq, s, lds, a);
    else if (sr)
        hipLaunchKernelGGL((k_quantize_1x128<false, true>), grid, dim3(256), 0, stream,
                           x, R, C, ldx, amax_floor, q, ldq, s, lds, a);
    else
        hipLaunchKernelGGL((k_quantize_1x128<false, false>), grid, dim3(256), 0, stream,
                           x, R, C, ldx, amax_floor, q, ldq, s, lds, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128-element tile kernels (128x1 columns, 128x128 weight tiles, requant,
// and the dual 1x128 + 128x1 quantization of one tensor).
// Block = 256 threads over rows [r0, r0+128) x columns [c0, c0+128).  Thread t
// holds an 8x8 patch: columns c0 + 8*(t%16) .. +8, rows r0 + 8*(t/16) .. +8.
// Column maxima combine the 4 patches of a wave with lane swizzles and the 4
// waves through LDS.  Transposed codes are staged in LDS as [column][row] so
// every global store writes whole 16-byte pieces of 128-byte qT rows.
// ---------------------------------------------------------------------------
constexpr int kTrStride = 136;   // bytes per staged qT row (128 + 8 to spread banks)

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }


// PO2: the scales written are powers of two (the UE8M0 values, held in fp32).
// SR: stochastic rounding of every cast with the words of `sr` (element (r, c)
// of the input draws word (r, c), so q, qT and the dual outputs of one element
// use the same word); absmax/448 scales, not for the requant.
template <int MODE, bool PO2, bool SR>
__global__ __launch_bounds__(256) void k_tile128(
    const void* __restrict__ in, int64_t R, int64_t C, int64_t ldin,
    const float* __restrict__ s_in, int64_t lds_in, float amax_floor,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qT, int64_t ldqT,
    float* __restrict__ s_out, int64_t lds_out, float* __restrict__ s_row, int64_t lds_row, SrArgs sr,
    TileBatch bt, int cols_fast)
{
    static_assert(!(SR && (PO2 || MODE == kTileRequant || MODE == kTileRequant128x128)),
                  "stochastic rounding: absmax/448 scales, no requant");
    // batched launches: matrix blockIdx.z of a stack (byte strides; scales in floats)
    if (blockIdx.z > 0) {
        const int64_t z = blockIdx.z;
        in = static_cast<const uint8_t*>(in) + z * bt.in;
        if (q != nullptr) q += z * bt.q;
        if (qT != nullptr) qT += z * bt.qT;
        s_out += z * bt.s;
    }
    // one scale per 128x128 tile: the weight quantizer and its requant
    constexpr bool TILE = MODE == kTile128x128 || MODE == kTileRequant128x128;
    // scale of absmax a: fp32 (s = a/448, mul = 448/a) or power of two (E8M0 byte, mul = 2^-e)
    auto scale_of = [&](float a, float& sc, uint32_t& eb, float& mul) {
        if constexpr (PO2) tile_scale_ue8m0(a, eb, mul);
        else tile_scale(a, sc, mul);
    };
    auto put_scale = [&](float* base, int64_t idx, float sc, uint32_t eb) {
        base[idx] = PO2 ? e8m0_to_f32(eb) : sc;
    };
    __shared__ uint32_t red[4][kTile];
    __shared__ float col_mul[kTile];
    __shared__ __attribute__((aligned(16))) uint8_t tr[kTile * kTrStride];

    const int t = threadIdx.x;
    const int cg = t & 15, rg = t >> 4, wave = t >> 6;
    const BlockRC bl = block_rc(cols_fast != 0, (R + kTile - 1) / kTile, (C + kTile - 1) / kTile);
    const int64_t r0 = bl.r * kTile;
    const int64_t c0 = bl.c * kTile;
    const int64_t cc = c0 + cg * 8;
    const bool cok = cc < C;
    // the whole 128x128 tile lies inside the tensor (block-uniform): then no
    // row or column checks, and row i of a patch is its row 0 plus i leading
    // dimensions (one 64-bit address per thread, scalar row steps)
    const bool full = r0 + kTile <= R && c0 + kTile <= C;

    // The thread's 8x8 patch, V(i, k) = row i, column k: bf16 inputs stay
    // packed two to a word and are widened where used (exact); requant inputs
    // are dequantized once into fp32.
    constexpr bool REQ = MODE == kTileRequant || MODE == kTileRequant128x128;
    uint32_t vw[REQ ? 1 : 8][4];
    float vf[REQ ? 8 : 1][8];
    if constexpr (REQ) {
        // dequantize: v = fl32(dec(q) * s) with the row's 1x128 scale, or the
        // tile's scale s_in[i * lds_in + j] for a 128x128 weight tile.  The
        // codes are requested first; the 128 row scales of the block go through
        // LDS, one load per thread instead of eight per thread.
        const uint8_t* prow = static_cast<const uint8_t*>(in) + (r0 + rg * 8) * ldin + cc;
        uint2 w[8];
        if (full) {
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = ld8(prow + i * ldin);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[i] = (cok && r0 + rg * 8 + i < R) ? ld8(prow + i * ldin) : make_uint2(0u, 0u);
        }
        float sr[8];
        if constexpr (MODE == kTileRequant) {
            if (t < kTile) col_mul[t] = r0 + t < R ? s_in[bl.c * lds_in + r0 + t] : 0.0f;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) sr[i] = col_mul[rg * 8 + i];
            // (col_mul is rewritten with the column multipliers only after the
            // barrier that publishes the column maxima, which every thread
            // reaches after these reads)
        } else {
            const float st = s_in[bl.r * lds_in + bl.c];
#pragma unroll
            for (int i = 0; i < 8; ++i) sr[i] = st;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float si = (cok && r0 + rg * 8 + i < R) ? sr[i] : 0.0f;
            const float2 d0 = e4m3x2_decode<false>(w[i].x), d1 = e4m3x2_decode<true>(w[i].x);
            const float2 d2 = e4m3x2_decode<false>(w[i].y), d3 = e4m3x2_decode<true>(w[i].y);
            vf[i][0] = d0.x * si; vf[i][1] = d0.y * si; vf[i][2] = d1.x * si; vf[i][3] = d1.y * si;
            vf[i][4] = d2.x * si; vf[i][5] = d2.y * si; vf[i][6] = d3.x * si; vf[i][7] = d3.y * si;
        }
    }
    if constexpr (!REQ) {
        const uint16_t* prow = static_cast<const uint16_t*>(in) + (r0 + rg * 8) * ldin + cc;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = full || (cok && r0 + rg * 8 + i < R);
            const uint4 w = ok ? ld16_stream(prow + i * ldin) : make_uint4(0u, 0u, 0u, 0u);
            vw[i][0] = w.x; vw[i][1] = w.y; vw[i][2] = w.z; vw[i][3] = w.w;
        }
    }
    auto V = [&](int i, int k) __attribute__((always_inline)) -> float {
        if constexpr (REQ) return vf[i][k];
        else return (k & 1) ? bf16_hi(vw[i][k >> 1]) : bf16_lo(vw[i][k >> 1]);
    };

    // Dual mode, 1x128 part (first: it needs no other thread's values): row r's
    // tile is the block's 128 columns of row r, held by the 16 lanes that share
    // rg; their absmax is one DPP reduction.
    if constexpr (MODE == kTileDual && !SR) {
        // the 8 row maxima of the patch rows; lane cg = i of the 16-lane row
        // group then computes row i's scale (one pair of divisions per wave) and
        // every lane fetches the multiplier of row i from that lane
        float a_own = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) m = max(m, abs_bits(V(i, k)));
            m = max16(m);
            if (cg == i) a_own = floored_absmax(m, amax_floor);
        }
        float sr_own = 0.0f, iv_own;
        uint32_t er_own = 0;
        scale_of(a_own, sr_own, er_own, iv_own);
        const int lane = t & 63;
        float ivs[8];
        bool plain = true;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ivs[i] = __shfl(iv_own, (lane & 48) | i, 64);
            plain = plain && plain_mul_t<PO2>(ivs[i]);
        }
        auto emit = [&](auto fix) __attribute__((always_inline)) {
            constexpr bool FIX = decltype(fix)::value;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float iv = ivs[i];
                const int64_t r = r0 + rg * 8 + i;
                const uint32_t o0 = fix_codes_if<FIX>(e4m3x4_t<FIX>(V(i, 0) * iv, V(i, 1) * iv, V(i, 2) * iv, V(i, 3) * iv),
                                                      iv, V(i, 0) * iv, V(i, 1) * iv, V(i, 2) * iv, V(i, 3) * iv);
                const uint32_t o1 = fix_codes_if<FIX>(e4m3x4_t<FIX>(V(i, 4) * iv, V(i, 5) * iv, V(i, 6) * iv, V(i, 7) * iv),
                                                      iv, V(i, 4) * iv, V(i, 5) * iv, V(i, 6) * iv, V(i, 7) * iv);
                if (full || (cok && r < R)) st8(q + (r0 + rg * 8) * ldq + cc + i * ldq, make_uint2(o0, o1));
            }
        };
        if (plain) emit(std::false_type{});
        else emit(std::true_type{});
        // lanes cg = 0..7 of each row group write the scales of rows rg*8 + cg
        const int64_t rr = r0 + rg * 8 + cg;
        if (cg < 8 && rr < R) put_scale(s_row, bl.c * lds_row + rr, sr_own, er_own);
    }

    float inv[8];
    if constexpr (TILE) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int k = 0; k < 8; ++k) m = max(m, abs_bits(V(i, k)));
        m = max16(m);
        m = max(m, shfl_xor_u32(m, 16));
        m = max(m, shfl_xor_u32(m, 32));
        if ((t & 63) == 0) red[wave][0] = m;
        __syncthreads();
        m = max(max(red[0][0], red[1][0]), max(red[2][0], red[3][0]));
        const float a = floored_absmax(m, amax_floor);
        float sc = 0.0f, iv;
        uint32_t eb = 0;
        scale_of(a, sc, eb, iv);
#pragma unroll
        for (int k = 0; k < 8; ++k) inv[k] = iv;
        if (t == 0) put_scale(s_out, bl.r * lds_out + bl.c, sc, eb);
    } else {
        uint32_t mc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = max(m, abs_bits(V(i, k)));
            m = max(m, shfl_xor_u32(m, 16));
            m = max(m, shfl_xor_u32(m, 32));
            mc[k] = m;
        }
        if ((t & 63) < 16) {
#pragma unroll
            for (int k = 0; k < 8; ++k) red[wave][cg * 8 + k] = mc[k];
        }
        __syncthreads();
        // thread c < 128 computes column c's scale (two IEEE divisions) once for
        // the block and shares its multiplier through LDS
        if (t < kTile) {
            const uint32_t m = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
            const float a = floored_absmax(m, amax_floor);
            float sc = 0.0f, iv;
            uint32_t eb = 0;
            scale_of(a, sc, eb, iv);
            col_mul[t] = iv;
            if (c0 + t < C) put_scale(s_out, bl.r * lds_out + c0 + t, sc, eb);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) inv[k] = col_mul[cg * 8 + k];
    }

    if constexpr (SR) {
        // Row by row: the 8 words of the patch row, then its codes -- with the
        // row's own 1x128 scale (dual), the column scales (128x1, dual) or the
        // tile scale (128x128) -- kept as row-major bytes cr[i] and transposed
        // through LDS like the round-to-nearest path.
        uint32_t cr[8][2];
        float sr_own = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + rg * 8 + i;
            uint32_t u[8];
            sr_words8(sr, r, cc, u);
            if constexpr (MODE == kTileDual) {
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) m = max(m, abs_bits(V(i, k)));
                m = max16(m);
                const float a = floored_absmax(m, amax_floor);
                float sc, iv;
                tile_scale(a, sc, iv);
                if (cg == i) sr_own = sc;
                const uint32_t o0 = fix_codes(e4m3x4_sr(V(i, 0) * iv, V(i, 1) * iv, V(i, 2) * iv,
                                                        V(i, 3) * iv, u[0], u[1], u[2], u[3]), iv,
                                              V(i, 0) * iv, V(i, 1) * iv, V(i, 2) * iv, V(i, 3) * iv);
                const uint32_t o1 = fix_codes(e4m3x4_sr(V(i, 4) * iv, V(i, 5) * iv, V(i, 6) * iv,
                                                        V(i, 7) * iv, u[4], u[5], u[6], u[7]), iv,
                                              V(i, 4) * iv, V(i, 5) * iv, V(i, 6) * iv, V(i, 7) * iv);
                if (cok && r < R) st8(q + r * ldq + cc, make_uint2(o0, o1));
            }
            // rows past R are the zero padding of the transposed codes
            const bool rok = r < R;
            cr[i][0] = rok ? fix_codes4(e4m3x4_sr(V(i, 0) * inv[0], V(i, 1) * inv[1], V(i, 2) * inv[2],
                                                  V(i, 3) * inv[3], u[0], u[1], u[2], u[3]),
                                        inv[0], inv[1], inv[2], inv[3],
                                        V(i, 0) * inv[0], V(i, 1) * inv[1], V(i, 2) * inv[2], V(i, 3) * inv[3])
                           : 0u;
            cr[i][1] = rok ? fix_codes4(e4m3x4_sr(V(i, 4) * inv[4], V(i, 5) * inv[5], V(i, 6) * inv[6],
                                                  V(i, 7) * inv[7], u[4], u[5], u[6], u[7]),
                                        inv[4], inv[5], inv[6], inv[7],
                                        V(i, 4) * inv[4], V(i, 5) * inv[5], V(i, 6) * inv[6], V(i, 7) * inv[7])
                           : 0u;
            if constexpr (TILE) {
                if (q != nullptr && cok && r < R) st8(q + r * ldq + cc, make_uint2(cr[i][0], cr[i][1]));
            }
        }
        if constexpr (MODE == kTileDual) {
            const int64_t rr = r0 + rg * 8 + cg;
            if (cg < 8 && rr < R) s_row[bl.c * lds_row + rr] = sr_own;
        }
        if constexpr (TILE) {
            if (qT == nullptr) return;
        }
        // column k of the patch: byte k & 3 of cr[i][k >> 2] for rows i = 0..7
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int sh = (k & 3) * 8, h = k >> 2;
            const uint32_t lo = ((cr[0][h] >> sh) & 0xFFu) | (((cr[1][h] >> sh) & 0xFFu) << 8) |
                                (((cr[2][h] >> sh) & 0xFFu) << 16) | (((cr[3][h] >> sh) & 0xFFu) << 24);
            const uint32_t hi = ((cr[4][h] >> sh) & 0xFFu) | (((cr[5][h] >> sh) & 0xFFu) << 8) |
                                (((cr[6][h] >> sh) & 0xFFu) << 16) | (((cr[7][h] >> sh) & 0xFFu) << 24);
            *reinterpret_cast<uint2*>(&tr[(cg * 8 + k) * kTrStride + rg * 8]) = make_uint2(lo, hi);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = p * 32 + (t >> 3);
            const int seg = t & 7;
            const int64_t c = c0 + row;
            const uint2 a = *reinterpret_cast<const uint2*>(&tr[row * kTrStride + seg * 16]);
            const uint2 b = *reinterpret_cast<const uint2*>(&tr[row * kTrStride + seg * 16 + 8]);
            if (c < C) st16(qT + c * ldqT + r0 + seg * 16, make_uint4(a.x, a.y, b.x, b.y));
        }
        return;
    }

    // Row-major codes (128x128 weights, q != nullptr): 8 bytes per patch row.
    if constexpr (TILE) {
        if (q != nullptr) {
            auto emit = [&](auto fix) __attribute__((always_inline)) {
                constexpr bool FIX = decltype(fix)::value;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t r = r0 + rg * 8 + i;
                    const uint32_t o0 = fix_codes_if<FIX>(
                        e4m3x4_t<FIX>(V(i, 0) * inv[0], V(i, 1) * inv[1], V(i, 2) * inv[2], V(i, 3) * inv[3]), inv[0],
                        V(i, 0) * inv[0], V(i, 1) * inv[1], V(i, 2) * inv[2], V(i, 3) * inv[3]);
                    const uint32_t o1 = fix_codes_if<FIX>(
                        e4m3x4_t<FIX>(V(i, 4) * inv[4], V(i, 5) * inv[5], V(i, 6) * inv[6], V(i, 7) * inv[7]), inv[4],
                        V(i, 4) * inv[4], V(i, 5) * inv[5], V(i, 6) * inv[6], V(i, 7) * inv[7]);
                    if (full || (cok && r < R)) st8(q + (r0 + rg * 8) * ldq + cc + i * ldq, make_uint2(o0, o1));
                }
            };
            if (plain_mul_t<PO2>(inv[0])) emit(std::false_type{});          // one multiplier for the whole tile
            else emit(std::true_type{});
        }
        if (qT == nullptr) return;
    }

    // Transposed codes: column k of the patch -> 8 row bytes, staged in LDS;
    // rows past R are the zero padding (a NaN tile's codes must not reach it).
    const int nv = (int)(R - (r0 + rg * 8) < 8 ? (R - (r0 + rg * 8) < 0 ? 0 : R - (r0 + rg * 8)) : 8);
    const uint32_t vlo = rows_mask_lo(nv), vhi = rows_mask_hi(nv);
    auto emit_t = [&](auto fix) __attribute__((always_inline)) {
        constexpr bool FIX = decltype(fix)::value;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t lo = fix_codes_if<FIX>(
                                    e4m3x4_t<FIX>(V(0, k) * inv[k], V(1, k) * inv[k], V(2, k) * inv[k], V(3, k) * inv[k]),
                                    inv[k], V(0, k) * inv[k], V(1, k) * inv[k], V(2, k) * inv[k], V(3, k) * inv[k])
                                & vlo;
            const uint32_t hi = fix_codes_if<FIX>(
                                    e4m3x4_t<FIX>(V(4, k) * inv[k], V(5, k) * inv[k], V(6, k) * inv[k], V(7, k) * inv[k]),
                                    inv[k], V(4, k) * inv[k], V(5, k) * inv[k], V(6, k) * inv[k], V(7, k) * inv[k])
                                & vhi;
            *reinterpret_cast<uint2*>(&tr[(cg * 8 + k) * kTrStride + rg * 8]) = make_uint2(lo, hi);
        }
    };
    bool plain = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) plain = plain && plain_mul_t<PO2>(inv[k]);
    if (plain) emit_t(std::false_type{});
    else emit_t(std::true_type{});
    __syncthreads();
    // 128 staged rows of 128 bytes; 8 threads per row, 16 bytes each, 4 passes.
    uint8_t* const pq = qT + (c0 + (t >> 3)) * ldqT + r0 + (t & 7) * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = p * 32 + (t >> 3);
        const int seg = t & 7;
        const uint2 a = *reinterpret_cast<const uint2*>(&tr[row * kTrStride + seg * 16]);
        const uint2 b = *reinterpret_cast<const uint2*>(&tr[row * kTrStride + seg * 16 + 8]);
        if (full || c0 + row < C) st16(pq + p * 32 * ldqT, make_uint4(a.x, a.y, b.x, b.y));
    }
}

template <bool PO2, bool SR>
static void launch_tile128_t(TileMode mode, dim3 grid, const void* in, int64_t R, int64_t C, int64_t ldin,
                             const float* s_in, int64_t lds_in, float amax_floor,
                             uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                             float* s_out, int64_t lds_out, hipStream_t stream, float* s_row, int64_t lds_row,
                             SrArgs a, TileBatch bt, int cols_fast)
{
    switch (mode) {
    case kTile128x1:
        hipLaunchKernelGGL((k_tile128<kTile128x1, PO2, SR>), grid, dim3(256), 0, stream, in, R, C, ldin,
                           s_in, lds_in, amax_floor, q, ldq, qT, ldqT, s_out, lds_out, s_row, lds_row, a, bt, cols_fast);
        break;
    case kTile128x128:
        hipLaunchKernelGGL((k_tile128<kTile128x128, PO2, SR>), grid, dim3(256), 0, stream, in, R, C, ldin,
                           s_in, lds_in, amax_floor, q, ldq, qT, ldqT, s_out, lds_out, s_row, lds_row, a, bt, cols_fast);
        break;
    case kTileRequant:
        if constexpr (!SR)
            hipLaunchKernelGGL((k_tile128<kTileRequant, PO2, false>), grid, dim3(256), 0, stream, in, R, C, ldin,
                               s_in, lds_in, amax_floor, q, ldq, qT, ldqT, s_out, lds_out, s_row, lds_row, a, bt, cols_fast);
        break;
    case kTileDual:
        hipLaunchKernelGGL((k_tile128<kTileDual, PO2, SR>), grid, dim3(256), 0, stream, in, R, C, ldin,
                           s_in, lds_in, amax_floor, q, ldq, qT, ldqT, s_out, lds_out, s_row, lds_row, a, bt, cols_fast);
        break;
    case kTileRequant128x128:
        if constexpr (!SR)
            hipLaunchKernelGGL((k_tile128<kTileRequant128x128, PO2, false>), grid, dim3(256), 0, stream, in, R, C,
                               ldin, s_in, lds_in, amax_floor, q, ldq, qT, ldqT, s_out, lds_out, s_row, lds_row, a, bt, cols_fast);
        break;
    }
}

hipError_t launch_tile128(TileMode mode, const void* in, int64_t R, int64_t C, int64_t ldin,
                          const float* s_in, int64_t lds_in, float amax_floor,
                          uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                          float* s_out, int64_t lds_out, bool po2, hipStream_t stream,
                          float* s_row, int64_t lds_row, const SrParams* sr, int64_t batch, TileBatch bt)
{
    if (sr && (po2 || mode == kTileRequant || mode == kTileRequant128x128)) return hipErrorInvalidValue;
    if (batch < 1 || batch > 65535) return hipErrorInvalidValue;
    const dim3 grid(grid_rc((R + kTile - 1) / kTile, (C + kTile - 1) / kTile), 1, (unsigned)batch);
    if (grid.x == 0) return hipErrorInvalidValue;
    const SrArgs a = sr_args(sr);
    // block order (block_rc): column blocks fastest for the row-major-output
    // tilings when the input pitch is a multiple of 8 KB, row blocks otherwise
    const int64_t pitch = ldin * (mode == kTileRequant || mode == kTileRequant128x128 ? 1 : 2);
    const int cols_fast = (mode == kTile128x128 || mode == kTileDual || mode == kTileRequant128x128) &&
                          pitch % 8192 == 0;
    if (po2)
        launch_tile128_t<true, false>(mode, grid, in, R, C, ldin, s_in, lds_in, amax_floor, q, ldq, qT, ldqT,
                                      s_out, lds_out, stream, s_row, lds_row, a, bt, cols_fast);
    else if (sr)
        launch_tile128_t<false, true>(mode, grid, in, R, C, ldin, s_in, lds_in, amax_floor, q, ldq, qT, ldqT,
                                      s_out, lds_out, stream, s_row, lds_row, a, bt, cols_fast);
    else
        launch_tile128_t<false, false>(mode, grid, in, R, C, ldin, s_in, lds_in, amax_floor, q, ldq, qT, ldqT,
                                       s_out, lds_out, stream, s_row, lds_row, a, bt, cols_fast);
    return hipGetLastError();
}

}  // namespace fgb
