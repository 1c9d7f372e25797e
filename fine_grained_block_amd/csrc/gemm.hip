// Block-scaled FP8 GEMM for gfx950.
//
// out[m][n] = sum_b SA(m,b) * SB(n,b) * P_b(m,n),
// P_b(m,n)  = sum over the 128-long contraction block b of dec(A[m][t]) * dec(B[n][t]).
//
// Each P_b is one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output piece (the
// block is exactly the instruction's K), computed into a fresh FP32 register
// quad and folded into the FP32 accumulator with one FMA per element:
// acc = fma(P_b, SA*SB, acc).  This is the per-128 "promotion" of the
// partial-sum-drift notes (section 3 row (b), section 5): the matrix core's
// chain never spans more than one 128-block, and dequantization plus the
// running sum happen in FP32 on the vector ALUs.
//
// Tile: 128x128 per block of 4 waves (2x2), 64x64 per wave; the 128-byte K
// slices of A and B are staged through LDS.

#include "device_common.hpp"
#include "fgb_internal.hpp"

namespace fgb {

constexpr int kBM = 128, kBN = 128;
constexpr int kLdsStride = 128 + 16;   // bytes per staged row

__device__ __forceinline__ v8i lds_frag(const uint8_t* base) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 16);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// OUTER: SB(n,b) per output column (Wgrad); otherwise one weight-tile scale per
// 128 output columns.  BF16_OUT: Fprop/Dgrad epilogue; else FP32 (+accumulate).
// GROUP_M: rows grouped per expert (B and its scales chosen per 128-row tile).
// GROUP_K: contraction grouped per expert (blockIdx.z = expert).
template <bool OUTER, bool BF16_OUT, bool GROUP_M, bool GROUP_K>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint8_t As[kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[kBN * kLdsStride];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;

    const uint8_t* B = g.B;
    const float* sb = g.sb;
    int64_t kb0 = 0, kb1 = g.nkb;
    int64_t mend = g.M;
    uint8_t* outp = static_cast<uint8_t*>(g.out);

    if constexpr (GROUP_M) {
        // segments are 128-aligned, so the whole 128-row tile is in one expert
        int64_t total = g.offsets[g.E];
        total = total < g.M ? total : g.M;       // never past R_pad
        if (m0 >= total) return;
        int64_t lo = 0, hi = g.E - 1;             // first e with offsets[e+1] > m0
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (g.offsets[mid + 1] > m0) hi = mid; else lo = mid + 1;
        }
        B += lo * g.b_expert_stride;
        sb += lo * g.sb_expert_stride;
        mend = total;
    }
    if constexpr (GROUP_K) {
        // contraction blocks of expert e, clamped to the R_pad/128 blocks that exist
        const int64_t e = blockIdx.z;
        kb0 = g.offsets[e] / kTile;
        kb1 = g.offsets[e + 1] / kTile;
        kb0 = kb0 < 0 ? 0 : (kb0 > g.nkb ? g.nkb : kb0);
        kb1 = kb1 < kb0 ? kb0 : (kb1 > g.nkb ? g.nkb : kb1);
        outp += e * g.out_expert_stride * (int64_t)sizeof(float);
    }

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int frow = lane & 15;          // fragment row within a 16-row piece
    const int fk = (lane >> 4) * 32;     // this lane's 32-byte K slice
    const int orow = (lane >> 4) * 4;    // output rows orow..orow+3 of a 16x16 piece

    for (int64_t kb = kb0; kb < kb1; ++kb) {
        uint4 ga[4], gb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, seg = id & 7;
            int64_t ar = m0 + row;
            ar = ar < g.M ? ar : g.M - 1;
            ga[i] = ld16(g.A + ar * g.lda + kb * kTile + seg * 16);
            gb[i] = ld16(B + (n0 + row) * g.ldb + kb * kTile + seg * 16);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, seg = id & 7;
            *reinterpret_cast<uint4*>(&As[row * kLdsStride + seg * 16]) = ga[i];
            *reinterpret_cast<uint4*>(&Bs[row * kLdsStride + seg * 16]) = gb[i];
        }
        __syncthreads();

        v8i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = lds_frag(&As[(wm * 64 + i * 16 + frow) * kLdsStride + fk]);
            bf[i] = lds_frag(&Bs[(wn * 64 + i * 16 + frow) * kLdsStride + fk]);
        }

        // scales of this block: SA for the lane's 16 rows, SB per column or per tile
        float sa[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int64_t row = m0 + wm * 64 + i * 16 + orow + r;
                row = row < g.M ? row : g.M - 1;
                sa[i][r] = g.sa[kb * g.sa_ld + row];
            }
        float sbv[4];
        if constexpr (OUTER) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sbv[j] = sb[kb * g.sb_kb + n0 + wn * 64 + j * 16 + frow];
        } else {
            const float s1 = sb[kb * g.sb_kb + (n0 / kTile) * g.sb_n];
#pragma unroll
            for (int j = 0; j < 4; ++j) sbv[j] = s1;
        }

#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bf[j], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sa[i][r] * sbv[j], acc[i][j][r]);
            }
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + orow + r;
                const int64_t col = n0 + wn * 64 + j * 16 + frow;
                if (row >= mend) continue;
                if constexpr (BF16_OUT) {
                    reinterpret_cast<uint16_t*>(outp)[row * g.ldo + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
                } else {
                    float* o = reinterpret_cast<float*>(outp) + row * g.ldo + col;
                    *o = g.accumulate ? *o + acc[i][j][r] : acc[i][j][r];
                }
            }
}

hipError_t launch_gemm(GemmKind kind, bool grouped, const GemmArgs& a, hipStream_t stream)
{
    const dim3 block(256);
    if (kind == kWgrad) {
        dim3 grid((unsigned)(a.N / kBN), (unsigned)((a.M + kBM - 1) / kBM), grouped ? (unsigned)a.E : 1u);
        if (grouped)
            hipLaunchKernelGGL((k_gemm<true, false, false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_gemm<true, false, false, false>), grid, block, 0, stream, a);
    } else {
        dim3 grid((unsigned)(a.N / kBN), (unsigned)((a.M + kBM - 1) / kBM));
        if (grouped)
            hipLaunchKernelGGL((k_gemm<false, true, true, false>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_gemm<false, true, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace fgb
