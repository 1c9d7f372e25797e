// Internal launch interface of libfgb: the C ABI (abi.hip) validates arguments
// and calls these; the kernels live in quant.hip, gemm.hip and swiglu.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgb {

// ----------------------------- quantizers ---------------------------------
// Stochastic rounding of the cast: Philox4x32-10 words keyed by seed, with the
// salt in the counter (NULL = round to nearest).
struct SrParams { uint64_t seed; uint32_t salt; };

// po2: power-of-two scales (the UE8M0 value set, in fp32); otherwise absmax/448.
// sr (absmax/448 scales only): stochastic rounding; NULL = round to nearest.
hipError_t launch_quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                                 float amax_floor, uint8_t* q, int64_t ldq,
                                 float* s, int64_t lds, bool po2, hipStream_t stream,
                                 const SrParams* sr = nullptr);

enum TileMode { kTile128x1 = 0, kTile128x128 = 1, kTileRequant = 2, kTileDual = 3, kTileRequant128x128 = 4 };

// 128x128 tile kernels over a [R][C] input:
//   kTile128x1:   bf16 in, per-column 128-row scales, transposed codes out (qT, sT)
//   kTile128x128: bf16 in, one scale per tile, q and/or qT out, s [R/128][C/128]
//   kTileRequant: E4M3 + 1x128 scales in, then as kTile128x1
//   kTileDual:    bf16 in, both the 1x128 codes and scales (q, s_row) and the
//                 128x1 transposed codes and scales (qT, sT) from one read
//   kTileRequant128x128: E4M3 + one fp32 scale per 128x128 tile in
//                 (s_in[i * lds_in + j]), then as kTile128x128
// po2 as above for every scale written (scales read by the requant are fp32 either way).
// sr: stochastic rounding for kTile128x1, kTile128x128 and kTileDual (absmax/448).
// A stack of `batch` matrices of the same shape, matrix z at z * (byte strides
// in, q, qT; float stride s) from the first (grid z; the 128x128 quantizer).
struct TileBatch { int64_t in = 0, q = 0, qT = 0, s = 0; };
hipError_t launch_tile128(TileMode mode, const void* in, int64_t R, int64_t C, int64_t ldin,
                          const float* s_in, int64_t lds_in, float amax_floor,
                          uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                          float* s_out, int64_t lds_out, bool po2, hipStream_t stream,
                          float* s_row = nullptr, int64_t lds_row = 0, const SrParams* sr = nullptr,
                          int64_t batch = 1, TileBatch bt = TileBatch{});

// ------------------------------- SwiGLU ------------------------------------
// [G | U] is one [R][2F] bf16 tensor, F % 128 == 0.  Forward: the 1x128 stash
// of [G | U] (q_gu, s_gu; both NULL to skip), the 1x128 codes of
// H = bf16(silu(G) U) (q_h, s_h), and H itself (h, NULL to skip).
hipError_t launch_swiglu_fwd(const uint16_t* gu, int64_t R, int64_t F, int64_t ldgu, float amax_floor,
                             uint8_t* q_gu, int64_t ldq_gu, float* s_gu, int64_t lds_gu,
                             uint8_t* q_h, int64_t ldq_h, float* s_h, int64_t lds_h,
                             uint16_t* h, int64_t ldh, hipStream_t stream);
// Backward: from the stash and dH [R][F], [dG | dU] [R][2F] quantized 1x128
// (q, s) and 128x1 (qT [2F][ldqT >= roundup(R,128)] zero padded, sT), and
// [dG | dU] itself (dgu, NULL to skip).
hipError_t launch_swiglu_bwd(const uint8_t* q_gu, int64_t R, int64_t F, int64_t ldq_gu,
                             const float* s_gu, int64_t lds_gu, const uint16_t* dh, int64_t lddh,
                             float amax_floor, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             uint16_t* dgu, int64_t lddgu, hipStream_t stream);

// ------------------------------- GEMMs -------------------------------------
// out[m][n] = sum_b SA(m,b) * SB(n,b) * sum_{t in block b} dec(A[m][t]) dec(B[n][t])
//   A [M][lda], B [N][ldb]: both contraction-contiguous E4M3 codes
//   SA(m,b) = sa[b*sa_ld + m]
//   SB(n,b) = sb[b*sb_kb + n]                 (outer-product scales, Wgrad)
//           = sb[b*sb_kb + (n/128)*sb_n]      (128x128 weight tiles, Fprop/Dgrad)
enum GemmKind { kFprop = 0, kDgrad = 1, kWgrad = 2 };

struct GemmArgs {
    int64_t M = 0, N = 0;       // output rows / columns
    int64_t nkb = 0;            // number of 128-long contraction blocks
    const uint8_t* A = nullptr; int64_t lda = 0;
    const uint8_t* B = nullptr; int64_t ldb = 0;
    const float* sa = nullptr;  int64_t sa_ld = 0;
    const float* sb = nullptr;  int64_t sb_kb = 0, sb_n = 0;
    void* out = nullptr;        int64_t ldo = 0;
    int accumulate = 0;         // Wgrad: out += result
    // dense only: the tiles from split_from on (those that do not fill a whole
    // round of CUs) are computed as column halves by two blocks each (set by
    // launch_gemm)
    int64_t split_from = -1;
    // grouped forms
    const int32_t* offsets = nullptr;  // device, E+1 entries
    int64_t E = 0;
    int64_t b_expert_stride = 0;       // elements of B per expert   (M-grouped)
    int64_t sb_expert_stride = 0;      // floats of sb per expert    (M-grouped)
    int64_t out_expert_stride = 0;     // elements of out per expert (K-grouped)
};

// Whether launch_gemm can address the operands: the kernel uses 32-bit byte
// offsets inside each operand.  Dense GEMMs are cut into pieces that fit (so
// only a leading dimension above ~16M bytes is refused); grouped operands must
// each stay within 4 GiB.
bool gemm_supported(const GemmArgs& args, bool grouped);

// po2: every scale is a power of two (the matrix core applies them; no rescale).
hipError_t launch_gemm(GemmKind kind, bool grouped, const GemmArgs& args, hipStream_t stream, bool po2 = false);

}  // namespace fgb
