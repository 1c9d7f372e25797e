/*
 * fgb.h -- fine-grained block-scaled FP8 linear layers on MI355X (gfx950).
 *
 * C ABI of libfgb.so.  The library computes the FP8 path of one linear layer:
 * dynamic E4M3 tile quantization (1x128 activation/gradient tiles, 128x128
 * weight tiles, 128x1 re-tiling of Wgrad's transposed operands) and the
 * block-scaled GEMM that multiplies each 128-long contraction segment's FP8
 * partial sum by s_a * s_b and accumulates in FP32, for Fprop (Y = X W, BF16),
 * Dgrad (dX = dY W^T, BF16) and Wgrad (dW = X^T dY, FP32), dense and grouped
 * per MoE expert.
 *
 * Sources (by page and section):
 *   [scratch]  "scratch: the backward pass, unrolled" (deepseek-v3.ezyang.com),
 *              section "What is asserted, and from where".
 *   [drift]    "FP8 dynamic quantization partial-sum drift" (foosynaptic
 *              deepseek tech notes), section 3 table rows (a)/(b), section 5.
 *   [conv]     prime-rl PR #4073, table "Trainer / vLLM quantization
 *              conventions" (448 denominator, -0 = 0x80, RN cast, FP32
 *              scale containers).
 *   [grouped]  prime-rl PR #4073, "Validation completed" (grouped/empty
 *              experts) and TransformerEngine PR #3573 "Changes" (per-group
 *              GEMM paths).
 *   [po2]      prime-rl PR #4073, conventions table rows "Two-stage
 *              weights", "Activation floors" and "Compact formats" (UE8M0
 *              power-of-two scales, held in FP32 containers on Hopper).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer.  No call allocates, frees, synchronizes or
 *     keeps state between calls; calls are reentrant and thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; the call returns before the work finishes.
 *   - Matrices are row-major with an explicit leading dimension in ELEMENTS
 *     (bf16 = uint16_t bit patterns, E4M3 codes = uint8_t, scales = float).
 *   - Element format: E4M3 = OCP E4M3FN (bias 7, max 448, no infinities,
 *     NaN = S.1111.111, -0 = 0x80 distinct from +0).  Casts round to nearest,
 *     ties to even, and saturate to +-448; the sign of zero is kept.
 *   - Tile quantization of a tile T (128, or 128x128 elements; fewer for a
 *     partial edge tile, over its valid elements only):
 *         a   = max(max_{x in T} |x|, amax_floor)
 *         s   = fl32(a / 448)                        (the stored scale)
 *         inv = (a == 0) ? 0 : min(fl32(448 / a), FLT_MAX)
 *         q   = e4m3(fl32(x * inv))                  (dequant: s * q)
 *     Inputs must be finite; a non-finite input makes its tile unspecified.
 *   - Scale arrays are FP32, one per tile ([conv] "FP32 scale containers"),
 *     laid out block-major: the scales of consecutive rows (or columns) of
 *     one 128-block are contiguous.
 *   - Alignment: bf16 arrays are 16-byte aligned with leading dimensions a
 *     multiple of 8 elements; row-major 1x128 / 128x128 code arrays written
 *     by the quantizers are 8-byte aligned with ld % 8 == 0; transposed code
 *     arrays and every GEMM operand are 16-byte aligned with ld % 16 == 0;
 *     fp32 dW is 16-byte aligned with ld % 4 == 0; scale pointers are 4-byte
 *     aligned.
 *   - Errors: argument errors return a negative fgb_status synchronously and
 *     launch nothing; a launch failure returns FGB_E_HIP.  Faults during
 *     execution surface at the caller's next synchronization (HIP semantics).
 */
#ifndef FGB_H
#define FGB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FGB_OK = 0,
    FGB_E_NULL = -1,        /* a required pointer is NULL                        */
    FGB_E_SHAPE = -2,       /* a dimension is negative or violates a multiple-of rule */
    FGB_E_ALIGN = -3,       /* a pointer or leading dimension is misaligned      */
    FGB_E_LD = -4,          /* a leading dimension is smaller than required     */
    FGB_E_UNSUPPORTED = -5, /* a valid request this library does not implement  */
    FGB_E_HIP = -6,         /* the HIP runtime reported an error at launch      */
    FGB_E_ARG = -7          /* another invalid argument (e.g. a negative floor)  */
} fgb_status;

/* Library version, (major << 16) | (minor << 8) | patch. */
int fgb_version(void);

/* Static description of a status code (never NULL). */
const char* fgb_status_string(int status);

/* ------------------------------------------------------------------------
 * Quantizers  ([scratch]: 1x128 activation / 128x128 weight tiles, Wgrad
 * operands re-tiled 128x1, backward casts emitting both orientations;
 * [drift] section 3 row (a): scale from the in-block absmax, N_c = 128;
 * [conv]: /448, -0 kept, RN cast.)
 * ---------------------------------------------------------------------- */

/* 1x128 tiles of x [R][C] (bf16, leading dim ldx >= C): tile (r, j) covers
 * x[r][128j .. min(128j+128, C)).  Writes the codes q [R][C] (ldq >= C) and
 * the scales s [ceil(C/128)][lds] with s[j*lds + r] the scale of tile (r, j),
 * lds >= R.  Requires C % 8 == 0.  R == 0 or C == 0 is a no-op.
 * amax_floor >= 0 (0 = no floor). */
int fgb_quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       float amax_floor,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds,
                       void* stream);

/* 128x1 tiles of x [R][C] (bf16): tile (i, c) covers column c, rows
 * 128i .. min(128i+128, R).  Writes the codes TRANSPOSED, qT [C][ldqT] with
 * ldqT >= roundup(R, 128): qT[c*ldqT + r] is the code of x[r][c], and the
 * padding qT[c*ldqT + r] for R <= r < roundup(R,128) is 0x00.  Scales
 * sT [ceil(R/128)][ldsT], sT[i*ldsT + c], ldsT >= C.  Equals
 * fgb_quantize_1x128 of x^T.  Requires C % 8 == 0. */
int fgb_quantize_128x1(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       float amax_floor,
                       uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                       void* stream);

/* Both orientations of one tensor from a single read of x [R][C] (bf16):
 * the 1x128 codes and scales of fgb_quantize_1x128 (q [R][ldq], s
 * [ceil(C/128)][lds]) and the 128x1 transposed codes and scales of
 * fgb_quantize_128x1 (qT [C][ldqT] zero padded, sT [ceil(R/128)][ldsT]),
 * bit for bit the same as the two separate calls ([scratch]: backward casts
 * emit both tile orientations of dY, "+T").  Argument rules are those of
 * the two calls; C % 8 == 0. */
int fgb_quantize_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                      float amax_floor,
                      uint8_t* q, int64_t ldq, float* s, int64_t lds,
                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                      void* stream);

/* 128x128 tiles of a weight w [K][N] (bf16, ldw >= N), K and N multiples of
 * 128.  Writes q [K][N] (ldq >= N) and/or its transpose qT [N][K]
 * (ldqT >= K); either may be NULL but not both.  Scales s [K/128][N/128]
 * (dense), s[i*(N/128) + j] for rows 128i.., columns 128j...  One scale grid
 * serves both layouts (a tile's absmax does not depend on orientation). */
int fgb_quantize_128x128(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                         float amax_floor,
                         uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                         float* s, void* stream);

/* E weights at once (the experts of a MoE layer): w [E][K][N] (dense, bf16)
 * -> q [E][K][N] and/or qT [E][N][K] (either may be NULL but not both) and
 * s [E][K/128][N/128], each matrix exactly as fgb_quantize_128x128 quantizes
 * it alone, in one launch.  K and N multiples of 128, 0 <= E <= 65535. */
int fgb_quantize_128x128_batched(int64_t E, const uint16_t* w, int64_t K, int64_t N,
                                 float amax_floor, uint8_t* q, uint8_t* qT, float* s,
                                 void* stream);

/* Re-tile a 1x128-quantized tensor to 128x1 ([scratch]: the Wgrad operand
 * is re-quantized 128x1 from the saved tensor by a small requant box).
 * Input codes q [R][C] (ldq >= C) with scales s [ceil(C/128)][lds],
 * lds >= R, as written by fgb_quantize_1x128.  Each element is dequantized
 * v = fl32(dec(q) * s) and v is quantized with 128x1 tiles exactly as
 * fgb_quantize_128x1 (no floor), writing qT [C][ldqT] (ldqT >=
 * roundup(R,128), zero padded) and sT [ceil(R/128)][ldsT] (ldsT >= C).
 * Requires C % 8 == 0. */
int fgb_requant_128x1(const uint8_t* q, int64_t R, int64_t C, int64_t ldq,
                      const float* s, int64_t lds,
                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                      void* stream);

/* ------------------------------------------------------------------------
 * Stochastic rounding ([sr]: prime-rl PR #4073, conventions row "SR
 * agreement" -- a stateless seed/salt/counter Philox word per element and the
 * lower- or upper-magnitude E4M3 neighbour; the word layout is this
 * library's reading).  Each call below is its round-to-nearest twin with the
 * same arguments, tiles and scales (s = a/448 bit for bit), except the cast:
 *   v = fl32(x * inv), m = |v|; lo, hi = the E4M3 magnitudes with
 *   lo <= m <= hi adjacent on the grid (lo = hi when m is on it);
 *   code = hi when u < (m - lo)/(hi - lo) * 2^32 (real comparison), else lo;
 *   m >= 448 -> 448; the sign of v is kept (-0 too).
 * u, the element's word: element (r, c) of the INPUT tensor (x[r][c] or
 * w[r][c], whatever the output layout) takes word c % 4 of the
 * Philox4x32-10 block with counter (c / 4, r, salt, 0) and key
 * (seed & 0xFFFFFFFF, seed >> 32).  So one element gets the same word in
 * q, qT and in both outputs of the dual call, and equal (seed, salt) give
 * equal codes (calls are deterministic).  Scales are absmax/448 (no _ue8m0
 * twin); there is no stochastic requant.
 * ---------------------------------------------------------------------- */
int fgb_quantize_1x128_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                          float amax_floor,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds,
                          uint64_t seed, uint32_t salt, void* stream);
int fgb_quantize_128x1_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                          float amax_floor,
                          uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                          uint64_t seed, uint32_t salt, void* stream);
int fgb_quantize_dual_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                         float amax_floor,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                         uint64_t seed, uint32_t salt, void* stream);
int fgb_quantize_128x128_sr(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                            float amax_floor,
                            uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                            float* s, uint64_t seed, uint32_t salt, void* stream);

/* ------------------------------------------------------------------------
 * SwiGLU with its casts fused ([scratch], section "What is asserted, and
 * from where": the SwiGLU input is saved as E4M3; a cast rides the nearest
 * vector kernel -- the SwiGLU forward emits the down projection's E4M3
 * operand, the SwiGLU backward emits the gate/up projection's dgrad and
 * wgrad operands in both tile orientations -- and the backward computes in
 * BF16 from the dequantized E4M3 input).
 *
 * The gate/up output is ONE bf16 tensor gu [R][2F] (ldgu >= 2F): G is
 * columns 0..F-1, U columns F..2F-1; F % 128 == 0 so no tile straddles the
 * two halves.  silu(g) = g / (1 + exp(-g)).  Every bf16 result below is the
 * exact real value rounded ONCE to bf16 (to nearest, ties to even), and a
 * zero result carries the sign the product has in IEEE arithmetic (e.g.
 * silu(g) * (+0) = -0 for g < 0); the quantizations are exactly
 * fgb_quantize_1x128 / fgb_quantize_128x1 of the bf16 tensors named.  Inputs
 * and results must be finite.
 * ---------------------------------------------------------------------- */

/* Forward: H = bf16(silu(G) * U) [R][F].  Writes the 1x128 stash of gu
 * (q_gu [R][2F], s_gu [2F/128][lds_gu >= R]; both NULL to skip), the 1x128
 * codes and scales of H (q_h [R][F] with ldq_h >= F, s_h [F/128][lds_h >= R])
 * and H itself (h [R][ldh >= F], 16-byte aligned; NULL to skip). */
int fgb_swiglu_fwd_quant(const uint16_t* gu, int64_t R, int64_t F, int64_t ldgu,
                         float amax_floor,
                         uint8_t* q_gu, int64_t ldq_gu, float* s_gu, int64_t lds_gu,
                         uint8_t* q_h, int64_t ldq_h, float* s_h, int64_t lds_h,
                         uint16_t* h, int64_t ldh, void* stream);

/* Backward, from the stash (q_gu [R][2F], s_gu [2F/128][lds_gu >= R], as
 * written by the forward) and dH [R][F] (bf16, 16-byte aligned):
 *   G~ = bf16(fl32(dec(q_gu[r][c]) * s_gu)), U~ likewise (columns F + c);
 *   dG = bf16(dH * U~ * silu'(G~)), dU = bf16(dH * silu(G~)),
 *   silu'(g) = sigma(g) (1 + g (1 - sigma(g))), sigma(g) = 1 / (1 + exp(-g)).
 * Writes [dG | dU] [R][2F] quantized both ways: 1x128 (q [R][ldq >= 2F],
 * s [2F/128][lds >= R]) and 128x1 (qT [2F][ldqT >= roundup(R,128)] zero
 * padded, sT [ceil(R/128)][ldsT >= 2F]), and optionally [dG | dU] itself
 * (dgu [R][lddgu >= 2F], 16-byte aligned; NULL to skip). */
int fgb_swiglu_bwd_quant(const uint8_t* q_gu, int64_t R, int64_t F, int64_t ldq_gu,
                         const float* s_gu, int64_t lds_gu,
                         const uint16_t* dh, int64_t lddh, float amax_floor,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                         uint16_t* dgu, int64_t lddgu, void* stream);

/* ------------------------------------------------------------------------
 * Power-of-two scales ([po2]).  Each quantizer above has a _ue8m0 twin with
 * the same arguments and layouts whose scales are powers of two:
 *     e = the smallest integer with 448 * 2^e >= a, clamped to [-127, 127]
 *         (an all-zero tile gets -127); s = 2^e (an fp32 holding the UE8M0
 *         value: its exponent field is the E8M0 byte e + 127)
 *     q = e4m3(x * 2^-e)           (exact scaling; |x * 2^-e| <= 448)
 * The requant twin dequantizes with the given power-of-two scales and
 * re-tiles with this rule.
 * ---------------------------------------------------------------------- */
int fgb_quantize_1x128_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                             float amax_floor,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             void* stream);
int fgb_quantize_128x1_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                             float amax_floor,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             void* stream);
int fgb_quantize_dual_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                            float amax_floor,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                            void* stream);
int fgb_quantize_128x128_ue8m0(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                               float amax_floor,
                               uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                               float* s, void* stream);
int fgb_quantize_128x128_batched_ue8m0(int64_t E, const uint16_t* w, int64_t K, int64_t N,
                                       float amax_floor, uint8_t* q, uint8_t* qT, float* s,
                                       void* stream);
int fgb_requant_128x1_ue8m0(const uint8_t* q, int64_t R, int64_t C, int64_t ldq,
                            const float* s, int64_t lds,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                            void* stream);

/* Second stage of the two-stage weight cast ([prime] conventions row
 * "Two-stage weights": the weight's online FP8 cast, then its decoded values
 * requantized to power-of-two scales).  Input: a 128x128-tiled E4M3 weight as
 * fgb_quantize_128x128 writes it, codes q [K][N] (ldq >= N) and fp32 tile
 * scales s [K/128][N/128] (dense).  Each element is dequantized
 * v = fl32(dec(q) * s) and every 128x128 tile of v is requantized with the
 * power-of-two rule above (a = max(absmax, amax_floor)), writing q2 [K][N]
 * (ldq2 >= N) and/or its transpose q2T [N][K] (ldq2T >= K), either may be
 * NULL but not both, and the power-of-two scales s2 [K/128][N/128].  An amax
 * floor of 1e-10 gives the minimum scale 2^-42; flooring the scale itself at
 * 1e-10 (minimum 2^-33) is the floor 448 * 2^-33 here ([prime] row
 * "Activation floors").  K and N multiples of 128; outputs must not overlap
 * the inputs. */
int fgb_requant_128x128_ue8m0(const uint8_t* q, int64_t K, int64_t N, int64_t ldq,
                              const float* s, float amax_floor,
                              uint8_t* q2, int64_t ldq2, uint8_t* q2T, int64_t ldq2T,
                              float* s2, void* stream);

/* ------------------------------------------------------------------------
 * Block-scaled GEMMs ([drift] section 3 rows (a)/(b) and section 5: the
 * partial sum of every 128-long contraction segment is multiplied by
 * s_a * s_b and promoted into an FP32 accumulator; [scratch]: all three
 * GEMMs of a linear in E4M3, Fprop/Dgrad to BF16, Wgrad to FP32).
 * Output BF16 is rounded to nearest even from the FP32 accumulator.
 * Outputs are written with non-temporal stores: they are not left in L2 or
 * the MALL, so a kernel that reads them next fetches them from HBM.
 * ---------------------------------------------------------------------- */

/* Fprop: Y[m][n] = bf16( sum_b sx[b][m] * sw[b][n/128] *
 *                         sum_{k in b} dec(qx[m][k]) * dec(qwT[n][k]) ).
 * qx [M][K] (ldqx >= K), 1x128 scales sx [K/128][ldsx] (ldsx >= M);
 * qwT [N][K] (ldqwT >= K) = W's codes transposed (fgb_quantize_128x128 qT),
 * sw [K/128][N/128] dense; y [M][N] bf16 (ldy >= N).
 * Requires K % 128 == 0 and N % 128 == 0; M is free.  K == 0 writes zeros. */
int fgb_gemm_fprop(int64_t M, int64_t N, int64_t K,
                   const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                   const uint8_t* qwT, int64_t ldqwT, const float* sw,
                   uint16_t* y, int64_t ldy, void* stream);

/* Dgrad: dX[m][k] = bf16( sum_b sdy[b][m] * sw[k/128][b] *
 *                          sum_{n in b} dec(qdy[m][n]) * dec(qw[k][n]) ).
 * qdy [M][N] (ldqdy >= N), 1x128 scales sdy [N/128][ldsdy] (ldsdy >= M);
 * qw [K][N] (ldqw >= N) = W's codes (fgb_quantize_128x128 q), sw [K/128][N/128];
 * dx [M][K] bf16 (lddx >= K).  The 128x128 weight tiles are reused
 * transposed.  Requires K % 128 == 0 and N % 128 == 0. */
int fgb_gemm_dgrad(int64_t M, int64_t K, int64_t N,
                   const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy,
                   const uint8_t* qw, int64_t ldqw, const float* sw,
                   uint16_t* dx, int64_t lddx, void* stream);

/* Wgrad: dW[k][n] (W's [K][N] shape, i.e. (dY^T X)^T) =
 *     (accumulate ? dW[k][n] : 0) + sum_b sxT[b][k] * sdyT[b][n] *
 *                                   sum_{m in b} dec(qxT[k][m]) * dec(qdyT[n][m])
 * over b < ceil(M/128).  qxT [K][ldqxT] and qdyT [N][ldqdyT] are 128x1
 * operands (fgb_requant_128x1 / fgb_quantize_128x1) with
 * ld >= roundup(M,128) and zero padding beyond M; sxT [ceil(M/128)][ldsxT]
 * (ldsxT >= K), sdyT [ceil(M/128)][ldsdyT] (ldsdyT >= N); dw [K][N] fp32
 * (lddw >= N).  Requires K % 128 == 0 and N % 128 == 0; M == 0 writes zeros
 * (or leaves dW unchanged when accumulating). */
int fgb_gemm_wgrad(int64_t K, int64_t N, int64_t M,
                   const uint8_t* qxT, int64_t ldqxT, const float* sxT, int64_t ldsxT,
                   const uint8_t* qdyT, int64_t ldqdyT, const float* sdyT, int64_t ldsdyT,
                   float* dw, int64_t lddw, int accumulate, void* stream);

/* ------------------------------------------------------------------------
 * Grouped (MoE expert) GEMMs ([grouped]).  Rows are grouped per expert in
 * segments [offsets[e], offsets[e+1]) of a padded tensor with R_pad rows;
 * every offset is a multiple of 128, offsets[0] == 0, offsets are
 * non-decreasing and offsets[E] <= R_pad; rows of a segment beyond the
 * expert's tokens are zero.  With that layout, fgb_quantize_1x128 and
 * fgb_quantize_128x1 over the whole padded tensor equal per-expert
 * quantization, so no grouped quantizer is needed.  `offsets` is a DEVICE
 * array of E+1 int32, read by the kernels (no host synchronization).  All
 * operands are dense (leading dimension = row length).  Rows at or beyond
 * offsets[E] are not written.  0 <= E <= 65535 (else FGB_E_SHAPE).  The
 * kernels address an operand with 32-bit byte offsets: the token-side
 * operand (all R_pad rows of qx or qdy, or the K or N rows of qxT or qdyT)
 * and one expert's weight must each end within 4 GiB of their base, else
 * FGB_E_UNSUPPORTED (nothing is launched).
 * ---------------------------------------------------------------------- */

/* Y[r] = X[r] W_e for rows r of segment e.  qx [R_pad][K], sx [K/128][R_pad],
 * qwT [E][N][K], sw [E][K/128][N/128], y [R_pad][N] bf16. */
int fgb_gemm_fprop_grouped(int64_t E, const int32_t* offsets, int64_t R_pad,
                           int64_t N, int64_t K,
                           const uint8_t* qx, const float* sx,
                           const uint8_t* qwT, const float* sw,
                           uint16_t* y, void* stream);

/* dX[r] = dY[r] W_e^T for rows r of segment e.  qdy [R_pad][N],
 * sdy [N/128][R_pad], qw [E][K][N], sw [E][K/128][N/128], dx [R_pad][K] bf16. */
int fgb_gemm_dgrad_grouped(int64_t E, const int32_t* offsets, int64_t R_pad,
                           int64_t K, int64_t N,
                           const uint8_t* qdy, const float* sdy,
                           const uint8_t* qw, const float* sw,
                           uint16_t* dx, void* stream);

/* dW_e = X_e^T dY_e over the rows of segment e (contraction blocks
 * offsets[e]/128 .. offsets[e+1]/128).  qxT [K][R_pad], sxT [R_pad/128][K],
 * qdyT [N][R_pad], sdyT [R_pad/128][N], dw [E][K][N] fp32.  An empty expert
 * gets dW_e = 0 (unchanged when accumulating).  R_pad % 128 == 0. */
int fgb_gemm_wgrad_grouped(int64_t E, const int32_t* offsets, int64_t R_pad,
                           int64_t K, int64_t N,
                           const uint8_t* qxT, const float* sxT,
                           const uint8_t* qdyT, const float* sdyT,
                           float* dw, int accumulate, void* stream);

/* ------------------------------------------------------------------------
 * GEMMs on power-of-two scales ([po2]; [drift] section 5).  Same arguments,
 * layouts and results as the GEMMs above, for operands quantized by the
 * _ue8m0 quantizers: EVERY scale must be an exact power of two (2^-127 ..
 * 2^127).  The matrix core applies the scales (its E8M0 block-scale operands
 * are the fp32 exponent fields) and adds each 128-block's partial sums into
 * the FP32 accumulator with round-to-nearest-even adds, so the per-block
 * promotion happens inside the matrix core.  A scale that is not a power of
 * two gives a wrong result (only its exponent field is used).
 * ---------------------------------------------------------------------- */
int fgb_gemm_fprop_ue8m0(int64_t M, int64_t N, int64_t K,
                         const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                         const uint8_t* qwT, int64_t ldqwT, const float* sw,
                         uint16_t* y, int64_t ldy, void* stream);
int fgb_gemm_dgrad_ue8m0(int64_t M, int64_t K, int64_t N,
                         const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy,
                         const uint8_t* qw, int64_t ldqw, const float* sw,
                         uint16_t* dx, int64_t lddx, void* stream);
int fgb_gemm_wgrad_ue8m0(int64_t K, int64_t N, int64_t M,
                         const uint8_t* qxT, int64_t ldqxT, const float* sxT, int64_t ldsxT,
                         const uint8_t* qdyT, int64_t ldqdyT, const float* sdyT, int64_t ldsdyT,
                         float* dw, int64_t lddw, int accumulate, void* stream);
int fgb_gemm_fprop_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad,
                                 int64_t N, int64_t K,
                                 const uint8_t* qx, const float* sx,
                                 const uint8_t* qwT, const float* sw,
                                 uint16_t* y, void* stream);
int fgb_gemm_dgrad_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad,
                                 int64_t K, int64_t N,
                                 const uint8_t* qdy, const float* sdy,
                                 const uint8_t* qw, const float* sw,
                                 uint16_t* dx, void* stream);
int fgb_gemm_wgrad_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad,
                                 int64_t K, int64_t N,
                                 const uint8_t* qxT, const float* sxT,
                                 const uint8_t* qdyT, const float* sdyT,
                                 float* dw, int accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FGB_H */
