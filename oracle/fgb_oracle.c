/*
 * Plain CPU oracle for the fine-grained FP8 linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the GPU library, and the GPU
 * library never calls it.
 *
 * Everything here is written for a reader to check against the method by
 * eye: one element, one tile, one output at a time, in double precision
 * wherever the method leaves the precision free.  Sources, by page:
 *
 *  - "scratch: the backward pass, unrolled" (deepseek-v3.ezyang.com),
 *    section "What is asserted, and from where": all three GEMMs of a
 *    linear take E4M3 operands with 1x128 activation tiles and 128x128
 *    weight tiles and FP32-promoted accumulation; Fprop/Dgrad write BF16,
 *    Wgrad writes FP32; the Wgrad operands are re-tiled 128x1 from the
 *    saved tensors.
 *  - "FP8 dynamic quantization partial-sum drift" (foosynaptic deepseek
 *    tech notes), section 3 table row (a): per-block dynamic scales from the
 *    in-block absmax, N_c = 128, partial sums multiplied by s_x*s_w; row (b)
 *    and section 5: the partial sum of each 128-long segment is promoted
 *    into an FP32 accumulator.
 *  - prime-rl PR #4073, table "Trainer / vLLM quantization conventions":
 *    scale denominator 448, negative zero 0x80 kept distinct from +0,
 *    round-to-nearest online cast, FP32 scale containers on Hopper.
 *
 * The E4M3 element format is OCP E4M3FN (bias 7, no infinities, NaN =
 * S.1111.111, largest finite 448): the only variant with both the 448 bound
 * and a distinct -0 = 0x80 that the prime-rl conventions table states.
 *
 * Readings where the pages are silent (each is restated in the design
 * notes): ties round to even; |x| > 448 saturates to +-448; the cast
 * multiplies by fl32(448/amax) (one division per tile); an all-zero tile
 * gets scale +0 and codes +-0; a partial edge tile takes the absmax over
 * its valid elements; an optional amax floor is applied before /448.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_TILE 128

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest integer, ties to the even integer. */
static double rne_integer(double x)
{
    double lo = floor(x);
    double frac = x - lo; /* exact for |x| < 2^52 */
    if (frac > 0.5) return lo + 1.0;
    if (frac < 0.5) return lo;
    return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
}

/* E4M3FN decode: S EEEE MMM with bias 7.
 *   E == 0           -> (-1)^S * M * 2^-9              (subnormal, includes +-0)
 *   E == 15, M == 7  -> NaN
 *   otherwise        -> (-1)^S * (1 + M/8) * 2^(E-7)                         */
double orc_e4m3_decode(uint8_t u)
{
    int sign = (u >> 7) & 1;
    int e = (u >> 3) & 15;
    int m = u & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = (double)m * ldexp(1.0, -9);
    else
        mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
    return sign ? -mag : mag;
}

/* E4M3FN encode of one fp32 value: round to nearest, ties to even;
 * magnitudes above 448 (and infinities) saturate to 448; NaN -> S.1111.111;
 * the sign bit of the input is always kept, so -0 and negative values that
 * round to zero give 0x80. */
uint8_t orc_e4m3_encode(float f)
{
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (isnan(f)) return sign | 0x7F;
    if (a > 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: integer multiples of 2^-9; 8 * 2^-9 is the
         * smallest normal 2^-6 whose code is 0x08, so m = 8 needs no carry */
        double m = rne_integer(a * 512.0);
        return sign | (uint8_t)m;
    }
    int e2;
    frexp(a, &e2);       /* a = f * 2^e2, f in [0.5, 1) */
    int ex = e2 - 1;     /* a in [2^ex, 2^(ex+1)) */
    double m = rne_integer((a / ldexp(1.0, ex) - 1.0) * 8.0);
    if (m == 8.0) {      /* rounding carried into the next binade */
        m = 0.0;
        ex += 1;
    }
    return sign | (uint8_t)(((ex + 7) << 3) | (int)m);
}

/* bfloat16 (8 significant bits, fp32 exponent range) -> float: exact. */
float orc_bf16_to_float(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Round a double to bfloat16, to nearest with ties to even, in one step. */
uint16_t orc_bf16_round(double r)
{
    uint16_t sign = signbit(r) ? 0x8000 : 0x0000;
    double a = fabs(r);
    if (isnan(r)) return sign | 0x7FC0;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;             /* a in [2^ex, 2^(ex+1)) */
    if (ex < -126) ex = -126;    /* subnormal bf16: quantum 2^-133 */
    double ulp = ldexp(1.0, ex - 7);
    double v = rne_integer(a / ulp) * ulp;
    if (v >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow -> Inf */
    float fv = (float)v;         /* exact: v has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &fv, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

/* ------------------------------------------------------------------ */
/* One tile of dynamic quantization                                    */
/* ------------------------------------------------------------------ */

/* Quantize the n fp32 values of one tile.
 *   a   = max |v|                        (exact)
 *   a'  = max(a, amax_floor)
 *   s   = fl32(a' / 448)                 (stored scale; dequant = s * dec(q))
 *   inv = a' == 0 ? 0 : min(fl32(448 / a'), FLT_MAX)
 *   q_i = enc(fl32(v_i * inv))
 * A NaN anywhere in the tile makes a NaN: the pages say nothing about
 * NaN; read here as propagating it to the scale (the quiet NaN) and to every
 * code of the tile (the E4M3 NaN 0x7F), so that it reaches the GEMM.    */
static void quantize_tile(const float* v, int64_t n, float amax_floor,
                          float* s_out, uint8_t* q_out)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float av = fabsf(v[i]);
        if (isnan(av) || av > a) a = av;
        if (isnan(a)) break;
    }
    if (isnan(a)) {
        *s_out = NAN;
        for (int64_t i = 0; i < n; ++i) q_out[i] = 0x7F;
        return;
    }
    if (amax_floor > a) a = amax_floor;
    float s = a / 448.0f;
    float inv;
    if (a == 0.0f) {
        inv = 0.0f;
    } else {
        inv = 448.0f / a;
        if (inv > FLT_MAX) inv = FLT_MAX;
    }
    *s_out = s;
    for (int64_t i = 0; i < n; ++i) {
        float t = v[i] * inv;
        /* t is NaN only for an infinite element of an infinite tile (Inf * 0): the
         * sign of that NaN is not fixed by IEEE arithmetic; it encodes as 0x7F */
        q_out[i] = isnan(t) ? 0x7F : orc_e4m3_encode(t);
    }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* 1x128 tiling of a row-major bf16 matrix x[R][C] (leading dim ldx):
 * tile (r, j) is x[r][128j .. min(128j+128, C)).
 * q[r][c] (leading dim ldq) holds the codes; s[j][r] (leading dim lds)
 * the scale of tile (r, j).                                           */
void orc_quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                        float amax_floor, uint8_t* q, int64_t ldq,
                        float* s, int64_t lds)
{
    int64_t nb = ceil_div(C, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        float v[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t j = 0; j < nb; ++j) {
            int64_t c0 = j * ORC_TILE;
            int64_t n = (C - c0 < ORC_TILE) ? C - c0 : ORC_TILE;
            for (int64_t i = 0; i < n; ++i) v[i] = orc_bf16_to_float(x[r * ldx + c0 + i]);
            quantize_tile(v, n, amax_floor, &s[j * lds + r], code);
            for (int64_t i = 0; i < n; ++i) q[r * ldq + c0 + i] = code[i];
        }
    }
}

/* 128x1 tiling of x[R][C]: tile (i, c) is column c, rows 128i .. min(128i+128, R).
 * The codes are written transposed, qT[c][r] (leading dim ldqT >= roundup(R,128)),
 * with qT[c][r] = 0x00 for R <= r < roundup(R,128); sT[i][c] (leading dim ldsT)
 * holds the scale of tile (i, c).                                      */
static void quantize_128x1_f32(const float* xf, int64_t R, int64_t C, int64_t ldxf,
                               float amax_floor, uint8_t* qT, int64_t ldqT,
                               float* sT, int64_t ldsT)
{
    int64_t nb = ceil_div(R, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float v[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t i = 0; i < nb; ++i) {
            int64_t r0 = i * ORC_TILE;
            int64_t n = (R - r0 < ORC_TILE) ? R - r0 : ORC_TILE;
            for (int64_t k = 0; k < n; ++k) v[k] = xf[(r0 + k) * ldxf + c];
            quantize_tile(v, n, amax_floor, &sT[i * ldsT + c], code);
            for (int64_t k = 0; k < ORC_TILE; ++k)
                qT[c * ldqT + r0 + k] = (k < n) ? code[k] : 0x00;
        }
    }
}

void orc_quantize_128x1(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                        float amax_floor, uint8_t* qT, int64_t ldqT,
                        float* sT, int64_t ldsT)
{
    float* xf = (float*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) xf[r * C + c] = orc_bf16_to_float(x[r * ldx + c]);
    quantize_128x1_f32(xf, R, C, C, amax_floor, qT, ldqT, sT, ldsT);
    free(xf);
}

/* 128x128 tiling of a weight w[K][N] (K, N multiples of 128 not required
 * here; edge tiles take the absmax over their valid elements).  Writes
 * q[k][n] (if q != NULL), its transpose qT[n][k] (if qT != NULL) and
 * s[i][j] = scale of tile (rows 128i.., cols 128j..), row length ceil(N/128). */
void orc_quantize_128x128(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                          float amax_floor, uint8_t* q, int64_t ldq,
                          uint8_t* qT, int64_t ldqT, float* s)
{
    int64_t kb = ceil_div(K, ORC_TILE), nb = ceil_div(N, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < kb * nb; ++t) {
        int64_t i = t / nb, j = t % nb;
        int64_t k0 = i * ORC_TILE, n0 = j * ORC_TILE;
        int64_t kn = (K - k0 < ORC_TILE) ? K - k0 : ORC_TILE;
        int64_t nn = (N - n0 < ORC_TILE) ? N - n0 : ORC_TILE;
        float v[ORC_TILE * ORC_TILE];
        uint8_t code[ORC_TILE * ORC_TILE];
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b)
                v[a * nn + b] = orc_bf16_to_float(w[(k0 + a) * ldw + n0 + b]);
        quantize_tile(v, kn * nn, amax_floor, &s[i * nb + j], code);
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b) {
                if (q) q[(k0 + a) * ldq + n0 + b] = code[a * nn + b];
                if (qT) qT[(n0 + b) * ldqT + k0 + a] = code[a * nn + b];
            }
    }
}

/* Re-tile a 1x128-quantized tensor (codes q[R][C], scales s[ceil(C/128)][R])
 * to 128x1: dequantize v = fl32(dec(q) * s) (one fp32 rounding), then
 * quantize v with 128x1 tiles exactly as orc_quantize_128x1 does.      */
void orc_requant_128x1(const uint8_t* q, int64_t R, int64_t C, int64_t ldq,
                       const float* s, int64_t lds,
                       uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT)
{
    float* v = (float*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            double d = orc_e4m3_decode(q[r * ldq + c]);
            float sc = s[(c / ORC_TILE) * lds + r];
            v[r * C + c] = (float)(d * (double)sc); /* exact product, one rounding */
        }
    quantize_128x1_f32(v, R, C, C, 0.0f, qT, ldqT, sT, ldsT);
    free(v);
}

/* ------------------------------------------------------------------ */
/* Power-of-two (UE8M0) scale variant                                  */
/* ------------------------------------------------------------------ */

/* One tile with a power-of-two scale (prime-rl PR #4073, "Results": the
 * power-of-two / UE8M0 scale format and its two-stage requant; the pages fix
 * no rounding direction, read here as rounding the scale up):
 *   a   = max |v|, a' = max(a, amax_floor)
 *   e   = the smallest integer with 448 * 2^e >= a', clamped to [-127, 127]
 *         (an all-zero tile gets -127); stored as the byte e + 127, the E8M0
 *         encoding of 2^e
 *   q_i = enc(fl32(v_i * 2^-e))
 * The scaled values never exceed 448 in magnitude, so no code saturates
 * unless e was clamped.  A NaN in the tile stores the E8M0 NaN byte 0xFF. */
static void quantize_tile_ue8m0(const float* v, int64_t n, float amax_floor,
                                uint8_t* e_out, uint8_t* q_out)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float av = fabsf(v[i]);
        if (isnan(av) || av > a) a = av;
        if (isnan(a)) break;
    }
    if (amax_floor > a) a = amax_floor;
    if (isnan(a)) {
        *e_out = 0xFF;
        for (int64_t i = 0; i < n; ++i) q_out[i] = 0x7F;
        return;
    }
    int e = -127;
    while (e < 127 && ldexp(448.0, e) < (double)a) ++e;
    *e_out = (uint8_t)(e + 127);
    const double m = ldexp(1.0, -e);
    for (int64_t i = 0; i < n; ++i) q_out[i] = orc_e4m3_encode((float)((double)v[i] * m));
}

/* E8M0 byte -> the scale 2^(byte - 127); 0xFF is NaN. */
double orc_e8m0_decode(uint8_t b)
{
    return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127);
}

/* As orc_quantize_1x128, with the UE8M0 rule; e[j*lde + r] is the byte of tile (r, j). */
void orc_quantize_1x128_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                              float amax_floor, uint8_t* q, int64_t ldq,
                              uint8_t* e, int64_t lde)
{
    int64_t nb = ceil_div(C, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        float v[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t j = 0; j < nb; ++j) {
            int64_t c0 = j * ORC_TILE;
            int64_t n = (C - c0 < ORC_TILE) ? C - c0 : ORC_TILE;
            for (int64_t i = 0; i < n; ++i) v[i] = orc_bf16_to_float(x[r * ldx + c0 + i]);
            quantize_tile_ue8m0(v, n, amax_floor, &e[j * lde + r], code);
            for (int64_t i = 0; i < n; ++i) q[r * ldq + c0 + i] = code[i];
        }
    }
}

/* As quantize_128x1_f32, with the UE8M0 rule. */
static void quantize_128x1_f32_ue8m0(const float* xf, int64_t R, int64_t C, int64_t ldxf,
                                     float amax_floor, uint8_t* qT, int64_t ldqT,
                                     uint8_t* eT, int64_t ldeT)
{
    int64_t nb = ceil_div(R, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float v[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t i = 0; i < nb; ++i) {
            int64_t r0 = i * ORC_TILE;
            int64_t n = (R - r0 < ORC_TILE) ? R - r0 : ORC_TILE;
            for (int64_t k = 0; k < n; ++k) v[k] = xf[(r0 + k) * ldxf + c];
            quantize_tile_ue8m0(v, n, amax_floor, &eT[i * ldeT + c], code);
            for (int64_t k = 0; k < ORC_TILE; ++k)
                qT[c * ldqT + r0 + k] = (k < n) ? code[k] : 0x00;
        }
    }
}

void orc_quantize_128x1_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                              float amax_floor, uint8_t* qT, int64_t ldqT,
                              uint8_t* eT, int64_t ldeT)
{
    float* xf = (float*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) xf[r * C + c] = orc_bf16_to_float(x[r * ldx + c]);
    quantize_128x1_f32_ue8m0(xf, R, C, C, amax_floor, qT, ldqT, eT, ldeT);
    free(xf);
}

/* As orc_quantize_128x128, with the UE8M0 rule; e[i*ceil(N/128) + j]. */
void orc_quantize_128x128_ue8m0(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                                float amax_floor, uint8_t* q, int64_t ldq,
                                uint8_t* qT, int64_t ldqT, uint8_t* e)
{
    int64_t kb = ceil_div(K, ORC_TILE), nb = ceil_div(N, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < kb * nb; ++t) {
        int64_t i = t / nb, j = t % nb;
        int64_t k0 = i * ORC_TILE, n0 = j * ORC_TILE;
        int64_t kn = (K - k0 < ORC_TILE) ? K - k0 : ORC_TILE;
        int64_t nn = (N - n0 < ORC_TILE) ? N - n0 : ORC_TILE;
        float v[ORC_TILE * ORC_TILE];
        uint8_t code[ORC_TILE * ORC_TILE];
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b)
                v[a * nn + b] = orc_bf16_to_float(w[(k0 + a) * ldw + n0 + b]);
        quantize_tile_ue8m0(v, kn * nn, amax_floor, &e[i * nb + j], code);
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b) {
                if (q) q[(k0 + a) * ldq + n0 + b] = code[a * nn + b];
                if (qT) qT[(n0 + b) * ldqT + k0 + a] = code[a * nn + b];
            }
    }
}

/* Re-tile a UE8M0 1x128 tensor (codes q [R][C], bytes e [ceil(C/128)][R]) to
 * 128x1: v = fl32(dec(q) * 2^(e-127)) (exact: a 4-bit significand times a
 * power of two), then the UE8M0 128x1 rule on v. */
void orc_requant_128x1_ue8m0(const uint8_t* q, int64_t R, int64_t C, int64_t ldq,
                             const uint8_t* e, int64_t lde,
                             uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT)
{
    float* v = (float*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            double d = orc_e4m3_decode(q[r * ldq + c]);
            double sc = orc_e8m0_decode(e[(c / ORC_TILE) * lde + r]);
            v[r * C + c] = (float)(d * sc);
        }
    quantize_128x1_f32_ue8m0(v, R, C, C, 0.0f, qT, ldqT, eT, ldeT);
    free(v);
}

/* Second stage of the two-stage weight cast (prime-rl PR #4073 conventions
 * table, row "Two-stage weights": the online FP8 cast of a weight, then its
 * decoded values requantized to power-of-two scales).  Input: a 128x128-tiled
 * E4M3 weight, codes q [K][N] and fp32 tile scales s[i*ceil(N/128) + j] as
 * orc_quantize_128x128 writes them.  Each element is dequantized
 * v = fl32(dec(q) * s) (one rounding of the exact product) and the tiles of v
 * are requantized with the UE8M0 rule (same 128x128 tiles), writing q2 and/or
 * its transpose q2T and the bytes e[i*ceil(N/128) + j]. */
void orc_requant_128x128_ue8m0(const uint8_t* q, int64_t K, int64_t N, int64_t ldq,
                               const float* s, float amax_floor,
                               uint8_t* q2, int64_t ldq2, uint8_t* q2T, int64_t ldq2T, uint8_t* e)
{
    int64_t kb = ceil_div(K, ORC_TILE), nb = ceil_div(N, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < kb * nb; ++t) {
        int64_t i = t / nb, j = t % nb;
        int64_t k0 = i * ORC_TILE, n0 = j * ORC_TILE;
        int64_t kn = (K - k0 < ORC_TILE) ? K - k0 : ORC_TILE;
        int64_t nn = (N - n0 < ORC_TILE) ? N - n0 : ORC_TILE;
        float v[ORC_TILE * ORC_TILE];
        uint8_t code[ORC_TILE * ORC_TILE];
        const double sc = (double)s[i * nb + j];
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b)
                v[a * nn + b] = (float)(orc_e4m3_decode(q[(k0 + a) * ldq + n0 + b]) * sc);
        quantize_tile_ue8m0(v, kn * nn, amax_floor, &e[i * nb + j], code);
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b) {
                if (q2) q2[(k0 + a) * ldq2 + n0 + b] = code[a * nn + b];
                if (q2T) q2T[(n0 + b) * ldq2T + k0 + a] = code[a * nn + b];
            }
    }
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM                                                   */
/* ------------------------------------------------------------------ */

/* out[i][j] = sum_b  SA(i,b) * SB(j,b) * S_b(i,j),
 *   S_b(i,j) = sum_{t in block b, t < K} dec(A[i][t]) * dec(B[j][t])
 * with blocks of 128 along the contraction index t.  Both operands are
 * stored contraction-contiguous: A[i][t] = A[i*lda + t], B[j][t] = B[j*ldb + t].
 * Scales: SA(i,b) = sa[b*sa_sb + (i/sa_group)*sa_si], likewise SB.
 *
 * Every E4M3 value is an integer multiple of 2^-9 below 2^9, so every
 * product is a multiple of 2^-18 below 2^18 and a 128-term S_b is exact
 * in double.  The sum over blocks is in double (error ~1e-16 * aabs).
 * aabs[i][j] = sum_b |SA*SB| * sum_t |dec*dec| bounds cancellation.
 *
 * Only the sub-grid rows[0..nrows) x cols[0..ncols) is computed; out and
 * aabs are [nrows][ncols].                                           */
void orc_gemm_block_scaled(int64_t K,
                           const uint8_t* A, int64_t lda,
                           const float* sa, int64_t sa_sb, int64_t sa_si, int64_t sa_group,
                           const uint8_t* B, int64_t ldb,
                           const float* sb, int64_t sb_sb, int64_t sb_sj, int64_t sb_group,
                           const int64_t* rows, int64_t nrows,
                           const int64_t* cols, int64_t ncols,
                           double* out, double* aabs)
{
    double dec[256];
    for (int u = 0; u < 256; ++u) dec[u] = orc_e4m3_decode((uint8_t)u);
    int64_t nblk = ceil_div(K, ORC_TILE);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows[ii];
        for (int64_t jj = 0; jj < ncols; ++jj) {
            int64_t j = cols[jj];
            double r = 0.0, ra = 0.0;
            for (int64_t b = 0; b < nblk; ++b) {
                double sblk = 0.0, sabs = 0.0;
                int64_t t0 = b * ORC_TILE;
                int64_t t1 = (t0 + ORC_TILE < K) ? t0 + ORC_TILE : K;
                for (int64_t t = t0; t < t1; ++t) {
                    double p = dec[A[i * lda + t]] * dec[B[j * ldb + t]];
                    sblk += p;
                    sabs += fabs(p);
                }
                double scale = (double)sa[b * sa_sb + (i / sa_group) * sa_si] *
                               (double)sb[b * sb_sb + (j / sb_group) * sb_sj];
                r += scale * sblk;
                ra += fabs(scale) * sabs;
            }
            out[ii * ncols + jj] = r;
            aabs[ii * ncols + jj] = ra;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Vector helpers for the tests (one call per element, no shortcuts)   */
/* ------------------------------------------------------------------ */

void orc_e4m3_encode_array(const float* f, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(f[i]);
}

/* Encode the fp32 values whose bit patterns are start, start+1, ..., start+n-1. */
void orc_e4m3_encode_bits_range(uint32_t start, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits = start + (uint32_t)i;
        float f;
        memcpy(&f, &bits, sizeof f);
        out[i] = orc_e4m3_encode(f);
    }
}

void orc_e4m3_decode_array(const uint8_t* u, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(u[i]);
}

void orc_bf16_round_array(const double* r, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(r[i]);
}

/* Thread count for the OpenMP loops that follow (n >= 1); benchmark plumbing only. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding (SR)                                            */
/* ------------------------------------------------------------------ */
/*
 * prime-rl PR #4073, conventions row "SR agreement": SR draws from a
 * stateless seed / salt / counter contract through a Philox helper and picks
 * the lower- or upper-magnitude neighbour; the exact contract lives in a PR
 * the pages do not include.  Reading used here:
 *
 *  - random word: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 *    numbers: as easy as 1, 2, 3", SC'11) with key (seed mod 2^32,
 *    seed div 2^32) and counter (c div 4, r, salt, 0) for the element at row r,
 *    column c of the tensor being quantized (the source tensor, whatever the
 *    output layout); the element takes word c mod 4 of the output block;
 *  - the tile scale is the round-to-nearest quantizer's (s = a'/448, the same
 *    v = fl32(x * inv)); only the final cast changes;
 *  - with m = |v|, lo = the largest E4M3 magnitude <= m and hi = the smallest
 *    E4M3 magnitude >= m, the cast takes hi when u < (m - lo)/(hi - lo) * 2^32
 *    (u the 32-bit word, compared as real numbers) and lo otherwise, so
 *    P(hi) = (m - lo)/(hi - lo) up to 2^-32 and E[dec(q)] = v; m >= 448
 *    saturates to 448, NaN gives S.1111.111, the sign of v is kept (-0 too).
 */

/* One Philox4x32-10 block: ten rounds of the two 32x32 -> 64-bit products
 * with multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl
 * constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The random word of element (r, c) under (seed, salt). */
uint32_t orc_sr_word(uint64_t seed, uint32_t salt, int64_t r, int64_t c)
{
    uint32_t ctr[4] = {(uint32_t)(c / 4), (uint32_t)r, salt, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[c % 4];
}

/* The 127 finite non-negative E4M3 magnitudes in increasing order (codes
 * 0x00 .. 0x7E decode to increasing values). */
static double e4m3_magnitude(int code) { return orc_e4m3_decode((uint8_t)code); }

/* E4M3 code of v under stochastic rounding with random word u. */
uint8_t orc_e4m3_encode_sr(float v, uint32_t u)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    double m = fabs((double)v);
    if (m >= 448.0) return sign | 0x7E;
    /* lo: largest code whose magnitude is <= m (binary search over 0..0x7E) */
    int a = 0, b = 0x7E;          /* invariant: mag(a) <= m < mag(b) */
    while (b - a > 1) {
        int mid = (a + b) / 2;
        if (e4m3_magnitude(mid) <= m) a = mid; else b = mid;
    }
    double lo = e4m3_magnitude(a);
    if (lo == m) return sign | (uint8_t)a;
    double hi = e4m3_magnitude(a + 1);
    double frac = (m - lo) / (hi - lo);              /* exact: hi - lo is a power of two */
    int up = (double)u < frac * 4294967296.0;        /* exact comparison in double */
    return sign | (uint8_t)(up ? a + 1 : a);
}

/* One tile as quantize_tile, with the SR cast; u[i] is element i's word.
 * A NaN tile as in quantize_tile.                                      */
static void quantize_tile_sr(const float* v, const uint32_t* u, int64_t n, float amax_floor,
                             float* s_out, uint8_t* q_out)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float av = fabsf(v[i]);
        if (isnan(av) || av > a) a = av;
        if (isnan(a)) break;
    }
    if (isnan(a)) {
        *s_out = NAN;
        for (int64_t i = 0; i < n; ++i) q_out[i] = 0x7F;
        return;
    }
    if (amax_floor > a) a = amax_floor;
    float s = a / 448.0f;
    float inv;
    if (a == 0.0f) {
        inv = 0.0f;
    } else {
        inv = 448.0f / a;
        if (inv > FLT_MAX) inv = FLT_MAX;
    }
    *s_out = s;
    for (int64_t i = 0; i < n; ++i) {
        float t = v[i] * inv;
        q_out[i] = isnan(t) ? 0x7F : orc_e4m3_encode_sr(t, u[i]);      /* Inf * 0: as quantize_tile */
    }
}

/* As orc_quantize_1x128 with the SR cast. */
void orc_quantize_1x128_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                           float amax_floor, uint8_t* q, int64_t ldq,
                           float* s, int64_t lds, uint64_t seed, uint32_t salt)
{
    int64_t nb = ceil_div(C, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        float v[ORC_TILE];
        uint32_t u[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t j = 0; j < nb; ++j) {
            int64_t c0 = j * ORC_TILE;
            int64_t n = (C - c0 < ORC_TILE) ? C - c0 : ORC_TILE;
            for (int64_t i = 0; i < n; ++i) {
                v[i] = orc_bf16_to_float(x[r * ldx + c0 + i]);
                u[i] = orc_sr_word(seed, salt, r, c0 + i);
            }
            quantize_tile_sr(v, u, n, amax_floor, &s[j * lds + r], code);
            for (int64_t i = 0; i < n; ++i) q[r * ldq + c0 + i] = code[i];
        }
    }
}

/* As orc_quantize_128x1 with the SR cast; element (r, c) of x draws word (r, c). */
void orc_quantize_128x1_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                           float amax_floor, uint8_t* qT, int64_t ldqT,
                           float* sT, int64_t ldsT, uint64_t seed, uint32_t salt)
{
    int64_t nb = ceil_div(R, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float v[ORC_TILE];
        uint32_t u[ORC_TILE];
        uint8_t code[ORC_TILE];
        for (int64_t i = 0; i < nb; ++i) {
            int64_t r0 = i * ORC_TILE;
            int64_t n = (R - r0 < ORC_TILE) ? R - r0 : ORC_TILE;
            for (int64_t k = 0; k < n; ++k) {
                v[k] = orc_bf16_to_float(x[(r0 + k) * ldx + c]);
                u[k] = orc_sr_word(seed, salt, r0 + k, c);
            }
            quantize_tile_sr(v, u, n, amax_floor, &sT[i * ldsT + c], code);
            for (int64_t k = 0; k < ORC_TILE; ++k)
                qT[c * ldqT + r0 + k] = (k < n) ? code[k] : 0x00;
        }
    }
}

/* As orc_quantize_128x128 with the SR cast; element (k, n) of w draws word (k, n),
 * and q and qT hold the same codes. */
void orc_quantize_128x128_sr(const uint16_t* w, int64_t K, int64_t N, int64_t ldw,
                             float amax_floor, uint8_t* q, int64_t ldq,
                             uint8_t* qT, int64_t ldqT, float* s, uint64_t seed, uint32_t salt)
{
    int64_t kb = ceil_div(K, ORC_TILE), nb = ceil_div(N, ORC_TILE);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < kb * nb; ++t) {
        int64_t i = t / nb, j = t % nb;
        int64_t k0 = i * ORC_TILE, n0 = j * ORC_TILE;
        int64_t kn = (K - k0 < ORC_TILE) ? K - k0 : ORC_TILE;
        int64_t nn = (N - n0 < ORC_TILE) ? N - n0 : ORC_TILE;
        float* v = (float*)malloc(sizeof(float) * ORC_TILE * ORC_TILE);
        uint32_t* u = (uint32_t*)malloc(sizeof(uint32_t) * ORC_TILE * ORC_TILE);
        uint8_t* code = (uint8_t*)malloc(ORC_TILE * ORC_TILE);
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b) {
                v[a * nn + b] = orc_bf16_to_float(w[(k0 + a) * ldw + n0 + b]);
                u[a * nn + b] = orc_sr_word(seed, salt, k0 + a, n0 + b);
            }
        quantize_tile_sr(v, u, kn * nn, amax_floor, &s[i * nb + j], code);
        for (int64_t a = 0; a < kn; ++a)
            for (int64_t b = 0; b < nn; ++b) {
                if (q) q[(k0 + a) * ldq + n0 + b] = code[a * nn + b];
                if (qT) qT[(n0 + b) * ldqT + k0 + a] = code[a * nn + b];
            }
        free(v); free(u); free(code);
    }
}

/* Vector helper for the tests: codes of v[i] with words u[i]. */
void orc_e4m3_encode_sr_array(const float* v, const uint32_t* u, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode_sr(v[i], u[i]);
}

/* Words of elements (r0 .. r0+R-1) x (c0 .. c0+C-1), row-major into out. */
void orc_sr_words(uint64_t seed, uint32_t salt, int64_t r0, int64_t R, int64_t c0, int64_t C, uint32_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) out[i * C + j] = orc_sr_word(seed, salt, r0 + i, c0 + j);
}

/* ------------------------------------------------------------------ */
/* SwiGLU with its casts fused (the producer vector kernels)          */
/* ------------------------------------------------------------------ */
/*
 * "scratch: the backward pass, unrolled", section "What is asserted, and from
 * where": the SwiGLU input is saved as E4M3 (a quantize box); a cast rides the
 * nearest vector kernel, so the SwiGLU forward emits the next GEMM's E4M3
 * operand and the SwiGLU backward emits the next dgrad's and wgrad's operands
 * in both tile orientations (+T); the backward computes in BF16 from the
 * dequantized E4M3 input (marked as inferred on the page).
 *
 * Readings used here:
 *  - the gate/up output is one tensor [G | U] of shape [R][2F] (G = columns
 *    0..F-1, U = columns F..2F-1), in BF16;
 *  - forward:  H = bf16(silu(G) * U), silu(g) = g / (1 + exp(-g)), the exact
 *    value rounded once (RNE) -- computed here in long double, with the exact
 *    g*u/2 split off for tiny g so that a tie of g*u/2 is broken by the sign
 *    of the correction, as the exact value breaks it;
 *  - backward: G~ = bf16(fl32(dec(q_g) * s_g)), U~ likewise (the requant's
 *    fp32 dequantization, then the BF16 compute dtype);
 *    dG = bf16(dH * U~ * silu'(G~)), dU = bf16(dH * silu(G~)),
 *    silu'(g) = sigma(g) * (1 + g * (1 - sigma(g))), each exact value rounded
 *    once;
 *  - the fused casts are exactly the quantizers above applied to [G | U]
 *    (1x128, the stash), to H (1x128) and to [dG | dU] (1x128 and 128x1).
 */

/* Round a long double once to bfloat16 bits (to nearest, ties to even); the
 * value is finite and its magnitude below 2^128. */
static uint16_t bf16_round_ld(long double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    long double a = fabsl(v);
    if (a == 0.0L) return sign;
    int e2;
    frexpl(a, &e2);
    int ex = e2 - 1;                         /* a in [2^ex, 2^(ex+1)) */
    if (ex < -126) ex = -126;                /* bf16 subnormals: quantum 2^-133 */
    long double q = ldexpl(a, 7 - ex);       /* a / ulp, exact */
    long double lo = floorl(q), frac = q - lo;
    long double m = frac > 0.5L ? lo + 1.0L : (frac < 0.5L ? lo : (fmodl(lo, 2.0L) == 0.0L ? lo : lo + 1.0L));
    float fv = (float)ldexpl(m, ex - 7);     /* exact: m has at most 9 bits */
    uint32_t bits;
    memcpy(&bits, &fv, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

/* One RNE rounding to bfloat16 of the exact value hi * (1 + c), where hi has at
 * most 17 significant bits (a product of bf16 values, or half of one) and
 * |c| <= 2^-10, whose sign is c_sign (+1, -1, or 0 when the correction is
 * exactly zero; c itself may underflow to 0 for a huge gate).  A value with at most
 * 17 significant bits that is not a bf16 midpoint lies at least 2^-17 |hi|
 * from every midpoint, so when |c| < 2^-40 the correction only breaks a tie:
 * a positive c rounds the magnitude up, a negative c down.  Otherwise
 * hi + hi*c is formed in long double, where the correction (>= 2^-40
 * relative) survives. */
static uint16_t bf16_of_scaled(long double hi, long double c, int c_sign)
{
    /* an exact zero product keeps its sign, as hi * (1 + c) does with 1 + c > 0
     * (hi + hi*c would turn -0 into +0 when hi*c is +0) */
    if (hi == 0.0L) return bf16_round_ld(hi);
    if (fabsl(c) >= ldexpl(1.0L, -40)) return bf16_round_ld(hi + hi * c);
    if (c_sign == 0) return bf16_round_ld(hi);
    uint16_t sign = signbit(hi) ? 0x8000 : 0x0000;
    long double a = fabsl(hi);
    int e2;
    frexpl(a, &e2);
    int ex = e2 - 1;
    if (ex < -126) ex = -126;
    long double q = ldexpl(a, 7 - ex);
    long double lo = floorl(q);
    if (q - lo != 0.5L) return bf16_round_ld(hi);
    long double m = c_sign > 0 ? lo + 1.0L : lo;
    float fv = (float)ldexpl(m, ex - 7);
    uint32_t bits;
    memcpy(&bits, &fv, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

/* sigma(g) = 1/(1 + e^-g) and 1 - sigma(g), each without cancellation. */
static void sigma_ld(long double g, long double* sig, long double* one_minus)
{
    if (g >= 0.0L) {
        long double e = expl(-g);
        *sig = 1.0L / (1.0L + e);
        *one_minus = e / (1.0L + e);
    } else {
        long double e = expl(g);
        *sig = e / (1.0L + e);
        *one_minus = 1.0L / (1.0L + e);
    }
}

/* bf16(silu(g) * f), f a bf16 value or a product of two.  silu(g) = g sigma(g)
 *   = (g/2) (1 + tanh(g/2))        split off for |g| < 2^-10,
 *   = g (1 - (1 - sigma(g)))        split off where 1 - sigma(g) < 2^-10,
 * so that an exact product on a bf16 midpoint is moved off it the way the
 * exact value is; elsewhere g f sigma(g) in long double. */
static uint16_t bf16_silu_times(long double g, long double f)
{
    if (fabsl(g) < ldexpl(1.0L, -10))
        return bf16_of_scaled(g * f * 0.5L, tanhl(0.5L * g), g > 0.0L ? 1 : (g < 0.0L ? -1 : 0));
    long double sig, om;
    sigma_ld(g, &sig, &om);
    if (om < ldexpl(1.0L, -10)) return bf16_of_scaled(g * f, -om, -1);
    return bf16_round_ld(g * f * sig);
}

/* bf16(silu'(g) * f).  silu'(g) = sigma (1 + g (1 - sigma))
 *   = (1/2) (1 + tanh(g/2) + g / (2 cosh^2(g/2)))   split off for |g| < 2^-10,
 *   = 1 + (1 - sigma) (g sigma - 1)                  split off where that term
 *                                                    is below 2^-10,
 * elsewhere f sigma (1 + g (1 - sigma)) in long double. */
static uint16_t bf16_dsilu_times(long double g, long double f)
{
    if (fabsl(g) < ldexpl(1.0L, -10)) {
        long double ch = coshl(0.5L * g);
        return bf16_of_scaled(f * 0.5L, tanhl(0.5L * g) + g / (2.0L * ch * ch),
                              g > 0.0L ? 1 : (g < 0.0L ? -1 : 0));
    }
    long double sig, om;
    sigma_ld(g, &sig, &om);
    long double c = om * (g * sig - 1.0L);
    if (g > 2.0L && fabsl(c) < ldexpl(1.0L, -10)) return bf16_of_scaled(f, c, 1);   /* g sigma > 1 */
    return bf16_round_ld(f * (sig * (1.0L + g * om)));
}

/* H [R][F] bf16 bits from GU [R][2F] (ld ldgu). */
void orc_swiglu_h(const uint16_t* gu, int64_t R, int64_t F, int64_t ldgu, uint16_t* h, int64_t ldh)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < F; ++c) {
            long double g = orc_bf16_to_float(gu[r * ldgu + c]);
            long double u = orc_bf16_to_float(gu[r * ldgu + F + c]);
            h[r * ldh + c] = bf16_silu_times(g, u);
        }
}

/* [dG | dU] [R][2F] bf16 bits from the 1x128 stash (codes q [R][2F], scales
 * s [2F/128][R]) and dH [R][F] bf16. */
void orc_swiglu_dgu(const uint8_t* q, int64_t R, int64_t F, int64_t ldq, const float* s, int64_t lds,
                    const uint16_t* dh, int64_t lddh, uint16_t* dgu, int64_t lddgu)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < F; ++c) {
            float gq = (float)(orc_e4m3_decode(q[r * ldq + c]) * (double)s[(c / ORC_TILE) * lds + r]);
            float uq = (float)(orc_e4m3_decode(q[r * ldq + F + c]) * (double)s[((F + c) / ORC_TILE) * lds + r]);
            long double g = orc_bf16_to_float(orc_bf16_round((double)gq));
            long double u = orc_bf16_to_float(orc_bf16_round((double)uq));
            long double d = orc_bf16_to_float(dh[r * lddh + c]);
            dgu[r * lddgu + c] = bf16_dsilu_times(g, d * u);      /* d * u exact */
            dgu[r * lddgu + F + c] = bf16_silu_times(g, d);
        }
}
