// C ABI of libfgb: argument validation, then one launch per call on the
// caller's stream.  Declarations and the full contract are in include/fgb.h.

#include <math.h>

#include "../../include/fgb.h"
#include "fgb_internal.hpp"

#define FGB_VERSION_MAJOR 0
#define FGB_VERSION_MINOR 1
#define FGB_VERSION_PATCH 0

namespace {

constexpr int64_t T = 128;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
int hip_status(hipError_t e) { return e == hipSuccess ? FGB_OK : FGB_E_HIP; }

// bf16 input: 16-byte aligned rows of 16-byte multiples
int check_bf16(const uint16_t* p, int64_t ld, int64_t cols) {
    if (!p) return FGB_E_NULL;
    if (ld < cols) return FGB_E_LD;
    if (!aligned(p, 16) || ld % 8 != 0) return FGB_E_ALIGN;
    return FGB_OK;
}

// E4M3 array with rows of `cols` codes, accessed in `vec`-byte pieces
int check_codes(const uint8_t* p, int64_t ld, int64_t cols, int vec) {
    if (!p) return FGB_E_NULL;
    if (ld < cols) return FGB_E_LD;
    if (!aligned(p, vec) || ld % vec != 0) return FGB_E_ALIGN;
    return FGB_OK;
}

int check_scales(const void* p, int64_t ld, int64_t need) {
    if (!p) return FGB_E_NULL;
    if (ld < need) return FGB_E_LD;
    if (!aligned(p, 4)) return FGB_E_ALIGN;
    return FGB_OK;
}

bool bad_floor(float f) { return !(f >= 0.0f) || isinf(f); }

#define FGB_TRY(expr)                 \
    do {                              \
        int _st = (expr);             \
        if (_st != FGB_OK) return _st; \
    } while (0)

}  // namespace

extern "C" {

int fgb_version(void)
{
    return (FGB_VERSION_MAJOR << 16) | (FGB_VERSION_MINOR << 8) | FGB_VERSION_PATCH;
}

const char* fgb_status_string(int status)
{
    switch (status) {
    case FGB_OK: return "ok";
    case FGB_E_NULL: return "a required pointer is NULL";
    case FGB_E_SHAPE: return "invalid dimension (negative, or not a required multiple)";
    case FGB_E_ALIGN: return "misaligned pointer or leading dimension";
    case FGB_E_LD: return "leading dimension smaller than required";
    case FGB_E_UNSUPPORTED: return "unsupported request";
    case FGB_E_HIP: return "HIP runtime error at launch";
    case FGB_E_ARG: return "invalid argument";
    default: return "unknown status";
    }
}

// ------------------------------ quantizers --------------------------------
// Each quantizer exists for scales absmax/448 and for power-of-two scales (po2,
// the UE8M0 value set); both are fp32 arrays with the same layout and rules.
static int check_sc(const float* p, int64_t ld, int64_t need, bool) { return check_scales(p, ld, need); }

static int quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds, bool po2, void* stream,
                          const fgb::SrParams* sr = nullptr)
{
    if (R < 0 || C < 0 || C % 8 != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (R == 0 || C == 0) return FGB_OK;
    FGB_TRY(check_bf16(x, ldx, C));
    FGB_TRY(check_codes(q, ldq, C, 8));
    FGB_TRY(check_sc(s, lds, R, po2));
    return hip_status(fgb::launch_quantize_1x128(x, R, C, ldx, amax_floor, q, ldq, s, lds, po2, as_stream(stream), sr));
}

static int quantize_128x1(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                          uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, bool po2, void* stream,
                          const fgb::SrParams* sr = nullptr)
{
    if (R < 0 || C < 0 || C % 8 != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (R == 0 || C == 0) return FGB_OK;
    FGB_TRY(check_bf16(x, ldx, C));
    FGB_TRY(check_codes(qT, ldqT, rup(R, T), 16));
    FGB_TRY(check_sc(sT, ldsT, C, po2));
    return hip_status(fgb::launch_tile128(fgb::kTile128x1, x, R, C, ldx, nullptr, 0, amax_floor,
                                          nullptr, 0, qT, ldqT, sT, ldsT, po2, as_stream(stream),
                                          nullptr, 0, sr));
}

static int quantize_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, bool po2, void* stream,
                         const fgb::SrParams* sr = nullptr)
{
    if (R < 0 || C < 0 || C % 8 != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (R == 0 || C == 0) return FGB_OK;
    FGB_TRY(check_bf16(x, ldx, C));
    FGB_TRY(check_codes(q, ldq, C, 8));
    FGB_TRY(check_sc(s, lds, R, po2));
    FGB_TRY(check_codes(qT, ldqT, rup(R, T), 16));
    FGB_TRY(check_sc(sT, ldsT, C, po2));
    return hip_status(fgb::launch_tile128(fgb::kTileDual, x, R, C, ldx, nullptr, 0, amax_floor,
                                          q, ldq, qT, ldqT, sT, ldsT, po2, as_stream(stream), s, lds, sr));
}

static int quantize_128x128(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, float amax_floor,
                            uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s, bool po2, void* stream,
                            const fgb::SrParams* sr = nullptr)
{
    if (K < 0 || N < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (K == 0 || N == 0) return FGB_OK;
    FGB_TRY(check_bf16(w, ldw, N));
    if (!q && !qT) return FGB_E_NULL;
    if (q) FGB_TRY(check_codes(q, ldq, N, 8));
    if (qT) FGB_TRY(check_codes(qT, ldqT, K, 16));
    FGB_TRY(check_sc(s, N / T, N / T, po2));
    return hip_status(fgb::launch_tile128(fgb::kTile128x128, w, K, N, ldw, nullptr, 0, amax_floor,
                                          q, ldq, qT, ldqT, s, N / T, po2, as_stream(stream), nullptr, 0, sr));
}

// E stacked weights w [E][K][N] -> q [E][K][N], qT [E][N][K], s [E][K/128][N/128].
static int quantize_128x128_batched(int64_t E, const uint16_t* w, int64_t K, int64_t N, float amax_floor,
                                    uint8_t* q, uint8_t* qT, float* s, bool po2, void* stream)
{
    if (E < 0 || E > 65535 || K < 0 || N < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (E == 0 || K == 0 || N == 0) return FGB_OK;
    FGB_TRY(check_bf16(w, N, N));
    if (!q && !qT) return FGB_E_NULL;
    if (q) FGB_TRY(check_codes(q, N, N, 8));
    if (qT) FGB_TRY(check_codes(qT, K, K, 16));
    FGB_TRY(check_sc(s, N / T, N / T, po2));
    fgb::TileBatch bt;
    bt.in = K * N * 2; bt.q = K * N; bt.qT = N * K; bt.s = (K / T) * (N / T);
    return hip_status(fgb::launch_tile128(fgb::kTile128x128, w, K, N, N, nullptr, 0, amax_floor,
                                          q, N, qT, K, s, N / T, po2, as_stream(stream), nullptr, 0, nullptr,
                                          E, bt));
}

int fgb_quantize_128x128_batched(int64_t E, const uint16_t* w, int64_t K, int64_t N, float amax_floor,
                                 uint8_t* q, uint8_t* qT, float* s, void* stream)
{
    return quantize_128x128_batched(E, w, K, N, amax_floor, q, qT, s, false, stream);
}

int fgb_quantize_128x128_batched_ue8m0(int64_t E, const uint16_t* w, int64_t K, int64_t N, float amax_floor,
                                       uint8_t* q, uint8_t* qT, float* s, void* stream)
{
    return quantize_128x128_batched(E, w, K, N, amax_floor, q, qT, s, true, stream);
}

static int requant_128x1(const uint8_t* q, int64_t R, int64_t C, int64_t ldq, const float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, bool po2, void* stream)
{
    if (R < 0 || C < 0 || C % 8 != 0) return FGB_E_SHAPE;
    if (R == 0 || C == 0) return FGB_OK;
    FGB_TRY(check_codes(q, ldq, C, 8));
    FGB_TRY(check_sc(s, lds, R, po2));
    FGB_TRY(check_codes(qT, ldqT, rup(R, T), 16));
    FGB_TRY(check_sc(sT, ldsT, C, po2));
    return hip_status(fgb::launch_tile128(fgb::kTileRequant, q, R, C, ldq, s, lds, 0.0f,
                                          nullptr, 0, qT, ldqT, sT, ldsT, po2, as_stream(stream)));
}

int fgb_quantize_1x128(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream)
{
    return quantize_1x128(x, R, C, ldx, amax_floor, q, ldq, s, lds, false, stream);
}

int fgb_quantize_128x1(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                       uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return quantize_128x1(x, R, C, ldx, amax_floor, qT, ldqT, sT, ldsT, false, stream);
}

int fgb_quantize_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                      uint8_t* q, int64_t ldq, float* s, int64_t lds,
                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return quantize_dual(x, R, C, ldx, amax_floor, q, ldq, s, lds, qT, ldqT, sT, ldsT, false, stream);
}

int fgb_quantize_128x128(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, float amax_floor,
                         uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s, void* stream)
{
    return quantize_128x128(w, K, N, ldw, amax_floor, q, ldq, qT, ldqT, s, false, stream);
}

int fgb_requant_128x1(const uint8_t* q, int64_t R, int64_t C, int64_t ldq, const float* s, int64_t lds,
                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return requant_128x1(q, R, C, ldq, s, lds, qT, ldqT, sT, ldsT, false, stream);
}

int fgb_quantize_1x128_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream)
{
    return quantize_1x128(x, R, C, ldx, amax_floor, q, ldq, s, lds, true, stream);
}

int fgb_quantize_128x1_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return quantize_128x1(x, R, C, ldx, amax_floor, qT, ldqT, sT, ldsT, true, stream);
}

int fgb_quantize_dual_ue8m0(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return quantize_dual(x, R, C, ldx, amax_floor, q, ldq, s, lds, qT, ldqT, sT, ldsT, true, stream);
}

int fgb_quantize_128x128_ue8m0(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, float amax_floor,
                               uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s, void* stream)
{
    return quantize_128x128(w, K, N, ldw, amax_floor, q, ldq, qT, ldqT, s, true, stream);
}

int fgb_requant_128x1_ue8m0(const uint8_t* q, int64_t R, int64_t C, int64_t ldq, const float* s, int64_t lds,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream)
{
    return requant_128x1(q, R, C, ldq, s, lds, qT, ldqT, sT, ldsT, true, stream);
}

int fgb_requant_128x128_ue8m0(const uint8_t* q, int64_t K, int64_t N, int64_t ldq, const float* s,
                              float amax_floor, uint8_t* q2, int64_t ldq2, uint8_t* q2T, int64_t ldq2T,
                              float* s2, void* stream)
{
    if (K < 0 || N < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (K == 0 || N == 0) return FGB_OK;
    FGB_TRY(check_codes(q, ldq, N, 8));
    FGB_TRY(check_sc(s, N / T, N / T, false));
    if (!q2 && !q2T) return FGB_E_NULL;
    if (q2) FGB_TRY(check_codes(q2, ldq2, N, 8));
    if (q2T) FGB_TRY(check_codes(q2T, ldq2T, K, 16));
    FGB_TRY(check_sc(s2, N / T, N / T, true));
    return hip_status(fgb::launch_tile128(fgb::kTileRequant128x128, q, K, N, ldq, s, N / T, amax_floor,
                                          q2, ldq2, q2T, ldq2T, s2, N / T, true, as_stream(stream)));
}

// ------------------------------- SwiGLU ------------------------------------
int fgb_swiglu_fwd_quant(const uint16_t* gu, int64_t R, int64_t F, int64_t ldgu, float amax_floor,
                         uint8_t* q_gu, int64_t ldq_gu, float* s_gu, int64_t lds_gu,
                         uint8_t* q_h, int64_t ldq_h, float* s_h, int64_t lds_h,
                         uint16_t* h, int64_t ldh, void* stream)
{
    if (R < 0 || F < 0 || F % T != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (R == 0 || F == 0) return FGB_OK;
    FGB_TRY(check_bf16(gu, ldgu, 2 * F));
    if ((q_gu == nullptr) != (s_gu == nullptr)) return FGB_E_NULL;
    if (q_gu) {
        FGB_TRY(check_codes(q_gu, ldq_gu, 2 * F, 8));
        FGB_TRY(check_scales(s_gu, lds_gu, R));
    }
    FGB_TRY(check_codes(q_h, ldq_h, F, 8));
    FGB_TRY(check_scales(s_h, lds_h, R));
    if (h) FGB_TRY(check_bf16(h, ldh, F));
    return hip_status(fgb::launch_swiglu_fwd(gu, R, F, ldgu, amax_floor, q_gu, ldq_gu, s_gu, lds_gu,
                                             q_h, ldq_h, s_h, lds_h, h, ldh, as_stream(stream)));
}

int fgb_swiglu_bwd_quant(const uint8_t* q_gu, int64_t R, int64_t F, int64_t ldq_gu, const float* s_gu, int64_t lds_gu,
                         const uint16_t* dh, int64_t lddh, float amax_floor,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                         uint16_t* dgu, int64_t lddgu, void* stream)
{
    if (R < 0 || F < 0 || F % T != 0) return FGB_E_SHAPE;
    if (bad_floor(amax_floor)) return FGB_E_ARG;
    if (R == 0 || F == 0) return FGB_OK;
    FGB_TRY(check_codes(q_gu, ldq_gu, 2 * F, 8));
    FGB_TRY(check_scales(s_gu, lds_gu, R));
    FGB_TRY(check_bf16(dh, lddh, F));
    FGB_TRY(check_codes(q, ldq, 2 * F, 8));
    FGB_TRY(check_scales(s, lds, R));
    FGB_TRY(check_codes(qT, ldqT, rup(R, T), 16));
    FGB_TRY(check_scales(sT, ldsT, 2 * F));
    if (dgu) FGB_TRY(check_bf16(dgu, lddgu, 2 * F));
    return hip_status(fgb::launch_swiglu_bwd(q_gu, R, F, ldq_gu, s_gu, lds_gu, dh, lddh, amax_floor,
                                             q, ldq, s, lds, qT, ldqT, sT, ldsT, dgu, lddgu, as_stream(stream)));
}

// Stochastic-rounding twins (absmax/448 scales): the same tiles and scales, the
// cast picks the lower or upper E4M3 neighbour with one Philox4x32-10 word per
// element.
int fgb_quantize_1x128_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds, uint64_t seed, uint32_t salt,
                          void* stream)
{
    const fgb::SrParams sr{seed, salt};
    return quantize_1x128(x, R, C, ldx, amax_floor, q, ldq, s, lds, false, stream, &sr);
}

int fgb_quantize_128x1_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                          uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, uint64_t seed, uint32_t salt,
                          void* stream)
{
    const fgb::SrParams sr{seed, salt};
    return quantize_128x1(x, R, C, ldx, amax_floor, qT, ldqT, sT, ldsT, false, stream, &sr);
}

int fgb_quantize_dual_sr(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float amax_floor,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds,
                         uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, uint64_t seed, uint32_t salt,
                         void* stream)
{
    const fgb::SrParams sr{seed, salt};
    return quantize_dual(x, R, C, ldx, amax_floor, q, ldq, s, lds, qT, ldqT, sT, ldsT, false, stream, &sr);
}

int fgb_quantize_128x128_sr(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, float amax_floor,
                            uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s,
                            uint64_t seed, uint32_t salt, void* stream)
{
    const fgb::SrParams sr{seed, salt};
    return quantize_128x128(w, K, N, ldw, amax_floor, q, ldq, qT, ldqT, s, false, stream, &sr);
}

static int gemm_fprop_impl(int64_t M, int64_t N, int64_t K,
                   const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                   const uint8_t* qwT, int64_t ldqwT, const float* sw,
                   uint16_t* y, int64_t ldy, void* stream, bool po2)
{
    if (M < 0 || N < 0 || K < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (M == 0 || N == 0) return FGB_OK;
    FGB_TRY(check_bf16(y, ldy, N));
    if (K > 0) {
        FGB_TRY(check_codes(qx, ldqx, K, 16));
        FGB_TRY(check_scales(sx, ldsx, M));
        FGB_TRY(check_codes(qwT, ldqwT, K, 16));
        FGB_TRY(check_scales(sw, 1, 1));
    }
    fgb::GemmArgs a;
    a.M = M; a.N = N; a.nkb = K / T;
    a.A = qx; a.lda = ldqx; a.sa = sx; a.sa_ld = ldsx;
    a.B = qwT; a.ldb = ldqwT; a.sb = sw; a.sb_kb = N / T; a.sb_n = 1;
    a.out = y; a.ldo = ldy;
    if (!fgb::gemm_supported(a, false)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kFprop, false, a, as_stream(stream), po2));
}

static int gemm_dgrad_impl(int64_t M, int64_t K, int64_t N,
                   const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy,
                   const uint8_t* qw, int64_t ldqw, const float* sw,
                   uint16_t* dx, int64_t lddx, void* stream, bool po2)
{
    if (M < 0 || N < 0 || K < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (M == 0 || K == 0) return FGB_OK;
    FGB_TRY(check_bf16(dx, lddx, K));
    if (N > 0) {
        FGB_TRY(check_codes(qdy, ldqdy, N, 16));
        FGB_TRY(check_scales(sdy, ldsdy, M));
        FGB_TRY(check_codes(qw, ldqw, N, 16));
        FGB_TRY(check_scales(sw, 1, 1));
    }
    fgb::GemmArgs a;
    a.M = M; a.N = K; a.nkb = N / T;
    a.A = qdy; a.lda = ldqdy; a.sa = sdy; a.sa_ld = ldsdy;
    // output column k uses weight tile row k/128: SB(k, b) = sw[(k/128)*(N/128) + b]
    a.B = qw; a.ldb = ldqw; a.sb = sw; a.sb_kb = 1; a.sb_n = N / T;
    a.out = dx; a.ldo = lddx;
    if (!fgb::gemm_supported(a, false)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kDgrad, false, a, as_stream(stream), po2));
}

static int gemm_wgrad_impl(int64_t K, int64_t N, int64_t M,
                   const uint8_t* qxT, int64_t ldqxT, const float* sxT, int64_t ldsxT,
                   const uint8_t* qdyT, int64_t ldqdyT, const float* sdyT, int64_t ldsdyT,
                   float* dw, int64_t lddw, int accumulate, void* stream, bool po2)
{
    if (M < 0 || N < 0 || K < 0 || K % T != 0 || N % T != 0) return FGB_E_SHAPE;
    if (K == 0 || N == 0) return FGB_OK;
    if (!dw) return FGB_E_NULL;
    if (lddw < N) return FGB_E_LD;
    if (!aligned(dw, 16) || lddw % 4 != 0) return FGB_E_ALIGN;
    if (M > 0) {
        FGB_TRY(check_codes(qxT, ldqxT, rup(M, T), 16));
        FGB_TRY(check_scales(sxT, ldsxT, K));
        FGB_TRY(check_codes(qdyT, ldqdyT, rup(M, T), 16));
        FGB_TRY(check_scales(sdyT, ldsdyT, N));
    }
    fgb::GemmArgs a;
    a.M = K; a.N = N; a.nkb = cdiv(M, T);
    a.A = qxT; a.lda = ldqxT; a.sa = sxT; a.sa_ld = ldsxT;
    a.B = qdyT; a.ldb = ldqdyT; a.sb = sdyT; a.sb_kb = ldsdyT;
    a.out = dw; a.ldo = lddw; a.accumulate = accumulate ? 1 : 0;
    if (!fgb::gemm_supported(a, false)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kWgrad, false, a, as_stream(stream), po2));
}

static int gemm_fprop_grouped_impl(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t N, int64_t K,
                           const uint8_t* qx, const float* sx, const uint8_t* qwT, const float* sw,
                           uint16_t* y, void* stream, bool po2)
{
    if (E < 0 || R_pad < 0 || N < 0 || K < 0) return FGB_E_SHAPE;
    if (R_pad % T != 0 || N % T != 0 || K % T != 0 || E > 65535) return FGB_E_SHAPE;
    if (E == 0 || R_pad == 0 || N == 0) return FGB_OK;
    if (!offsets || !y) return FGB_E_NULL;
    if (!aligned(offsets, 4) || !aligned(y, 16)) return FGB_E_ALIGN;
    if (K > 0) {
        FGB_TRY(check_codes(qx, K, K, 16));
        FGB_TRY(check_scales(sx, R_pad, R_pad));
        FGB_TRY(check_codes(qwT, K, K, 16));
        FGB_TRY(check_scales(sw, 1, 1));
    }
    fgb::GemmArgs a;
    a.M = R_pad; a.N = N; a.nkb = K / T;
    a.A = qx; a.lda = K; a.sa = sx; a.sa_ld = R_pad;
    a.B = qwT; a.ldb = K; a.sb = sw; a.sb_kb = N / T; a.sb_n = 1;
    a.out = y; a.ldo = N;
    a.offsets = offsets; a.E = E;
    a.b_expert_stride = N * K; a.sb_expert_stride = (K / T) * (N / T);
    if (!fgb::gemm_supported(a, true)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kFprop, true, a, as_stream(stream), po2));
}

static int gemm_dgrad_grouped_impl(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                           const uint8_t* qdy, const float* sdy, const uint8_t* qw, const float* sw,
                           uint16_t* dx, void* stream, bool po2)
{
    if (E < 0 || R_pad < 0 || N < 0 || K < 0) return FGB_E_SHAPE;
    if (R_pad % T != 0 || N % T != 0 || K % T != 0 || E > 65535) return FGB_E_SHAPE;
    if (E == 0 || R_pad == 0 || K == 0) return FGB_OK;
    if (!offsets || !dx) return FGB_E_NULL;
    if (!aligned(offsets, 4) || !aligned(dx, 16)) return FGB_E_ALIGN;
    if (N > 0) {
        FGB_TRY(check_codes(qdy, N, N, 16));
        FGB_TRY(check_scales(sdy, R_pad, R_pad));
        FGB_TRY(check_codes(qw, N, N, 16));
        FGB_TRY(check_scales(sw, 1, 1));
    }
    fgb::GemmArgs a;
    a.M = R_pad; a.N = K; a.nkb = N / T;
    a.A = qdy; a.lda = N; a.sa = sdy; a.sa_ld = R_pad;
    a.B = qw; a.ldb = N; a.sb = sw; a.sb_kb = 1; a.sb_n = N / T;
    a.out = dx; a.ldo = K;
    a.offsets = offsets; a.E = E;
    a.b_expert_stride = K * N; a.sb_expert_stride = (K / T) * (N / T);
    if (!fgb::gemm_supported(a, true)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kDgrad, true, a, as_stream(stream), po2));
}

static int gemm_wgrad_grouped_impl(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                           const uint8_t* qxT, const float* sxT, const uint8_t* qdyT, const float* sdyT,
                           float* dw, int accumulate, void* stream, bool po2)
{
    if (E < 0 || R_pad < 0 || N < 0 || K < 0) return FGB_E_SHAPE;
    if (R_pad % T != 0 || N % T != 0 || K % T != 0 || E > 65535) return FGB_E_SHAPE;
    if (E == 0 || K == 0 || N == 0) return FGB_OK;
    if (!offsets || !dw) return FGB_E_NULL;
    if (!aligned(offsets, 4) || !aligned(dw, 16)) return FGB_E_ALIGN;
    if (R_pad > 0) {
        FGB_TRY(check_codes(qxT, R_pad, R_pad, 16));
        FGB_TRY(check_scales(sxT, K, K));
        FGB_TRY(check_codes(qdyT, R_pad, R_pad, 16));
        FGB_TRY(check_scales(sdyT, N, N));
    }
    fgb::GemmArgs a;
    a.M = K; a.N = N; a.nkb = R_pad / T;
    a.A = qxT; a.lda = R_pad; a.sa = sxT; a.sa_ld = K;
    a.B = qdyT; a.ldb = R_pad; a.sb = sdyT; a.sb_kb = N;
    a.out = dw; a.ldo = N; a.accumulate = accumulate ? 1 : 0;
    a.offsets = offsets; a.E = E; a.out_expert_stride = K * N;
    if (!fgb::gemm_supported(a, true)) return FGB_E_UNSUPPORTED;
    return hip_status(fgb::launch_gemm(fgb::kWgrad, true, a, as_stream(stream), po2));
}

// Public GEMMs: scales absmax/448 (any fp32), or powers of two (_ue8m0).
int fgb_gemm_fprop(int64_t M, int64_t N, int64_t K, const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                   const uint8_t* qwT, int64_t ldqwT, const float* sw, uint16_t* y, int64_t ldy, void* stream)
{ return gemm_fprop_impl(M, N, K, qx, ldqx, sx, ldsx, qwT, ldqwT, sw, y, ldy, stream, false); }
int fgb_gemm_dgrad(int64_t M, int64_t K, int64_t N, const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy,
                   const uint8_t* qw, int64_t ldqw, const float* sw, uint16_t* dx, int64_t lddx, void* stream)
{ return gemm_dgrad_impl(M, K, N, qdy, ldqdy, sdy, ldsdy, qw, ldqw, sw, dx, lddx, stream, false); }
int fgb_gemm_wgrad(int64_t K, int64_t N, int64_t M, const uint8_t* qxT, int64_t ldqxT, const float* sxT, int64_t ldsxT,
                   const uint8_t* qdyT, int64_t ldqdyT, const float* sdyT, int64_t ldsdyT,
                   float* dw, int64_t lddw, int accumulate, void* stream)
{ return gemm_wgrad_impl(K, N, M, qxT, ldqxT, sxT, ldsxT, qdyT, ldqdyT, sdyT, ldsdyT, dw, lddw, accumulate, stream, false); }
int fgb_gemm_fprop_grouped(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t N, int64_t K,
                           const uint8_t* qx, const float* sx, const uint8_t* qwT, const float* sw,
                           uint16_t* y, void* stream)
{ return gemm_fprop_grouped_impl(E, offsets, R_pad, N, K, qx, sx, qwT, sw, y, stream, false); }
int fgb_gemm_dgrad_grouped(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                           const uint8_t* qdy, const float* sdy, const uint8_t* qw, const float* sw,
                           uint16_t* dx, void* stream)
{ return gemm_dgrad_grouped_impl(E, offsets, R_pad, K, N, qdy, sdy, qw, sw, dx, stream, false); }
int fgb_gemm_wgrad_grouped(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                           const uint8_t* qxT, const float* sxT, const uint8_t* qdyT, const float* sdyT,
                           float* dw, int accumulate, void* stream)
{ return gemm_wgrad_grouped_impl(E, offsets, R_pad, K, N, qxT, sxT, qdyT, sdyT, dw, accumulate, stream, false); }

int fgb_gemm_fprop_ue8m0(int64_t M, int64_t N, int64_t K, const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                         const uint8_t* qwT, int64_t ldqwT, const float* sw, uint16_t* y, int64_t ldy, void* stream)
{ return gemm_fprop_impl(M, N, K, qx, ldqx, sx, ldsx, qwT, ldqwT, sw, y, ldy, stream, true); }
int fgb_gemm_dgrad_ue8m0(int64_t M, int64_t K, int64_t N, const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy,
                         const uint8_t* qw, int64_t ldqw, const float* sw, uint16_t* dx, int64_t lddx, void* stream)
{ return gemm_dgrad_impl(M, K, N, qdy, ldqdy, sdy, ldsdy, qw, ldqw, sw, dx, lddx, stream, true); }
int fgb_gemm_wgrad_ue8m0(int64_t K, int64_t N, int64_t M, const uint8_t* qxT, int64_t ldqxT, const float* sxT, int64_t ldsxT,
                         const uint8_t* qdyT, int64_t ldqdyT, const float* sdyT, int64_t ldsdyT,
                         float* dw, int64_t lddw, int accumulate, void* stream)
{ return gemm_wgrad_impl(K, N, M, qxT, ldqxT, sxT, ldsxT, qdyT, ldqdyT, sdyT, ldsdyT, dw, lddw, accumulate, stream, true); }
int fgb_gemm_fprop_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t N, int64_t K,
                                 const uint8_t* qx, const float* sx, const uint8_t* qwT, const float* sw,
                                 uint16_t* y, void* stream)
{ return gemm_fprop_grouped_impl(E, offsets, R_pad, N, K, qx, sx, qwT, sw, y, stream, true); }
int fgb_gemm_dgrad_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                                 const uint8_t* qdy, const float* sdy, const uint8_t* qw, const float* sw,
                                 uint16_t* dx, void* stream)
{ return gemm_dgrad_grouped_impl(E, offsets, R_pad, K, N, qdy, sdy, qw, sw, dx, stream, true); }
int fgb_gemm_wgrad_grouped_ue8m0(int64_t E, const int32_t* offsets, int64_t R_pad, int64_t K, int64_t N,
                                 const uint8_t* qxT, const float* sxT, const uint8_t* qdyT, const float* sdyT,
                                 float* dw, int accumulate, void* stream)
{ return gemm_wgrad_grouped_impl(E, offsets, R_pad, K, N, qxT, sxT, qdyT, sdyT, dw, accumulate, stream, true); }

}  // extern "C"
