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

#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "fgb_internal.hpp"

namespace fgb {

// ===========================================================================
// 256 x TN output tile per block of 8 waves (two waves per SIMD, so the 112-128
// accumulator VGPRs of a wave fit beside its fragments).  Per 128-block the A
// and B slices (32 KB each) and the block's scales are brought into LDS by
// direct-to-LDS 16-byte loads, double buffered: the loads of block kb+1 are in
// flight while block kb is computed, and on the vector-rescale path they are
// issued one every other MFMA step of block kb's computation.
// ===========================================================================
constexpr int kTM = 256;                           // output rows per block tile
constexpr int kStageA = kTM * kTile;               // 32 KB
constexpr int kStageB = 256 * kTile;               // room for up to 256 B rows
constexpr int kStageBytes = kStageA + kStageB + 2 * 1024;   // + SA, SB (256 floats each)
constexpr int kV1Threads = 512;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct-to-LDS loads (global_load_lds): 64 lanes x 16 B (or x 4 B) land at
// consecutive addresses from the wave-uniform LDS byte address `lds`; the
// global address is the wave-uniform `base` (an SGPR pair) plus the lane's
// 32-bit byte offset.  Issued from inline assembly so that the compiler's wait
// insertion does not treat the in-flight loads as pending writes to every LDS
// location (which would make every LDS read wait for the prefetch); the kernel
// waits for each stage itself with vmcnt.  M0 carries the LDS address; the
// asm declares it clobbered, so the compiler re-establishes M0 only where it
// needs it itself, and no save and restore is spent per load.  The "memory"
// clobber keeps LDS accesses from moving across the issue; the _nc forms, used inside the computation for the stage
// that it does not read, leave the compiler free to schedule around them (the
// next barrier orders them).
// `lds` is the LDS byte address as an integer (wave-uniform): computed from
// the shared array's address once, so no generic-to-LDS pointer conversion
// (and its null check) is repeated per load.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "m0", "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "m0", "memory");
}
__device__ __forceinline__ void dma16_nc(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "m0");
}
__device__ __forceinline__ void dma4_nc(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "m0");
}

// Calls f(integral_constant<int, t>) for t = 0 .. N-1, so that every index
// derived from t is a compile-time constant.
template <int... ts, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, ts...>, F&& f) {
    (f(std::integral_constant<int, ts>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// Staged row r keeps its eight 16-byte chunks at slots c ^ swz(r), swz(r) =
// (r & 7) ^ ((r >> 3) & 1).  A fragment read has the 16 lanes of a lane group
// read one 16-byte chunk from each of 16 consecutive rows (128 bytes apart).
// The LDS counters (SQ_LDS_BANK_CONFLICT) show that such a read is free of bank
// conflicts only when every 8 consecutive lanes hit 8 distinct 16-byte slots of
// a 128-byte window AND all 16 lanes hit distinct slots of a 256-byte window:
// r & 7 separates rows 0..7 (and 8..15), the ^ ((r >> 3) & 1) separates row r
// from row r + 8, which shares its parity.  The swizzle depends on r mod 16
// only, and fragments start at multiples of 16 rows, so one per-lane value
// serves every fragment.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// A fragment from its two 16-byte chunks at lo + off and hi + off.
__device__ __forceinline__ v8i frag_at(const uint8_t* lo, const uint8_t* hi, int off) {
    const uint4 l = *reinterpret_cast<const uint4*>(lo + off);
    const uint4 h = *reinterpret_cast<const uint4*>(hi + off);
    v8i r;
    r[0] = (int)l.x; r[1] = (int)l.y; r[2] = (int)l.z; r[3] = (int)l.w;
    r[4] = (int)h.x; r[5] = (int)h.y; r[6] = (int)h.z; r[7] = (int)h.w;
    return r;
}

// Consecutive block ids go round-robin over the 8 XCDs: give each XCD a
// contiguous range of the tile order instead (bijective on [0, total)).
__device__ __forceinline__ int xcd_order(int bid, int total) {
    const int per = total / 8, rem = total % 8;
    const int xcd = bid % 8, local = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Tile t of a tiles_m x tiles_n grid, in groups of 8 M-tiles (column-major
// inside a group), so that the tiles an XCD runs together share A rows and B
// columns in its L2.
__device__ __forceinline__ void group_order(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int G = 8;
    const int in_group = G * tiles_n;
    const int first_m = (t / in_group) * G;
    const int gsize = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
    const int r = t % in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Row-grouped (MoE) tiles: expert e owns rows [o(e), o(e+1)) of the output,
// o(e) = offsets[e] clamped to [0, min(offsets[E], M)], and is cut into
// ceil(len/256) row tiles of its own (the last one may hold 128 rows).  ntm is
// the number of row tiles over all experts; the tiles are the experts' own
// (row tiles x tiles_n) grids in expert order.
struct RowTile { int e; int64_t m0, mend; };

__device__ __forceinline__ int clamp_off(int v, int total) { return v < 0 ? 0 : (v > total ? total : v); }

__device__ int row_tiles_total(const GemmArgs& g, int total) {
    const int lane = threadIdx.x & 63;
    int ntm = 0;
    for (int base = 0; base < g.E; base += 64) {
        const int e = base + lane;
        int te = 0;
        if (e < g.E) {
            const int lo = clamp_off(g.offsets[e], total), hi = clamp_off(g.offsets[e + 1], total);
            te = hi > lo ? (hi - lo + kTM - 1) / kTM : 0;
        }
        ntm += __builtin_amdgcn_readlane(wave_scan(te), 63);
    }
    return ntm;
}

// Tile t of the row-grouped sequence: every wave of the block finds the expert
// whose tiles hold t (a 64-lane prefix scan over the offsets), and orders that
// expert's tiles in groups of 8 row tiles, so that the tiles an XCD runs
// together share one expert's weight columns (a group over all row tiles
// would straddle experts; grouped Fprop 1.4-1.7% slower).  An empty result
// (mend == m0) means t lies past the last tile.
__device__ RowTile grouped_tile(const GemmArgs& g, int total, int t, int tiles_n, int& tn) {
    const int lane = threadIdx.x & 63;
    RowTile rt{0, 0, 0};
    tn = 0;
    int before = 0;                                 // row tiles of the experts before this chunk
    for (int base = 0; base < g.E; base += 64) {
        const int e = base + lane;
        int lo = 0, hi = 0, te = 0;
        if (e < g.E) {
            lo = clamp_off(g.offsets[e], total); hi = clamp_off(g.offsets[e + 1], total);
            te = hi > lo ? (hi - lo + kTM - 1) / kTM : 0;
        }
        const int incl = wave_scan(te), excl = incl - te;
        const bool mine = te > 0 && (before + excl) * tiles_n <= t && t < (before + incl) * tiles_n;
        const uint64_t hit = __ballot(mine);
        if (hit) {
            const int j = __builtin_ctzll(hit);
            int tm;
            group_order(t - (before + __builtin_amdgcn_readlane(excl, j)) * tiles_n, __builtin_amdgcn_readlane(te, j),
                        tiles_n, tm, tn);
            rt.e = base + j;
            rt.m0 = (int64_t)__builtin_amdgcn_readlane(lo, j) + (int64_t)kTM * tm;
            rt.mend = __builtin_amdgcn_readlane(hi, j);
            return rt;
        }
        before += __builtin_amdgcn_readlane(incl, 63);
    }
    return rt;
}

// Barrier between the waves of a block for LDS traffic: waits only for this
// wave's own LDS operations (lgkmcnt), never for its global or direct-to-LDS
// loads (the next stage's prefetch stays in flight; each stage is waited for
// explicitly with vmcnt), and the memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block tile kTM x TN with 8 waves.  TN = 256: waves 2 (M) x 4 (N), 128x64
// per wave.  TN = 224: waves 4 x 2, 64x112 per wave (used where N is a multiple
// of 224 and the tile count then fills whole waves of the GPU).
template <int TN> struct TileShape {
    static constexpr int WAVES_M = (TN == 256) ? 2 : 4;
    static constexpr int WAVES_N = 8 / WAVES_M;
    static constexpr int WTM = kTM / WAVES_M;     // rows per wave
    static constexpr int WTN = TN / WAVES_N;      // columns per wave
    static constexpr int MI = WTM / 16;           // 16-row pieces per wave
    static constexpr int NJ = WTN / 16;           // 16-column pieces per wave
    static_assert(WTN % 16 == 0 && WTM % 16 == 0, "wave tile");
};

// Each 16x16x128 MFMA takes the B fragment as its first operand, so a lane ends
// up holding ONE output row (lane & 15) and FOUR consecutive output columns
// (4 * (lane >> 4) .. +3) of every 16x16 piece: one row scale per piece, and
// 8- or 16-byte vector stores in the epilogue.
//
// GROUP = kDense: one GEMM.  kGroupRows: the output rows are cut into expert
// segments (row tiles never straddle two experts) and each segment uses its
// expert's B and weight scales.  kGroupK: the contraction blocks are cut into
// expert segments and expert e writes its own output g.out + e*out_expert_stride.
enum { kDense = 0, kGroupRows = 1, kGroupK = 2 };

//
// PO2: every scale is a power of two (the UE8M0 value set, held in fp32).  The
// matrix core then applies SA*SB itself (its E8M0 block-scale operands are the
// fp32 exponent fields) and adds each block's partial sums to the accumulator
// it is given as C: that addition is an fp32 round-to-nearest-even add, so
// chaining the accumulator through C promotes every 128-block into fp32 with
// no vector-ALU rescale at all.
//
// SPLIT (dense only): the tiles from g.split_from on (those that do not fill a
// whole round of CUs) are computed as column halves by two blocks each.
template <int TN, bool OUTER, bool BF16_OUT, int GROUP, bool PO2, bool SPLIT = false>
__global__ __launch_bounds__(kV1Threads) void k_gemm_block_scaled(GemmArgs g)
{
    using S = TileShape<TN>;
    constexpr int MI = S::MI, NJ = S::NJ, WTM = S::WTM, WTN = S::WTN;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];   // two stages
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_u8*)smem;           // its LDS byte address
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave % S::WAVES_M, wn = wave / S::WAVES_M;

    const int tiles_n = (int)((g.N + TN - 1) / TN);
    int tm, tn;
    int64_t m0, mend = g.M, kb0 = 0, kb1 = g.nkb;
    const uint8_t* Bp = g.B;
    const float* sbp = g.sb;
    void* outp = g.out;
    int half = -1;                                  // >= 0: this block computes column half `half`
    if constexpr (GROUP == kDense) {
        const int tiles_m = (int)((g.M + kTM - 1) / kTM);
        const int bid = (int)blockIdx.x;
        if (!SPLIT) {
            group_order(xcd_order(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
        } else {
            // Tiles split_from .. total-1 (the tail) run as two column halves
            // each.  Block order: the tail's first halves, then the whole tiles,
            // then the tail's second halves.  Half the CUs then run [1/2, 1, 1,
            // ...] and the other half [1, 1, ..., 1/2], so their tiles end, and
            // their epilogue stores hit memory, at alternating times rather than
            // all at once (Wgrad at the DSv3 shape 3% faster).  Both halves of a
            // tail tile use the same XCD (rem and split_from are multiples of 8).
            const int full = (int)g.split_from, rem = tiles_m * tiles_n - full;
            if (bid >= rem && bid < rem + full) {
                group_order(xcd_order(bid - rem, full), tiles_m, tiles_n, tm, tn);
            } else {
                const int h = bid < rem ? bid : bid - rem - full;
                half = bid < rem ? 0 : 1;
                group_order(full + xcd_order(h, rem), tiles_m, tiles_n, tm, tn);
            }
        }
        m0 = (int64_t)tm * kTM;
    } else if constexpr (GROUP == kGroupRows) {
        int total = g.offsets[g.E];
        total = total < 0 ? 0 : (total > g.M ? (int)g.M : total);     // never past the rows that exist
        const int ntm = row_tiles_total(g, total);
        if ((int)blockIdx.x >= ntm * tiles_n) return;                  // the grid is an upper bound
        const RowTile rt = grouped_tile(g, total, xcd_order(blockIdx.x, ntm * tiles_n), tiles_n, tn);
        if (rt.mend <= rt.m0) return;                                  // t < ntm * tiles_n always finds one
        m0 = rt.m0; mend = rt.mend;
        Bp += rt.e * g.b_expert_stride;
        sbp += rt.e * g.sb_expert_stride;
    } else {
        // experts in order, each expert's tiles spread over all 8 XCDs (experts
        // differ in contraction length, so whole experts per XCD would leave
        // the XCDs unevenly loaded).  Block b runs on XCD b % 8: each expert's
        // blocks start at a multiple of 8 (the grid pads every expert to one),
        // so that its tile order meets the XCDs it assumes.
        const int tiles_m = (int)((g.M + kTM - 1) / kTM), per_e = tiles_m * tiles_n;
        const int per_pad = (per_e + 7) & ~7;
        const int e = (int)blockIdx.x / per_pad, local = (int)blockIdx.x - e * per_pad;
        if (local >= per_e) return;                                    // padding block
        group_order(xcd_order(local, per_e), tiles_m, tiles_n, tm, tn);
        m0 = (int64_t)tm * kTM;
        // contraction blocks of expert e, clamped to the nkb blocks that exist
        int64_t b0 = g.offsets[e] / kTile, b1 = g.offsets[e + 1] / kTile;
        b0 = b0 < 0 ? 0 : (b0 > g.nkb ? g.nkb : b0);
        b1 = b1 < b0 ? b0 : (b1 > g.nkb ? g.nkb : b1);
        kb0 = b0; kb1 = b1;
        outp = reinterpret_cast<uint8_t*>(g.out) + e * g.out_expert_stride * (int64_t)sizeof(float);
    }
    // A half block covers TN/2 columns from n0 with the waves of the first half
    // of the wave columns; the other waves only share the loads and barriers.
    const int64_t n0 = (int64_t)tn * TN + (half > 0 ? TN / 2 : 0);
    const int b_rows = SPLIT && half >= 0 ? TN / 2 : TN;     // staged B rows this block needs
    const bool active = !SPLIT || half < 0 || wn < S::WAVES_N / 2;

    // ---- load plan: A rows in 32 groups of 8, B rows in TN/8 groups; group q is
    // loaded by wave q % 8 with one direct-to-LDS instruction.  Lane -> staged
    // row r = 8*q + lane/8 at slot lane&7, which holds source chunk
    // (lane&7) ^ swz(r); 32-bit byte offsets from the operand base (operands are
    // cut below 4 GiB on the host).
    constexpr int NB = (TN / 8 + 7) / 8;            // B groups per wave (upper bound)
    constexpr int NL = 4 + NB + 1;                  // load instructions per wave and block
    uint32_t a_off[4], b_off[NB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave + 8 * i) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(r);
        int64_t ar = m0 + r; ar = ar < mend ? ar : mend - 1;
        a_off[i] = (uint32_t)ar * (uint32_t)g.lda + (uint32_t)(chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int r = (wave + 8 * i) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(r);
        int64_t br = n0 + r; br = br < g.N ? br : g.N - 1;
        b_off[i] = (uint32_t)br * (uint32_t)g.ldb + (uint32_t)(chunk * 16);
    }
    // Scales.  Waves 0..3 stage SA, permuted so that a lane fetches the scales of
    // its row in all MI row pieces with MI/4 16-byte reads: float p of the SA
    // area holds row WTM*h + 16*i + q for p = WTM*h + 64*(i>>2) + 4*q + (i&3).
    // Waves 4..7 stage SB: the column scales (Wgrad), or (Fprop/Dgrad) in word
    // SBW*c + j the weight-tile scale of piece j of wave column c, so that a wave
    // reads the scales of its NJ pieces from consecutive words.
    constexpr int SBW = NJ <= 4 ? 4 : 8;            // SB words per wave column
    static_assert(S::WAVES_N * SBW <= 16, "per-piece weight scales fit 16 words");
    const float* s_base;
    int64_t s_kb;
    uint32_t s_off;
    {
        const int sidx = (wave & 3) * 64 + lane;
        if (wave < 4) {
            const int h = sidx / WTM, q7 = sidx % WTM;
            const int i = ((q7 >> 6) << 2) | (q7 & 3), q = (q7 >> 2) & 15;
            int64_t r = m0 + h * WTM + 16 * i + q; r = r < mend ? r : mend - 1;
            s_base = g.sa; s_kb = g.sa_ld; s_off = (uint32_t)r;
        } else if (OUTER) {
            int64_t c = n0 + sidx; c = c < g.N ? c : g.N - 1;
            s_base = sbp; s_kb = g.sb_kb; s_off = (uint32_t)c;
        } else {
            const int w = lane & 15;
            const int pc = w / SBW, pj = w % SBW < NJ ? w % SBW : NJ - 1;
            int64_t t = (n0 + 16 * (pc * NJ + pj)) / kTile;
            const int64_t tmax = (g.N + kTile - 1) / kTile - 1;
            t = t < tmax ? t : tmax;
            s_base = sbp; s_kb = g.sb_kb; s_off = (uint32_t)t * (uint32_t)g.sb_n;
        }
    }

    // Load k (0 <= k < NL) of block kb into the stage at sbase.  SPREAD: issued
    // from inside the computation; B groups past b_rows are then loaded anyway
    // (from clamped, valid rows into staged rows no fragment read touches), so
    // that no branch splits the computation.
    auto issue_one = [&](int k, int64_t kb, uint32_t sbase, auto spread) __attribute__((always_inline)) {
        constexpr bool SP = decltype(spread)::value;
        if (k < 4) {
            const uint8_t* A = g.A + kb * kTile;
            const uint32_t d = sbase + (uint32_t)((wave + 8 * k) * 8 * kTile);
            if constexpr (SP) dma16_nc(A, a_off[k], d);
            else dma16(A, a_off[k], d);
        } else if (k < 4 + NB) {
            const int i = k - 4;
            const uint8_t* B = Bp + kb * kTile;
            const uint32_t d = sbase + (uint32_t)(kStageA + (wave + 8 * i) * 8 * kTile);
            if constexpr (SP) dma16_nc(B, b_off[i], d);
            else if ((wave + 8 * i) * 8 < b_rows) dma16(B, b_off[i], d);
        } else {
            const float* sp = s_base + kb * s_kb;
            const uint32_t d = sbase + (uint32_t)(kStageA + kStageB + wave * 256);
            if constexpr (SP) dma4_nc(sp, s_off * 4u, d);
            else dma4(sp, s_off * 4u, d);
        }
    };
    auto issue = [&](int64_t kb, uint32_t sbase) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NL; ++k) issue_one(k, kb, sbase, std::false_type{});
    };

    v4f acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int frow = lane & 15, fg = lane >> 4;
    // Byte offsets, from a stage's start, of a lane's two 16-byte chunks in its
    // first A and first B fragment row; later fragments are 16 rows (2 KB) on,
    // and the second chunk sits in slot (first ^ 1), i.e. at offset ^ 16.
    const uint32_t fo_lo = (uint32_t)(((2 * fg) ^ swz(frow)) << 4);
    const uint32_t a_lo = (uint32_t)((wm * WTM + frow) * kTile) + fo_lo, a_hi = a_lo ^ 16u;
    const uint32_t b_lo = (uint32_t)(kStageA + (wn * WTN + frow) * kTile) + fo_lo, b_hi = b_lo ^ 16u;

    // One 128-block: MI*NJ MFMAs in a flat schedule where step t issues MFMA t
    // and folds the partial of MFMA t-3 (a ring of four partials), so no fold
    // waits on a result still in the matrix pipeline and no wait states need
    // padding between an MFMA and the first read of its result.  The operands of the first
    // MFMA are requested first.  The shorter side's fragments (B for TN = 256,
    // A for TN = 224) stay in registers for the whole block; the other side's
    // stream two pieces ahead through a ring of three.  With a next block
    // (NEXT), its load k is issued at step 1 + 2k.
    constexpr int kLag = 3;                        // steps between an MFMA and the fold of its result
    constexpr bool ROW_MAJOR = MI >= NJ;           // steps walk columns inside a row piece
    constexpr int NH = ROW_MAJOR ? NJ : MI;        // held fragments
    constexpr int NS = ROW_MAJOR ? MI : NJ;        // streamed fragments
    constexpr int T = MI * NJ;
    constexpr int PER = ROW_MAJOR ? NJ : MI;       // steps per streamed fragment
    // (Wgrad without the half-tile split: loads at steps 0 .. NL-1, which keeps
    // that instantiation within 256 VGPRs without spilling)
    constexpr bool kDense1 = OUTER && !SPLIT;
    constexpr int kSpreadFirst = kDense1 ? 0 : 1, kSpreadEvery = kDense1 ? 1 : 2;
    static_assert(kSpreadFirst + kSpreadEvery * (NL - 1) < T, "every spread load falls on a step");
    // The two waves of a SIMD share its issue port, and among waves of equal
    // priority the older one wins, so one wave of each pair would finish its
    // block early and then sit at the barrier while the other runs alone.  Each
    // wave takes the higher priority for the first half of its steps and drops
    // back for the second, so the one that is ahead yields.  (Not for Wgrad's
    // matrix-core outer products, where it measured no gain.)
    constexpr bool kBalance = !(OUTER && !PO2);
    auto balance_priority = [&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        if constexpr (kBalance && t == 0) __builtin_amdgcn_s_setprio(1);
        if constexpr (kBalance && t == T / 2) __builtin_amdgcn_s_setprio(0);
    };
    auto compute = [&](const uint8_t* sA, uint32_t nxt, int64_t kbn, auto next) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next)::value;
        const float* sSA = reinterpret_cast<const float*>(sA + kStageA + kStageB);
        const float* sSB = sSA + 4 * 64;           // region of wave 4 onwards
        const uint8_t *pal = sA + a_lo, *pah = sA + a_hi, *pbl = sA + b_lo, *pbh = sA + b_hi;
        auto afrag = [&](int i) { return frag_at(pal, pah, i * 16 * kTile); };
        auto bfrag = [&](int j) { return frag_at(pbl, pbh, j * 16 * kTile); };
        auto held = [&](int h) { return ROW_MAJOR ? bfrag(h) : afrag(h); };
        auto streamed = [&](int q) { return ROW_MAJOR ? afrag(q) : bfrag(q); };

        v8i hf[NH];
        v8i sf[3];
        sf[0] = streamed(0);
        hf[0] = held(0);
#pragma unroll
        for (int h = 1; h < NH; ++h) hf[h] = held(h);
        if (NS > 1) sf[1] = streamed(1);
        float sa[MI];
#pragma unroll
        for (int h = 0; h < MI / 4; ++h) {
            const float4 t = *reinterpret_cast<const float4*>(sSA + wm * WTM + 64 * h + frow * 4);
            sa[4 * h] = t.x; sa[4 * h + 1] = t.y; sa[4 * h + 2] = t.z; sa[4 * h + 3] = t.w;
        }
        // Fprop/Dgrad: the weight-tile scale of column piece j
        auto col_scales = [&](int j, float (&c)[4]) { c[0] = sSB[wn * SBW + j]; };
        // TN = 256, weight-tile scales: a wave's 64 columns start 64-aligned and
        // lie inside one 128-wide weight tile, so every piece of the block folds
        // with f[i] = SA(row piece i) * SB(the wave's tile): MI products per block
        // instead of one per piece
        constexpr bool ONE_TILE = !OUTER && TN == 256;
        static_assert(!ONE_TILE || (WTN == 64 && ROW_MAJOR), "one weight tile per wave");
        // Wgrad forms its outer-product scales on the matrix core (below): one
        // fp32 MFMA per four pieces costs less than the 4 vector multiplies per
        // piece it replaces
        constexpr bool MS = OUTER;
        float cs[ROW_MAJOR && !ONE_TILE && !MS ? NJ : 1][4];
        if constexpr (ROW_MAJOR && !ONE_TILE && !MS) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) col_scales(j, cs[j]);
        }
        if constexpr (ONE_TILE) {
            const float sbw = sSB[wn * SBW];
#pragma unroll
            for (int i = 0; i < MI; ++i) sa[i] *= sbw;
        }
        // column-major walk: the scales of column piece p live in cbuf[p & 1]
        // (not for matrix-core scales)
        float cbuf[2][4];
        if constexpr (!ROW_MAJOR && !MS) col_scales(0, cbuf[0]);

        // Outer-product scales (Wgrad): the products SA(row) * SB(column) of four
        // 16x16 pieces come from one fp32 4-block 16x16x1 MFMA, already in the
        // fold's lane layout -- output register 4*b + r of lane l is A_b[4*(l>>4)
        // + r] * B_b[l & 15] -- instead of 16 vector multiplies.  A group is the
        // PER pieces of one streamed fragment (a row piece for the row-major
        // walk, block b = column piece b; a column piece for the column-major
        // walk, block b = row piece b), so A_b carries the column scales and B_b
        // the row scales.  Two slots (224-wide tiles): the products of group g
        // are formed at the last step of group g-1 into S[g & 1]; a group's last
        // fold comes kLag < PER steps after its last MFMA, before group g+2
        // overwrites the slot.  One slot (256-wide tiles, whose 128 accumulators
        // leave no room for a second): group g's products are formed at step
        // PER*g + kLag - 1, right after the fold of group g-1's last piece, and
        // its first fold follows one step later.
        typedef float v16f __attribute__((ext_vector_type(16)));
        constexpr int NSLOT = TN == 224 ? 2 : 1;
        v16f S[MS ? NSLOT : 1];
        float ocol = 0.0f, orow = 0.0f, ocol_next = 0.0f;
        auto outer_products = [&](int g) __attribute__((always_inline)) {
            if constexpr (MS) {
                const v16f z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if constexpr (ROW_MAJOR)      // row piece g: columns of the wave (one per lane), row 16g + frow
                    S[g % NSLOT] = __builtin_amdgcn_mfma_f32_16x16x1f32(ocol, sa[g], z, 0, 0, 0);
                else                          // column piece g: its columns 16g + frow, rows 16b + frow
                    S[g % NSLOT] = __builtin_amdgcn_mfma_f32_16x16x1f32(ocol, orow, z, 0, 0, 0);
            }
        };
        if constexpr (MS) {
            static_assert(PER > kLag && PER == 4, "four pieces per outer-product MFMA; a slot frees in time");
            if constexpr (ROW_MAJOR) {
                ocol = sSB[wn * WTN + lane];                      // column 16*(lane>>4) + (lane&15) of the wave
            } else {
                ocol = sSB[wn * WTN + frow];                      // column piece 0
                ocol_next = sSB[wn * WTN + 16 + frow];
                orow = fg == 0 ? sa[0] : (fg == 1 ? sa[1] : (fg == 2 ? sa[2] : sa[3]));   // row 16*fg + frow
            }
            outer_products(0);
        }

        v4f P[4];
        auto fold = [&](int t, const float (&c)[4]) {
            const int i = ROW_MAJOR ? t / NJ : t % MI;
            const int j = ROW_MAJOR ? t % NJ : t / MI;
            if constexpr (MS) {
                const int g = t / PER, h = t % PER;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][r] = __builtin_fmaf(P[t & 3][r], S[g % NSLOT][4 * h + r], acc[i][j][r]);
            } else if constexpr (ONE_TILE) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[t & 3][r], sa[i], acc[i][j][r]);
            } else {
                const float f = sa[i] * c[0];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[t & 3][r], f, acc[i][j][r]);
            }
        };
        auto scales_of_step = [&](int t) -> const float (&)[4] {
            if constexpr (ONE_TILE || MS) return cs[0];
            else if constexpr (ROW_MAJOR) return cs[t % NJ];
            else return cbuf[(t / MI) & 1];
        };
        static_assert(ROW_MAJOR || MI > kLag, "column-major walk: a scale slot frees up inside a piece");
        static_for<T>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int q = t / PER, h = t % PER;        // streamed piece, held piece
            balance_priority(tc);
            if constexpr (NEXT && t >= kSpreadFirst && (t - kSpreadFirst) % kSpreadEvery == 0 &&
                          (t - kSpreadFirst) / kSpreadEvery < NL)
                issue_one((t - kSpreadFirst) / kSpreadEvery, kbn, nxt, std::true_type{});
            if constexpr (h == 0 && q + 2 < NS) sf[(q + 2) % 3] = streamed(q + 2);
            // piece q-1's last fold runs at step q*PER + kLag - 1, so its scale
            // slot is free from step q*PER + kLag on: load piece q+1's scales there
            if constexpr (!ROW_MAJOR && !MS && h == kLag && q + 1 < NS) col_scales(q + 1, cbuf[(q + 1) & 1]);
            if constexpr (MS && NSLOT == 2 && h == PER - 1 && q + 1 < NS) {
                if constexpr (!ROW_MAJOR) {
                    ocol = ocol_next;                                             // column piece q + 1
                    if (q + 2 < NS) ocol_next = sSB[wn * WTN + 16 * (q + 2) + frow];
                }
                outer_products(q + 1);
            }
            P[t & 3] = ROW_MAJOR
                ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(hf[h], sf[q % 3], zero, 0, 0, 0, 0, 0, 0)
                : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sf[q % 3], hf[h], zero, 0, 0, 0, 0, 0, 0);
            if constexpr (t >= kLag) fold(t - kLag, scales_of_step(t - kLag));
            if constexpr (MS && NSLOT == 1 && h == kLag - 1 && q >= 1) outer_products(q);
            // keep the steps in this order: the scheduler would otherwise pull
            // each fold up behind its own MFMA and pad the wait with s_nop
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<kLag>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            fold(T - kLag + u, scales_of_step(T - kLag + u));
        });
    };

    // Power-of-two scales: one MFMA per 16x16 piece and block, accumulating
    // through C; the scale operand of a lane is the exponent field (the E8M0
    // byte) of its fragment row's scale: B rows are output columns 16j + frow,
    // A rows are output rows 16i + frow.  Loads of the next block as above.
    auto compute_po2 = [&](const uint8_t* sA, uint32_t nxt, int64_t kbn, auto next) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next)::value;
        const float* sSA = reinterpret_cast<const float*>(sA + kStageA + kStageB);
        const float* sSB = sSA + 4 * 64;
        const uint8_t *pal = sA + a_lo, *pah = sA + a_hi, *pbl = sA + b_lo, *pbh = sA + b_hi;
        auto afrag = [&](int i) { return frag_at(pal, pah, i * 16 * kTile); };
        auto bfrag = [&](int j) { return frag_at(pbl, pbh, j * 16 * kTile); };
        auto held = [&](int h) { return ROW_MAJOR ? bfrag(h) : afrag(h); };
        auto streamed = [&](int q) { return ROW_MAJOR ? afrag(q) : bfrag(q); };
        v8i hf[NH];
        v8i sf[3];
        sf[0] = streamed(0);
#pragma unroll
        for (int h = 0; h < NH; ++h) hf[h] = held(h);
        if (NS > 1) sf[1] = streamed(1);
        int ea[MI], eb[NJ];
#pragma unroll
        for (int h = 0; h < MI / 4; ++h) {
            const float4 t = *reinterpret_cast<const float4*>(sSA + wm * WTM + 64 * h + frow * 4);
            ea[4 * h] = (int)(__float_as_uint(t.x) >> 23); ea[4 * h + 1] = (int)(__float_as_uint(t.y) >> 23);
            ea[4 * h + 2] = (int)(__float_as_uint(t.z) >> 23); ea[4 * h + 3] = (int)(__float_as_uint(t.w) >> 23);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if constexpr (OUTER)
                eb[j] = (int)(__float_as_uint(sSB[wn * WTN + j * 16 + frow]) >> 23);
            else
                eb[j] = (int)(__float_as_uint(sSB[wn * SBW + j]) >> 23);
        }
        static_for<T>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int q = t / PER, h = t % PER;
            balance_priority(tc);
            if constexpr (NEXT && t >= kSpreadFirst && (t - kSpreadFirst) % kSpreadEvery == 0 &&
                          (t - kSpreadFirst) / kSpreadEvery < NL)
                issue_one((t - kSpreadFirst) / kSpreadEvery, kbn, nxt, std::true_type{});
            if constexpr (h == 0 && q + 2 < NS) sf[(q + 2) % 3] = streamed(q + 2);
            constexpr int i = ROW_MAJOR ? q : h, j = ROW_MAJOR ? h : q;
            acc[i][j] = ROW_MAJOR
                ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(hf[h], sf[q % 3], acc[i][j], 0, 0, 0, eb[j], 0, ea[i])
                : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sf[q % 3], hf[h], acc[i][j], 0, 0, 0, eb[j], 0, ea[i]);
        });
    };

    // K loop, one barrier per block: wait for this wave's loads of block kb, then
    // the barrier (all waves' loads of kb have landed, and all waves are done
    // with block kb-1, so its stage can be refilled).  Waves that compute issue
    // the loads of kb+1 into that stage from inside the computation of kb; waves
    // of a half-tile block that do not compute issue them at once.  The last
    // block (no kb+1) is a separate instantiation without loads.
    auto kstep = [&](int64_t kb, auto next) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next)::value;
        const int st = (int)((kb - kb0) & 1);
        const uint32_t nxt = smem_lds + (uint32_t)((st ^ 1) * kStageBytes);
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): this wave's loads of block kb
        lds_barrier();
        if (!SPLIT || active) {
            if constexpr (PO2) compute_po2(smem + st * kStageBytes, nxt, kb + 1, next);
            else compute(smem + st * kStageBytes, nxt, kb + 1, next);
        } else if constexpr (NEXT) {
            issue(kb + 1, nxt);
        }
    };
    if (kb1 > kb0) issue(kb0, smem_lds);
    int64_t kb = kb0;
    for (; kb + 1 < kb1; ++kb) kstep(kb, std::true_type{});
    if (kb < kb1) kstep(kb, std::false_type{});
    // ---- Epilogue through LDS.  Stored straight from the MFMA layout, one store
    // instruction would write 16 rows x 32 bytes; instead the waves write the
    // tile into the (now idle) stage area in that layout, and every thread then
    // stores whole 16-byte pieces of output rows, a wave covering one to two
    // full rows.  Staged rows have a power-of-two pitch and their 16-byte
    // chunks are XOR-swizzled by (row & 15), so the 16 rows a fragment write
    // touches land in 16 different chunk positions.  BF16 tiles go in one pass;
    // FP32 tiles in two passes of 128 rows.  Waves of a half-tile block that
    // compute nothing still share the stores.
    constexpr int OB = BF16_OUT ? 2 : 4;                       // bytes per output element
    constexpr int PITCH = BF16_OUT ? 512 : 1024;               // staged row pitch (>= TN * OB)
    constexpr int CH = PITCH / 16;                             // 16-byte chunks per staged row
    constexpr int PASS_ROWS = BF16_OUT ? kTM : kTM / 2;
    constexpr int PASSES = kTM / PASS_ROWS;
    static_assert(TN * OB <= PITCH && PASS_ROWS * PITCH <= 2 * kStageBytes, "staged tile fits");
    static_assert(PASS_ROWS % WTM == 0, "a wave's rows fall in one pass");
    const int ncols = (int)((g.N - n0) < (SPLIT && half >= 0 ? TN / 2 : TN)
                            ? (g.N - n0) : (SPLIT && half >= 0 ? TN / 2 : TN));
    const int nch = ncols * OB / 16;                           // chunks of a stored row (N % 128 == 0)
    const int nrows = (int)((mend - m0) < kTM ? (mend - m0) : kTM);
    uint8_t* const st = smem;                                  // LDS (the stage area)
    __syncthreads();                                           // every wave is done with the stages
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        if (pass > 0) __syncthreads();                         // the previous pass's rows are stored
        const int prow0 = pass * PASS_ROWS;
        if (active && wm * WTM >= prow0 && wm * WTM < prow0 + PASS_ROWS) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = wm * WTM - prow0 + i * 16 + frow;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int byte = (wn * WTN + j * 16 + fg * 4) * OB;
                    const int off = r * PITCH + (((byte >> 4) ^ (r & 15)) << 4) + (byte & 15);
                    if constexpr (BF16_OUT) {
                        const uint2 v = make_uint2(cvt_pk_bf16(acc[i][j][0], acc[i][j][1]),
                                                   cvt_pk_bf16(acc[i][j][2], acc[i][j][3]));
                        *reinterpret_cast<uint2*>(st + off) = v;
                    } else {
                        const float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                        *reinterpret_cast<float4*>(st + off) = v;
                    }
                }
            }
        }
        __syncthreads();                                       // the pass's rows are staged
        // Stores in rounds of kU chunks per thread: a round's chunks are all read
        // from LDS (and, when accumulating, the old outputs all loaded) before the
        // first of them is stored, so each round waits for those latencies once.
        // A thread keeps its chunk column c; round chunk k is RS*k rows further.
        // Threads whose column lies past the tile's last column store nothing;
        // whether every row of the pass exists is decided once per pass (uniform
        // over the block), so full passes store without a per-chunk branch.
        // The stores are non-temporal: the output (hundreds of MB at these
        // shapes) is written once and never read back by this kernel, and kept
        // in L2 and the MALL it would displace the operand panels that the
        // later tiles re-read (dense FFN GEMMs 1-7% faster, grouped 1-5%).
        constexpr int RS = kV1Threads / CH;                  // rows one store of every thread covers
        constexpr int kIt = PASS_ROWS / RS;                    // chunks per thread and pass
        constexpr int kU = BF16_OUT ? 8 : 4;
        static_assert(kV1Threads % CH == 0 && PASS_ROWS % RS == 0 && kIt % kU == 0, "whole store rounds");
        const int c = tid % CH, r0 = tid / CH;
        uint8_t* const ob = reinterpret_cast<uint8_t*>(outp) + ((m0 + prow0 + r0) * g.ldo + n0) * OB + c * 16;
        const int64_t ostep = (int64_t)RS * g.ldo * OB;
        auto store_rounds = [&](auto accumulate, auto all_rows) __attribute__((always_inline)) {
            constexpr bool ACC = decltype(accumulate)::value, ALL = decltype(all_rows)::value;
#pragma unroll
            for (int it0 = 0; it0 < kIt; it0 += kU) {
                uint4 v[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int r = r0 + (it0 + u) * RS;
                    v[u] = *reinterpret_cast<const uint4*>(st + r * PITCH + ((c ^ (r & 15)) << 4));
                }
                auto row_ok = [&](int u) { return ALL || prow0 + r0 + (it0 + u) * RS < nrows; };
                if constexpr (ACC) {
                    float4 pv[kU];
#pragma unroll
                    for (int u = 0; u < kU; ++u)
                        if (row_ok(u)) pv[u] = *reinterpret_cast<const float4*>(ob + (it0 + u) * ostep);
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        if (!row_ok(u)) continue;
                        const float4 x = __builtin_bit_cast(float4, v[u]);
                        st16_stream(ob + (it0 + u) * ostep, __builtin_bit_cast(uint4, make_float4(x.x + pv[u].x, x.y + pv[u].y,
                                                                                          x.z + pv[u].z, x.w + pv[u].w)));
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < kU; ++u)
                        if (row_ok(u)) st16_stream(ob + (it0 + u) * ostep, v[u]);
                }
            }
        };
        if (c < nch) {
            const bool all_rows = prow0 + PASS_ROWS <= nrows;
            if (!BF16_OUT && g.accumulate) {
                if (all_rows) store_rounds(std::true_type{}, std::true_type{});
                else store_rounds(std::true_type{}, std::false_type{});
            } else {
                if (all_rows) store_rounds(std::false_type{}, std::true_type{});
                else store_rounds(std::false_type{}, std::false_type{});
            }
        }
    }
}

// Number of compute units of the current device (cached per device).
static int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Pick the tile width: each block takes about TN units of time, and the blocks
// run in rounds of (number of CUs) -- one block per CU.  A 224-wide tile also
// costs 3-5% more per unit of work: with per-weight-tile scales (Fprop/Dgrad)
// its wave columns can straddle two weight tiles, so the fold forms one scale
// product per MFMA instead of one per row piece; for Wgrad the difference is
// measured, not derived.  It is priced 5% higher.
static int pick_tn(int64_t M, int64_t N)
{
    const int64_t cus = device_cus();
    const int64_t tm = (M + kTM - 1) / kTM;
    auto cost = [&](int64_t tn_w) { return ((tm * ((N + tn_w - 1) / tn_w) + cus - 1) / cus) * tn_w; };
    if (N % 224 == 0 && 21 * cost(224) < 20 * cost(256)) return 224;
    return 256;
}

template <int TN, bool PO2>
static void launch_v1(GemmKind kind, bool grouped, const GemmArgs& a, hipStream_t stream)
{
    const int64_t tiles_m = (a.M + kTM - 1) / kTM, tiles_n = (a.N + TN - 1) / TN;
    const dim3 block(kV1Threads);
    if (!grouped) {
        // Tiles beyond the last whole round of CUs: when they fill at most half a
        // round and come in multiples of 8, each is computed as two column halves
        // by two blocks, so that round takes about half a tile's time.
        const int64_t total = tiles_m * tiles_n, cus = device_cus();
        const int64_t full = (total / cus) * cus, rem = total - full;
        GemmArgs p = a;
        p.split_from = -1;
        int64_t nblocks = total;
        if (full > 0 && rem > 0 && 2 * rem <= cus && rem % 8 == 0 && full % 8 == 0) {
            p.split_from = full;
            nblocks = full + 2 * rem;
        }
        const dim3 grid((unsigned)nblocks);
        if (p.split_from >= 0) {
            if (kind == kWgrad)
                hipLaunchKernelGGL((k_gemm_block_scaled<TN, true, false, kDense, PO2, true>), grid, block, 0, stream, p);
            else
                hipLaunchKernelGGL((k_gemm_block_scaled<TN, false, true, kDense, PO2, true>), grid, block, 0, stream, p);
        } else if (kind == kWgrad) {
            hipLaunchKernelGGL((k_gemm_block_scaled<TN, true, false, kDense, PO2>), grid, block, 0, stream, p);
        } else {
            hipLaunchKernelGGL((k_gemm_block_scaled<TN, false, true, kDense, PO2>), grid, block, 0, stream, p);
        }
    } else if (kind == kWgrad) {
        const dim3 grid((unsigned)(((tiles_m * tiles_n + 7) & ~7ll) * a.E));   // every expert padded to 8 blocks
        hipLaunchKernelGGL((k_gemm_block_scaled<TN, true, false, kGroupK, PO2>), grid, block, 0, stream, a);
    } else {
        // upper bound on the row tiles: sum over experts of ceil(len/256) <= ceil(M/256) + E
        const dim3 grid((unsigned)((tiles_m + a.E) * tiles_n));
        hipLaunchKernelGGL((k_gemm_block_scaled<TN, false, true, kGroupRows, PO2>), grid, block, 0, stream, a);
    }
}

// The kernel addresses each operand through 32-bit byte offsets from its base:
// row r of A is at r*lda, so (rows-1)*ld + 128 must stay within 2^32.
static bool fits_32bit(int64_t rows, int64_t ld) { return rows <= 0 || (rows - 1) * ld + kTile <= (1ll << 32); }

static bool gemm_offsets_fit(const GemmArgs& a)
{
    return fits_32bit(a.M, a.lda) && fits_32bit(a.N, a.ldb);
}

// Dense pieces: rows in steps of whole 256-row tiles, columns in steps of 1792
// (a multiple of both tile widths and of the 128-wide weight tiles).
static int64_t dense_row_step(const GemmArgs& a)
{
    const int64_t max_rows = a.lda > 0 ? ((1ll << 32) - kTile) / a.lda + 1 : a.M;
    return a.M <= max_rows ? a.M : (max_rows / kTM) * kTM;
}
static int64_t dense_col_step(const GemmArgs& a)
{
    const int64_t max_cols = a.ldb > 0 ? ((1ll << 32) - kTile) / a.ldb + 1 : a.N;
    return a.N <= max_cols ? a.N : (max_cols / 1792) * 1792;
}

// Grouped grids (one block per tile, an upper bound on the row tiles for
// row-grouped GEMMs, every expert padded to 8 blocks for contraction-grouped
// ones) must fit the kernels' int block indices, at either tile width.
static bool grouped_grid_fits(const GemmArgs& a)
{
    const int64_t tiles_m = (a.M + kTM - 1) / kTM, tiles_n = (a.N + 223) / 224;
    const int64_t lim = (1ll << 31) - 1;
    return (tiles_m + a.E) * tiles_n <= lim && ((tiles_m * tiles_n + 7) & ~7ll) * a.E <= lim;
}

bool gemm_supported(const GemmArgs& a, bool grouped)
{
    if (grouped) return gemm_offsets_fit(a) && a.M < (1ll << 31) && a.E < (1ll << 16) && grouped_grid_fits(a);
    return dense_row_step(a) > 0 && dense_col_step(a) > 0;
}

static hipError_t launch_one(GemmKind kind, bool grouped, bool po2, const GemmArgs& a, hipStream_t stream)
{
    const int64_t units = grouped && kind == kWgrad ? a.M * a.E : a.M;
    const bool w224 = pick_tn(units, a.N) == 224;
    if (po2) {
        if (w224) launch_v1<224, true>(kind, grouped, a, stream);
        else launch_v1<256, true>(kind, grouped, a, stream);
    } else {
        if (w224) launch_v1<224, false>(kind, grouped, a, stream);
        else launch_v1<256, false>(kind, grouped, a, stream);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(GemmKind kind, bool grouped, const GemmArgs& a, hipStream_t stream, bool po2)
{
    if (!gemm_supported(a, grouped)) return hipErrorInvalidValue;
    if (grouped) return launch_one(kind, true, po2, a, stream);
    // Dense operands beyond 4 GiB: cut the output into row and column ranges
    // whose operand slices fit the kernel's 32-bit offsets.
    const int64_t rstep = dense_row_step(a), cstep = dense_col_step(a);
    const int64_t osz = kind == kWgrad ? (int64_t)sizeof(float) : (int64_t)sizeof(uint16_t);
    for (int64_t r0 = 0; r0 < a.M; r0 += rstep)
        for (int64_t c0 = 0; c0 < a.N; c0 += cstep) {
            GemmArgs p = a;
            p.M = a.M - r0 < rstep ? a.M - r0 : rstep;
            p.N = a.N - c0 < cstep ? a.N - c0 : cstep;
            p.A = a.A + r0 * a.lda;
            p.sa = a.sa + r0;
            p.B = a.B + c0 * a.ldb;
            p.sb = kind == kWgrad ? a.sb + c0 : a.sb + (c0 / kTile) * a.sb_n;
            p.out = reinterpret_cast<uint8_t*>(a.out) + (r0 * a.ldo + c0) * osz;
            const hipError_t e = launch_one(kind, false, po2, p, stream);
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

}  // namespace fgb
