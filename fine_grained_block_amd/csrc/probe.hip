// Clock probe for the benchmark (libfgb_probe.so): the shader clock the GPU
// sustains while every SIMD's matrix core is saturated with FP8 MFMAs, the
// load under which the block-scaled GEMMs run.  Not part of the method.
//
// Every wave (two per SIMD, one block of 512 threads per CU) issues eight
// independent accumulation chains of v_mfma_f32_16x16x128_f8f6f4 for `iters`
// rounds and brackets them with s_memtime (shader clock ticks) and
// s_memrealtime (the constant-rate counter whose frequency the runtime
// reports as the wall-clock rate).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "fgb_probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void k_clock_probe(int iters, unsigned long long* out)
{
    // pseudo-random E4M3 operands, different in every lane (the data toggles the
    // matrix core like a GEMM's would; clearing bit 3 of each byte keeps the
    // exponent field even, so no code is NaN)
    uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
    v8i a[2], b[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            h ^= h << 13; h ^= h >> 17; h ^= h << 5;
            a[p][k] = (int)(h & 0xF7F7F7F7u);
            h ^= h << 13; h ^= h >> 17; h ^= h << 5;
            b[p][k] = (int)(h & 0xF7F7F7F7u);
        }
    v4f c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = v4f{0.f, 0.f, 0.f, 0.f};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            c[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[k & 1], b[(k >> 1) & 1], c[k],
                                                                     0, 0, 0, 0, 0, 0);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
    // keep the chains live (a NaN sum never occurs: every operand is finite)
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
    if (s != s) out[0] = 0;
}

// One wave per block that mostly sleeps: it reads both counters, sleeps in
// short steps until `window` ticks of the constant-rate counter have passed
// (at most `max_steps` steps, so the loop always ends), and reads both again.
// It runs beside whatever kernel occupies the GPU and takes almost no issue
// slots from it.
__global__ __launch_bounds__(64) void k_clock_sample(unsigned long long window, int max_steps,
                                                     unsigned long long* out)
{
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < max_steps; ++i) {
        __builtin_amdgcn_s_sleep(8);
        if (__builtin_amdgcn_s_memrealtime() - r0 >= window) break;
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Staging throughput: one 512-thread block per compute unit repeats, `iters`
// times, the LDS traffic that the block-scaled GEMM's 256x256 tile has per
// 128-deep block, with the GEMM's own instruction forms and layouts:
//   MODE 1: the fragment reads -- each of the 8 waves reads its 128 A rows and
//           64 B rows of the 128-byte stage rows, 24 ds_read_b128 at the GEMM's
//           XOR-swizzled slots (192 KB per round and block);
//   MODE 2: the direct-to-LDS loads of the next block's two 32 KB operand
//           slices -- 8 global_load_lds_dwordx4 per wave from an L2-resident
//           source (64 KB per round and block) into the other stage;
//   MODE 3: both, as in the GEMM's main loop.
// Each round ends as a GEMM block does: this wave's loads waited for, LDS
// drained, barrier.  Thread 0 records the round loop's s_memtime ticks.
typedef __attribute__((address_space(3))) uint8_t lds_u8_p;
constexpr int kStage = 65536;                      // one stage: 256 A rows + 256 B rows of 128 bytes
constexpr int kSrcBlocks = 8;                      // distinct 64 KB source blocks cycled through
__device__ __forceinline__ void probe_dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "m0", "memory");
}
__device__ __forceinline__ int probe_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int MODE>
__global__ __launch_bounds__(512) void k_staging_probe(int iters, const uint8_t* src, unsigned long long* out,
                                                       uint32_t* sink)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
    const uint32_t base_lds = (uint32_t)(uintptr_t)(lds_u8_p*)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < 2 * kStage / 4; i += 512) reinterpret_cast<uint32_t*>(smem)[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    // fragment slots as in the GEMM (waves 2 x 4, 128 x 64 each)
    const int frow = lane & 15, fg = lane >> 4, wm = wave & 1, wn = wave >> 1;
    const uint32_t fo = (uint32_t)(((2 * fg) ^ probe_swz(frow)) << 4);
    const uint32_t a_lo = (uint32_t)((wm * 128 + frow) * 128) + fo;
    const uint32_t b_lo = (uint32_t)(kStage / 2) + (uint32_t)((wn * 64 + frow) * 128) + fo;
    // load plan as in the GEMM: row group (wave + 8 i), lane -> row lane/8, chunk lane&7
    uint32_t goff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        goff[i] = (uint32_t)(((wave + 8 * i) * 8 + (lane >> 3)) * 128 + (lane & 7) * 16);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        const int st = it & 1;
        if (MODE & 2) {
            const uint8_t* blk = src + (size_t)(it % kSrcBlocks) * kStage;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                probe_dma16(blk, goff[i], base_lds + (uint32_t)((st ^ 1) * kStage + (wave + 8 * i) * 1024));
        }
        if (MODE & 1) {
            const uint8_t* sp = smem + st * kStage;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 l = *reinterpret_cast<const uint4*>(sp + a_lo + i * 2048);
                const uint4 h = *reinterpret_cast<const uint4*>(sp + (a_lo ^ 16u) + i * 2048);
                x.x ^= l.x ^ h.x; x.y ^= l.y ^ h.y; x.z ^= l.z ^ h.z; x.w ^= l.w ^ h.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 l = *reinterpret_cast<const uint4*>(sp + b_lo + j * 2048);
                const uint4 h = *reinterpret_cast<const uint4*>(sp + (b_lo ^ 16u) + j * 2048);
                x.x ^= l.x ^ h.x; x.y ^= l.y ^ h.y; x.z ^= l.z ^ h.z; x.w ^= l.w ^ h.w;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    if (tid == 0) out[blockIdx.x] = t1 - t0;
    sink[(size_t)blockIdx.x * 512 + tid] = x.x ^ x.y ^ x.z ^ x.w;   // keeps the reads
}

struct Sample {
    unsigned long long* d = nullptr;
    int blocks = 0;
    int rt_khz = 0;
};
Sample g_sample;

}  // namespace

extern "C" int fgb_probe_clock_begin(int blocks, double window_us, void* stream)
{
    if (blocks <= 0 || blocks > 4096 || !(window_us > 0.0) || window_us > 1e6) return -1;
    if (g_sample.d != nullptr) return -1;                 // a sample is already running
    int dev = 0, rt_khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -2;
    if (hipDeviceGetAttribute(&rt_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rt_khz <= 0) return -2;
    unsigned long long* d = nullptr;
    if (hipMalloc(&d, sizeof(unsigned long long) * 2 * (size_t)blocks) != hipSuccess) return -2;
    const unsigned long long window = (unsigned long long)(window_us * (double)rt_khz / 1e3);
    // s_sleep 8 lasts about 512 shader cycles, well under a microsecond at any clock;
    // the cap is 64 such steps per microsecond of window
    const int max_steps = (int)(window_us * 64.0) + 64;
    hipLaunchKernelGGL(k_clock_sample, dim3((unsigned)blocks), dim3(64), 0, static_cast<hipStream_t>(stream),
                       window, max_steps, d);
    if (hipGetLastError() != hipSuccess) {
        hipFree(d);
        return -2;
    }
    g_sample.d = d;
    g_sample.blocks = blocks;
    g_sample.rt_khz = rt_khz;
    return 0;
}

extern "C" int fgb_probe_clock_end(double* mhz, void* stream)
{
    if (mhz == nullptr || g_sample.d == nullptr) return -1;
    const int blocks = g_sample.blocks;
    std::vector<unsigned long long> h(2 * (size_t)blocks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h.data(), g_sample.d, sizeof(unsigned long long) * h.size(), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    hipFree(g_sample.d);
    g_sample.d = nullptr;
    if (e != hipSuccess) return -2;
    std::vector<double> f;
    for (int b = 0; b < blocks; ++b)
        if (h[2 * b + 1] > 0) f.push_back((double)h[2 * b] / (double)h[2 * b + 1] * (double)g_sample.rt_khz / 1e3);
    if (f.empty()) return -2;
    std::sort(f.begin(), f.end());
    *mhz = f[f.size() / 2];
    return 0;
}

extern "C" int fgb_probe_clock(int iters, double* mhz, void* stream)
{
    if (mhz == nullptr || iters <= 0) return -1;
    int dev = 0, cus = 0, rt_khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -2;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -2;
    if (hipDeviceGetAttribute(&rt_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rt_khz <= 0) return -2;
    unsigned long long* d = nullptr;
    const size_t bytes = sizeof(unsigned long long) * 2 * (size_t)cus;
    if (hipMalloc(&d, bytes) != hipSuccess) return -2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_clock_probe, dim3((unsigned)cus), dim3(512), 0, s, iters, d);
    std::vector<unsigned long long> h(2 * (size_t)cus);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(h.data(), d, bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    hipFree(d);
    if (e != hipSuccess) return -2;
    std::vector<double> f;
    for (int b = 0; b < cus; ++b)
        if (h[2 * b + 1] > 0) f.push_back((double)h[2 * b] / (double)h[2 * b + 1] * (double)rt_khz / 1e3);
    if (f.empty()) return -2;
    std::sort(f.begin(), f.end());
    *mhz = f[f.size() / 2];
    return 0;
}

extern "C" int fgb_probe_staging(int iters, double* cycles, void* stream)
{
    if (cycles == nullptr || iters <= 0 || iters > 10000000) return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -2;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the source: kSrcBlocks 64 KB blocks (512 KB, L2-resident), every block reads the same
    uint8_t* src = nullptr;
    unsigned long long* d = nullptr;
    uint32_t* sink = nullptr;
    const size_t src_bytes = (size_t)kSrcBlocks * kStage;
    if (hipMalloc(&src, src_bytes) != hipSuccess) return -2;
    if (hipMalloc(&d, sizeof(unsigned long long) * (size_t)cus) != hipSuccess) { hipFree(src); return -2; }
    if (hipMalloc(&sink, sizeof(uint32_t) * 512 * (size_t)cus) != hipSuccess) { hipFree(src); hipFree(d); return -2; }
    hipError_t e = hipMemsetAsync(src, 0x3C, src_bytes, s);
    std::vector<unsigned long long> h((size_t)cus);
    for (int mode = 1; mode <= 3 && e == hipSuccess; ++mode) {
        for (int pass = 0; pass < 2 && e == hipSuccess; ++pass) {     // pass 0 warms caches and clocks
            const int n = pass == 0 ? (iters < 100 ? iters : 100) : iters;
            if (mode == 1) hipLaunchKernelGGL(k_staging_probe<1>, dim3((unsigned)cus), dim3(512), 0, s, n, src, d, sink);
            else if (mode == 2) hipLaunchKernelGGL(k_staging_probe<2>, dim3((unsigned)cus), dim3(512), 0, s, n, src, d, sink);
            else hipLaunchKernelGGL(k_staging_probe<3>, dim3((unsigned)cus), dim3(512), 0, s, n, src, d, sink);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipMemcpyAsync(h.data(), d, sizeof(unsigned long long) * h.size(), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e == hipSuccess) {
            std::sort(h.begin(), h.end());
            cycles[mode - 1] = (double)h[h.size() / 2] / (double)iters;
        }
    }
    hipFree(src);
    hipFree(d);
    hipFree(sink);
    return e == hipSuccess ? 0 : -2;
}
