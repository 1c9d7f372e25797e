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
