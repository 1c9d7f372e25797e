/* libfgb_probe.so -- a measurement aid for the benchmark, not part of the
 * method's path and not linked into libfgb.so.
 *
 * fgb_probe_clock: runs FP8 MFMAs on every compute unit of the current device
 * (two waves per SIMD, eight independent accumulation chains each, `iters`
 * rounds of eight MFMAs per wave) and returns in *mhz the median over compute
 * units of the shader clock during the run: s_memtime ticks divided by the
 * elapsed time of the constant-rate counter (s_memrealtime at the runtime's
 * wall-clock rate).  The GEMMs are priced against the MFMA peak at 2.4 GHz;
 * this is the clock the chip actually sustains under a saturating MFMA load.
 *
 * Allocates a small device buffer, launches on `stream` (a hipStream_t) and
 * synchronizes it.  Returns 0, -1 for a bad argument (mhz NULL, iters <= 0),
 * -2 for a HIP error.
 *
 * fgb_probe_clock_begin / fgb_probe_clock_end: the clock while some other
 * kernel runs.  begin launches `blocks` single-wave blocks on `stream` (give
 * it a stream other than the measured kernel's, after that kernel was
 * launched); each mostly sleeps and measures s_memtime ticks over `window_us`
 * microseconds of the constant-rate counter.  end waits for them on `stream`
 * and returns in *mhz the median over the blocks.  One sample at a time per
 * process: begin returns -1 while one is running, as for a bad argument
 * (blocks outside 1..4096, window outside (0, 1e6] us); end returns -1 with no
 * sample running or mhz NULL; both return -2 for a HIP error.
 *
 * fgb_probe_staging: the per-compute-unit throughput of the GEMM's staging
 * traffic.  One 512-thread block per compute unit repeats `iters` rounds of
 * what the block-scaled GEMM's 256x256 tile moves per 128-deep block, with the
 * same instructions and layouts: cycles[0] for the fragment reads alone
 * (24 ds_read_b128 per wave, 192 KB per round), cycles[1] for the
 * direct-to-LDS loads alone (8 global_load_lds_dwordx4 per wave from an
 * L2-resident 512 KB source, 64 KB per round), cycles[2] for both together;
 * each is the median over compute units of s_memtime ticks per round (shader
 * clock cycles).  Allocates small device buffers, launches on `stream` and
 * synchronizes it.  Returns 0, -1 for a bad argument (cycles NULL, iters
 * outside 1..10^7), -2 for a HIP error.
 */
#ifndef FGB_PROBE_H
#define FGB_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

int fgb_probe_clock(int iters, double* mhz, void* stream);
int fgb_probe_clock_begin(int blocks, double window_us, void* stream);
int fgb_probe_clock_end(double* mhz, void* stream);
int fgb_probe_staging(int iters, double* cycles, void* stream);

#ifdef __cplusplus
}
#endif

#endif
