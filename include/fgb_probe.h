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
 */
#ifndef FGB_PROBE_H
#define FGB_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

int fgb_probe_clock(int iters, double* mhz, void* stream);

#ifdef __cplusplus
}
#endif

#endif
