/*
 * fa_probe.h -- C ABI of libfa_probe.so: a measurement aid, not part of the
 * attention computation.
 *
 * The attention kernels are compared against the matrix-core ceiling of the
 * device they run on.  The published dense bf16 figure assumes the peak
 * engine clock; under sustained MFMA load the clock settles lower.  This
 * probe measures the rate that matrix instructions actually reach on this
 * device: every wavefront issues independent 32x32x16 bf16 MFMAs
 * (v_mfma_f32_32x32x16_bf16, 32768 flops each) on register operands, two
 * wavefronts per SIMD on every compute unit, with no memory traffic in the
 * timed loop.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Runs the MFMA loop for `iters` iterations of 8 MFMAs per wavefront on the
 * current device, timed with HIP events around one launch after one warm-up
 * launch, and writes:
 *   tflops  dense bf16 TFLOP/s reached (flops of all MFMAs / event time)
 *   ghz     mean shader clock during the timed launch (GHz), from the
 *           wavefronts' shader-clock and 100 MHz real-time counters
 * Synchronous (returns after the device finished).  Allocates and frees a
 * small device buffer for the per-wavefront counters.
 * Returns 0 on success, 1 for a NULL output pointer or iters < 1, and 8 when
 * the HIP runtime reports an error.
 */
int fa_probe_mfma_peak(int32_t iters, double* tflops, double* ghz);

/*
 * The same loop with operands that switch: every wavefront holds eight A and
 * eight B fragments of pseudo-random bf16 values in +-[1, 2) (random sign and
 * mantissa bits from a hash of `seed` and the thread), and each of its 8
 * chains multiplies a different pair.  Attention feeds the matrix cores data
 * of this kind; the constant-operand loop above switches few operand bits
 * and so draws less power at the same rate.  Arguments, outputs, behaviour
 * and return codes as fa_probe_mfma_peak.
 */
int fa_probe_mfma_peak_random(int32_t iters, uint32_t seed, double* tflops, double* ghz);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
