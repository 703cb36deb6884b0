/* fa_ceiling.h -- measurement aids of libfa_ceiling.so (not part of the attention API).
 *
 * The attention kernels are priced against the published dense bf16 matrix peak.  How
 * much of it the part sustains depends on the operands' bit activity (power draw sets
 * the clock).  fa_ceiling_mfma runs nothing but bf16 32x32x16 matrix products on
 * register-resident operands, at the forward kernel's occupancy (workgroups of 8 waves,
 * two waves per SIMD), so its rate bounds what any kernel can reach on data of that
 * kind.  fa_ceiling_stream reads device memory once with a plain streaming kernel, the
 * HBM read rate a kernel that reads each byte once can reach.  Used by the benchmark's
 * --ceilings leg.
 */
#ifndef FA_CEILING_H
#define FA_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `workgroups` workgroups of 512 threads on `stream` (a hipStream_t; NULL for
 * the default stream), each wave running `iters` trips of 16 products.
 *   out      device float[workgroups * 512], caller-owned, written (one sum per thread,
 *            to keep every product live)
 *   pattern  0: bf16 operands of random sign, exponent and mantissa, magnitudes in
 *            [0.25, 4) (the spread of N(0,1) data); 1: every operand 1.0
 * Returns 0 on a launch, 1 on an invalid argument (nothing launched), 2 if the launch
 * failed.  Asynchronous: time it with events on `stream`. */
int fa_ceiling_mfma(float *out, int workgroups, int iters, int pattern, void *stream);

/* Matrix FLOPs of one fa_ceiling_mfma call with these arguments. */
double fa_ceiling_mfma_flops(int workgroups, int iters);

/* Launches `workgroups` workgroups of 256 threads on `stream` that read `bytes` bytes of
 * `src` once, as a plain streaming kernel: workgroup g reads the g-th of `workgroups`
 * equal contiguous slices with 16-byte non-temporal loads, eight in flight per thread.
 * Its rate bounds what a kernel that reads each byte once (the split-KV decode) can reach.
 *   src      device memory, caller-owned, 16-byte aligned, bytes long (contents ignored)
 *   bytes    a positive multiple of 32768 * workgroups
 *   out      device unsigned int[workgroups * 256], caller-owned, written (one word per
 *            thread, to keep every load)
 * Returns 0 on a launch, 1 on an invalid argument (nothing launched), 2 if the launch
 * failed.  Asynchronous: time it with events on `stream`. */
int fa_ceiling_stream(const void *src, int64_t bytes, unsigned int *out, int workgroups,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CEILING_H */
