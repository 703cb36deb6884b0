/* fa_ceiling.h -- measurement aid of libfa_ceiling.so (not part of the attention API).
 *
 * The attention kernels are priced against the published dense bf16 matrix peak.  How
 * much of it the part sustains depends on the operands' bit activity (power draw sets
 * the clock).  fa_ceiling_mfma runs nothing but bf16 32x32x16 matrix products on
 * register-resident operands, at the forward kernel's occupancy (workgroups of 8 waves,
 * two waves per SIMD), so its rate bounds what any kernel can reach on data of that
 * kind.  Used by the benchmark's --ceilings leg.
 */
#ifndef FA_CEILING_H
#define FA_CEILING_H

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

#ifdef __cplusplus
}
#endif

#endif /* FA_CEILING_H */
