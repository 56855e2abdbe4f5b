/* vstep_measure.h -- ceilings of the running GPU, for the measurement of libvstep.
 *
 * No page defines these: they measure the part, not the method.  Kernel fractions are
 * stated against the MI355X datasheet peaks and, with these, against what the same box
 * sustains.  Both calls only enqueue work on `stream` (NULL = the default stream);
 * the caller times them (HIP events) and derives the rate.
 */
#ifndef VSTEP_MEASURE_H
#define VSTEP_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read every byte of buf[0, bytes) once with 16-byte vector loads over n_wg workgroups
 * of 256 threads, eight loads in flight per thread, in one of two patterns:
 *   pattern 0: grid-strided (each step of the grid reads one contiguous span), loads
 *              marked non-temporal;
 *   pattern 1: workgroup w reads the contiguous slice [w*S, (w+1)*S), S = bytes/16/n_wg
 *              16-byte words (the remainder by the last workgroup), 4 KB per workgroup
 *              and step -- each workgroup one long sequential stream, as a weight
 *              stream is read.
 * One word per workgroup is XORed into sink[wg % 1024] (sink: uint32 [1024], device).
 * bytes >= 16 (a multiple of 16 is read whole; the tail below 16 bytes is not read).
 * Returns VS_ERR_INVALID_ARG (-1) for null pointers, sizes or a pattern out of range,
 * VS_ERR_HIP (-4) on a launch error, else 0. */
int vs_measure_read(const void *buf, size_t bytes, uint32_t *sink, int n_wg, int pattern,
                    void *stream);

/* n_wg workgroups of 4 waves, each wave issuing iters x 8 independent MFMA 32x32x16
 * bf16 products on register operands (32768 flops each): n_wg * 4 * iters * 8 * 32768
 * flops.  sink: float [n_wg] (device), written only on a value that does not occur.
 * Returns as vs_measure_read. */
int vs_measure_mfma(int n_wg, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VSTEP_MEASURE_H */
