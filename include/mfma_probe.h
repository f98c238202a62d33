/*
 * mfma_probe.h -- a measurement aid beside the attention library (its own
 * shared library, libmfma_probe.so): a kernel that issues nothing but bf16
 * matrix-core products, v_mfma_f32_32x32x16_bf16 on four independent
 * accumulators per wave with pseudo-random operands (a different pair for
 * each accumulator, so the products switch bits like real data).  Its rate
 * is the dense bf16 matrix-core throughput the chip sustains at the clock its
 * power limit allows under such a load, to set beside the published peak
 * (256 CUs x 4 SIMDs x 1024 flop per clock x 2.4 GHz = 2516.6 TFLOP/s).
 */
#ifndef MFMA_PROBE_H
#define MFMA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define MFMA_PROBE_THREADS 256          /* threads per workgroup (4 waves) */
#define MFMA_PROBE_FLOPS_PER_ITER 131072.0 /* per wave: 4 products x 2*32*32*16 */

/*
 * Launches `workgroups` workgroups of 256 threads on `stream` (a hipStream_t;
 * NULL = the null stream); each wave runs `iters` iterations of 4 products.
 * Flops of one launch: workgroups * 4 * iters * MFMA_PROBE_FLOPS_PER_ITER.
 * `sink` (device, workgroups * 256 floats) receives one sum per thread so
 * that the products are not removed.  Returns 0, -1 for a bad argument (NULL
 * sink, workgroups or iters < 1) or -4 when the launch fails.
 */
__attribute__((visibility("default")))
int mfma_probe_launch(int workgroups, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_PROBE_H */
