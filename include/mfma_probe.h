/*
 * mfma_probe.h — measurement support for the roofline of the GEMM kernels
 * (not part of the GEMM interface).
 *
 * The peak that the GEMM kernels are measured against is the fp32 matrix-core
 * peak of MI355X, 157.3 TFLOP/s (256 CUs x 256 flop per CU per clock at
 * 2.4 GHz).  This probe runs nothing but independent fp32 MFMAs so that a
 * harness can see how much of that peak the chip sustains and at which clock.
 */
#ifndef MFMA_PROBE_H
#define MFMA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue `blocks` workgroups of 256 threads on `stream` (a hipStream_t; NULL
 * is the null stream).  Each wave issues iters x 8 v_mfma_f32_16x16x4_f32.
 *   sink   : device array of blocks * 256 floats (written, so nothing is
 *            optimised away);
 *   clocks : device array of 2 * blocks counters; block b writes the shader-
 *            clock cycles (s_memtime) and the 100 MHz constant-clock ticks
 *            (s_memrealtime) of its first wave's loop.
 * Both arrays are owned by the caller.  Returns 0, -1 for a bad argument
 * (NULL array, blocks outside 1..2^20, iters outside 1..2^24; nothing is
 * enqueued), or -6 when the launch fails.
 */
int mfma_probe_launch(float *sink, unsigned long long *clocks, int blocks, int iters, void *stream);

/* Flops of one launch: blocks * 4 waves * iters * 8 MFMAs * 2048. */
long long mfma_probe_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_PROBE_H */
