/*
 * fp8attn_bench.h - measurement helper exported by libfp8attn.so (not part of
 * the attention API in fp8attn.h).
 *
 * fp8attn_mfma_peak - MFMA-only skeleton: runs v_mfma_f32_32x32x64_f8f6f4 (the
 * attention kernel's FP8 instruction) back to back on every CU, 8 waves per CU,
 * with no memory traffic or vector work, and reports
 *   tflops_out    achieved dense FP8 TFLOP/s (2*32*32*64 flops per MFMA);
 *   sclk_mhz_out  shader clock seen by one wave (s_memtime cycles over
 *                 s_memrealtime's 100 MHz ticks).
 * This is the measured ceiling reported beside the published FP8 peak, in the
 * way the FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page compares
 * its launch with an MMA-only skeleton.
 *
 * device           HIP device ordinal (the calling thread's current device is
 *                  restored).
 * iters            rounds of four independent MFMAs per wave (>= 1; 2000 takes
 *                  ~0.3 ms, 100000 ~30 ms).
 * random_operands  0: one fixed operand pattern; 1: four sets of pseudo-random
 *                  finite E4M3 codes rotated every product.  Random operands
 *                  draw more power and the device lowers its clock under a long
 *                  run, so the random, long measurement is the ceiling for
 *                  kernels that multiply random data.
 * Returns 0 on success, 1 for a bad argument, 3 if a small device allocation
 * failed, 5 for a HIP error.  Synchronous.
 */
#ifndef FP8ATTN_BENCH_H
#define FP8ATTN_BENCH_H

#ifdef __cplusplus
extern "C" {
#endif

int fp8attn_mfma_peak(int device, int iters, int random_operands, double* tflops_out, double* sclk_mhz_out);

#ifdef __cplusplus
}
#endif

#endif /* FP8ATTN_BENCH_H */
