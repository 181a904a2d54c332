// MFMA-only skeleton: the FP8 matrix-core throughput the attention kernel's
// instruction (v_mfma_f32_32x32x64_f8f6f4) reaches on this device with no
// memory traffic and no vector work, plus the shader clock it ran at.  It is
// the measured denominator that sits beside the published peak, as the
// FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page sets its launch
// against an "MMA-only skeleton" (performance-ceiling paragraph).
//
// The operands are either one fixed pattern or four sets of pseudo-random
// finite E4M3 codes rotated every product.  The two differ: the matrix core's
// power draw depends on how its operand bits toggle, and with random codes
// (like the attention kernel's) the device lowers its shader clock.
#include <hip/hip_runtime.h>

#include "../../include/fp8attn_bench.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__device__ __forceinline__ unsigned mix32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Every wave runs `iters` rounds of kChains independent MFMAs.
__global__ __launch_bounds__(256) void k_mfma_skeleton(float* sink, int iters, int random_operands, long long* clocks) {
  v8i a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; s++)
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // fixed: one pattern; random: codes with |code| < 0x78, all finite
      const unsigned r = mix32(threadIdx.x * 131u + blockIdx.x * 7919u + s * 17u + i * 1031u) & 0x77777777u;
      a[s][i] = (int)(random_operands ? r : ((threadIdx.x * 7u + i) & 0x3b3b3b3bu));
      b[s][i] = (int)(random_operands ? (mix32(r) & 0x77777777u) : ((threadIdx.x * 3u + i) & 0x3b3b3b3bu));
    }
  v16f c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; j++) c[j] = v16f{};
  const long long t0 = __builtin_readcyclecounter();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < kChains; j++)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(it + j) & 3], b[(it + 2 * j) & 3], c[j], 0, 0, 0, 0, 0, 0);
  }
  const long long t1 = __builtin_readcyclecounter();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; j++)
#pragma unroll
    for (int i = 0; i < 16; i++) s += c[j][i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;   // s_memrealtime ticks at 100 MHz
  }
}

}  // namespace

extern "C" int fp8attn_mfma_peak(int device, int iters, int random_operands, double* tflops_out,
                                 double* sclk_mhz_out) {
  if (tflops_out == nullptr || sclk_mhz_out == nullptr || iters < 1) return 1;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) return 5;
  hipDeviceProp_t prop;
  int status = 0;
  float* sink = nullptr;
  long long* clocks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  do {
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) { status = 5; break; }
    const int grid = prop.multiProcessorCount * 2;   // 8 waves per CU, 2 per SIMD
    if (hipMalloc(&sink, sizeof(float) * grid * 256) != hipSuccess) { status = 3; break; }
    if (hipMalloc(&clocks, 2 * sizeof(long long)) != hipSuccess) { status = 3; break; }
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) { status = 5; break; }
    hipLaunchKernelGGL(k_mfma_skeleton, dim3(grid), dim3(256), 0, 0, sink, iters, random_operands, clocks);   // warmup
    if (hipEventRecord(e0, 0) != hipSuccess) { status = 5; break; }
    hipLaunchKernelGGL(k_mfma_skeleton, dim3(grid), dim3(256), 0, 0, sink, iters, random_operands, clocks);
    if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) { status = 5; break; }
    float ms = 0.f;
    long long clk[2] = {0, 0};
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) { status = 5; break; }
    if (hipMemcpy(clk, clocks, sizeof clk, hipMemcpyDeviceToHost) != hipSuccess) { status = 5; break; }
    const double flops = (double)grid * 4 * iters * kChains * (32.0 * 32.0 * 64.0 * 2.0);
    *tflops_out = flops / (ms * 1e-3) / 1e12;
    *sclk_mhz_out = clk[1] > 0 ? (double)clk[0] / ((double)clk[1] / 100.0) : 0.0;
  } while (false);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (clocks) (void)hipFree(clocks);
  if (prev >= 0) (void)hipSetDevice(prev);
  return status;
}
