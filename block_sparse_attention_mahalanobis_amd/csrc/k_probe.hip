// Measurement helper: the bf16 matrix-core rate this part sustains, for the
// roofline the attention kernel is reported against.  Every wave keeps four
// independent v_mfma_f32_32x32x16_bf16 accumulator chains with both operands
// in registers (no memory traffic at all), so the rate is set by the matrix
// cores and the clock they run at under load.  Not part of the layer.
#include "common.hpp"

namespace spark {

constexpr int PROBE_T = 256;

__global__ __launch_bounds__(PROBE_T, 2) void mfma_peak_kernel(int iters, float magic,
                                                               float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int v = 0; v < 16; ++v) c0[v] = c1[v] = c2[v] = c3[v] = 0.f;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  // a store the compiler cannot prove dead (magic is never reached)
  if (s == magic) sink[blockIdx.x * PROBE_T + threadIdx.x] = s;
}

// flops of one launch: workgroups x 4 waves x 4 chains x iters x 32*32*16*2
int mfma_peak_launch(int workgroups, int iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(PROBE_T), 0, st, iters, -1.0f, sink);
  return spark_check_launch("mfma peak probe");
}

}  // namespace spark
