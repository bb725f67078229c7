// OCP E4M3 quantisation of row groups for the fp8 attention logits ("Spark-H3"
// blog, Benchmark Results: the DiT also runs in FP8).  Rows come in
// consecutive groups of G rows; each group is scaled by the smallest power of
// two s with max|x| <= 448 s -- exact in any binary floating point, found by
// comparisons against 448 * 2^e -- and every x / s (exact: a power of two) is
// rounded to the nearest E4M3 value, ties to even, by v_cvt_pk_fp8_f32.
#include "common.hpp"

namespace spark {

// Smallest power of two s with amax <= 448 s (1 for amax = 0, not finite: 1).
__device__ __forceinline__ float e4m3_pow2_scale(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 1.f;
  int e;
  frexpf(amax, &e);
  e -= 9;
  while (amax > 448.f * ldexpf(1.f, e)) ++e;
  while (amax <= 448.f * ldexpf(1.f, e - 1)) --e;
  return ldexpf(1.f, e);
}

// Two floats -> two E4M3 bytes in the low half of the result.
__device__ __forceinline__ uint32_t pk_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

constexpr int Q8_T = 256;

// One workgroup per (group g, head h): rows [g G, g G + G) of head h; rows at
// or past `in_rows` read as 0 (padding).  x8 holds out_rows rows per head.
template <typename Tin, int D>
__global__ __launch_bounds__(Q8_T) void quant_e4m3_kernel(const Tin* __restrict__ x, long in_rows,
                                                          long out_rows, int G,
                                                          uint8_t* __restrict__ x8,
                                                          float* __restrict__ scales, int ngroups) {
  __shared__ float s_max[Q8_T / 64];
  const int g = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const long r0 = (long)g * G;
  const int nrows = (int)min((long)G, out_rows - r0);
  const Tin* xh = x + (long)h * in_rows * D;
  constexpr int QPR = D / 4;                 // 4-element quads per row
  const int nq = nrows * QPR;
  float amax = 0.f;
  for (int e = tid; e < nq; e += Q8_T) {
    const long r = r0 + e / QPR;
    const int c = (e % QPR) * 4;
    if (r < in_rows)
#pragma unroll
      for (int u = 0; u < 4; ++u) amax = fmaxf(amax, fabsf(Elem<Tin>::load(xh + r * D + c + u)));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) s_max[tid >> 6] = amax;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int w = 0; w < Q8_T / 64; ++w) m = fmaxf(m, s_max[w]);
  const float s = e4m3_pow2_scale(m);
  const float inv = 1.f / s;                 // exact: s is a power of two
  if (tid == 0) scales[(long)h * ngroups + g] = s;
  uint8_t* oh = x8 + (long)h * out_rows * D;
  for (int e = tid; e < nq; e += Q8_T) {
    const long r = r0 + e / QPR;
    const int c = (e % QPR) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < in_rows)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = Elem<Tin>::load(xh + r * D + c + u) * inv;
    const uint32_t w = pk_e4m3(v[0], v[1]) | (pk_e4m3(v[2], v[3]) << 16);
    *reinterpret_cast<uint32_t*>(oh + r * D + c) = w;
  }
}

// H heads of in_rows rows (dtype SPARK_BF16 or SPARK_F32, or 2 = fp32 of any
// source), written as out_rows >= in_rows rows per head in groups of G.
int quant_e4m3_launch(int H, long in_rows, long out_rows, int D, int G, int dtype, const void* x,
                      uint8_t* x8, float* scales, hipStream_t st) {
  const int ngroups = (int)((out_rows + G - 1) / G);
  const dim3 grid(ngroups, H);
  if (dtype == SPARK_BF16) {
    if (D == 128)
      hipLaunchKernelGGL((quant_e4m3_kernel<uint16_t, 128>), grid, dim3(Q8_T), 0, st, (const uint16_t*)x,
                         in_rows, out_rows, G, x8, scales, ngroups);
    else
      hipLaunchKernelGGL((quant_e4m3_kernel<uint16_t, 64>), grid, dim3(Q8_T), 0, st, (const uint16_t*)x,
                         in_rows, out_rows, G, x8, scales, ngroups);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((quant_e4m3_kernel<float, 128>), grid, dim3(Q8_T), 0, st, (const float*)x, in_rows,
                         out_rows, G, x8, scales, ngroups);
    else
      hipLaunchKernelGGL((quant_e4m3_kernel<float, 64>), grid, dim3(Q8_T), 0, st, (const float*)x, in_rows,
                         out_rows, G, x8, scales, ngroups);
  }
  return spark_check_launch("quant_e4m3");
}

}  // namespace spark
