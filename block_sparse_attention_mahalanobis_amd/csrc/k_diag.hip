// Routing diagnostics of one layer ("Spark-H3" blog, 01 / Method:
// Spark-Reblock, the attention-mass recall of reblocked vs fixed blocks; and
// 02 / Method: Spark-Reweight, the log-mass error of a block summary), per
// query row p of the permuted order:
//   recall[p]  = the dense softmax probability that falls on the exact keys
//                of the query block's selected blocks
//              = exp(LSE_sel - LSE_all) over the exact logits q.k/sqrt(d);
//   logmass[p] = | LSE over the unselected blocks' exact logits
//                - LSE over the same blocks' compressed logits
//                  q.ksum_B/sqrt(d) + bias_B + log n_B |
//                (0 when every block is selected).
// They read every key of the head for every query (dense cost), so they sit
// outside the layer: tests, ablations and the density sweep call them.
//
// One workgroup per (head, query block), one thread per query row with its
// query in registers; keys are staged through LDS in chunks (broadcast
// reads); three online log-sum-exps per row in fp32.
#include "common.hpp"

namespace spark {

constexpr int DG_CH = 32;  // keys per LDS chunk

struct Lse {
  float m = -INFINITY, s = 0.f;
  __device__ __forceinline__ void add(float x) {
    if (x > m) {
      s = s * __expf(m - x) + 1.f;
      m = x;
    } else {
      s += __expf(x - m);
    }
  }
  __device__ __forceinline__ float value() const { return m + __logf(s); }
};

template <typename T, int D>
__global__ __launch_bounds__(128) void diag_kernel(const T* __restrict__ qp, const T* __restrict__ kp,
                                                   const int32_t* __restrict__ idx, int topk,
                                                   const float* __restrict__ ksum,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ recall,
                                                   float* __restrict__ logmass, int N, int BK, int nb,
                                                   float rsd) {
  __shared__ float sK[DG_CH][D];
  extern __shared__ unsigned char smask[];  // nb bytes: 1 = selected
  const int tid = threadIdx.x;
  const int h = blockIdx.x / nb, A = blockIdx.x % nb;
  const long Np = (long)nb * BK;
  const int row = A * BK + tid;
  const bool active = tid < BK && row < N;

  for (int i = tid; i < nb; i += blockDim.x) smask[i] = 0;
  __syncthreads();
  const int32_t* myidx = idx + ((long)h * nb + A) * topk;
  for (int t = tid; t < topk; t += blockDim.x) smask[myidx[t]] = 1;

  float q[D];
#pragma unroll
  for (int c = 0; c < D; ++c) q[c] = active ? Elem<T>::load(qp + ((long)h * Np + row) * D + c) : 0.f;

  Lse sel, uns, comp;
  const T* kh = kp + (long)h * Np * D;
  for (int c0 = 0; c0 < N; c0 += DG_CH) {
    __syncthreads();
    for (int e = tid; e < DG_CH * D; e += blockDim.x) {
      const int j = e / D, c = e % D;
      sK[j][c] = (c0 + j < N) ? Elem<T>::load(kh + (long)(c0 + j) * D + c) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
    const int jn = min(DG_CH, N - c0);
    for (int j = 0; j < jn; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], sK[j][c], acc);
      const float x = acc * rsd;
      if (smask[(c0 + j) / BK]) sel.add(x);
      else uns.add(x);
    }
  }
  if (!active) return;
  const float* kb = ksum + (long)h * nb * D;
  for (int B = 0; B < nb; ++B) {
    if (smask[B]) continue;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) acc = fmaf(q[c], kb[(long)B * D + c], acc);
    const int nB = (B == nb - 1) ? N - (nb - 1) * BK : BK;
    comp.add(acc * rsd + bias[(long)h * nb + B] + __logf((float)nB));
  }
  const float ls = sel.value();
  float la = ls;
  if (uns.s > 0.f) {
    const float lu = uns.value();
    la = fmaxf(ls, lu) + __logf(1.f + __expf(-fabsf(ls - lu)));
  }
  if (recall) recall[(long)h * N + row] = __expf(ls - la);
  if (logmass) logmass[(long)h * N + row] = (uns.s > 0.f) ? fabsf(uns.value() - comp.value()) : 0.f;
}

template <typename T, int D>
static int diag_t(int H, int N, int BK, const void* qp, const void* kp, const int32_t* idx, int topk,
                  const float* ksum, const float* bias, float* recall, float* logmass, hipStream_t st) {
  const int nb = cdiv(N, BK);
  hipLaunchKernelGGL((diag_kernel<T, D>), dim3(H * nb), dim3(128), (size_t)nb, st, (const T*)qp,
                     (const T*)kp, idx, topk, ksum, bias, recall, logmass, N, BK, nb,
                     1.f / sqrtf((float)D));
  return spark_check_launch("diagnostics");
}

int diag_launch(int H, int N, int D, int BK, int dtype, const void* qp, const void* kp,
                const int32_t* idx, int topk, const float* ksum, const float* bias, float* recall,
                float* logmass, hipStream_t st) {
  if (dtype == SPARK_F32)
    return D == 128 ? diag_t<float, 128>(H, N, BK, qp, kp, idx, topk, ksum, bias, recall, logmass, st)
                    : diag_t<float, 64>(H, N, BK, qp, kp, idx, topk, ksum, bias, recall, logmass, st);
  return D == 128 ? diag_t<uint16_t, 128>(H, N, BK, qp, kp, idx, topk, ksum, bias, recall, logmass, st)
                  : diag_t<uint16_t, 64>(H, N, BK, qp, kp, idx, topk, ksum, bias, recall, logmass, st);
}

}  // namespace spark
