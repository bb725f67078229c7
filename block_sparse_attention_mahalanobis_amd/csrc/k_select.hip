// Block scoring and fixed Top-K routing ("Spark-H3" blog, Discussion: blocks
// are scored from block-level means and the Top-K selected blocks get exact
// attention; 01 / Method: Spark-Reblock: a fixed Top-K budget per query block).
//
// One workgroup per (head, query block A): the row S[A, :] = qbar_A . kbar_B /
// sqrt(d) is computed into LDS (or read from scores_in), then an exact radix
// select over 32-bit order keys finds the k-th best (score desc, block asc);
// the selected blocks are written in ascending block order through a
// workgroup prefix sum.  Integer decisions only; bit-exact for given scores.
#include "common.hpp"

namespace spark {

constexpr int SEL_T = 256;

// Order key for "largest score first, NaN last": ascending key == preference.
__device__ __forceinline__ uint32_t pref_key(float s) {
  if (s != s) return 0xffffffffu;
  return ~float_key_asc(s);
}

// Exclusive prefix sum over the workgroup of one int per thread.
__device__ __forceinline__ int block_exscan(int v, int* s_tmp, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < SEL_T / 64; ++i) {
    if (i < w) base += s_tmp[i];
    tot += s_tmp[i];
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

template <int D>
__global__ __launch_bounds__(SEL_T) void select_kernel(const float* __restrict__ qbar,
                                                       const float* __restrict__ kbar,
                                                       const float* __restrict__ scores_in,
                                                       int topk, int32_t* __restrict__ idx,
                                                       float* __restrict__ scores_out, int nb,
                                                       float rsd) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* s_key = reinterpret_cast<uint32_t*>(smem);  // [nb]
  __shared__ int s_hist[256];
  __shared__ int s_tmp[SEL_T / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x / nb, A = blockIdx.x % nb;
  const long rowoff = ((long)h * nb + A) * nb;

  // --- scores -------------------------------------------------------------
  if (scores_in) {
    for (int B = tid; B < nb; B += SEL_T) {
      const float s = scores_in[rowoff + B];
      if (scores_out) scores_out[rowoff + B] = s;
      s_key[B] = pref_key(s);
    }
  } else {
    // half-wave per key block, 4 consecutive dims per lane (D/4 lanes used)
    constexpr int LPB = D / 4;  // lanes per block row: 32 or 16
    constexpr int BPW = 64 / LPB;
    const int sub = lane / LPB, l = lane % LPB;
    const float4 qa = *reinterpret_cast<const float4*>(qbar + ((long)h * nb + A) * D + 4 * l);
    for (int B0 = wave * BPW; B0 < nb; B0 += (SEL_T / 64) * BPW) {
      const int B = B0 + sub;
      float acc = 0.f;
      if (B < nb) {
        const float4 kb = *reinterpret_cast<const float4*>(kbar + ((long)h * nb + B) * D + 4 * l);
        acc = qa.x * kb.x;
        acc = fmaf(qa.y, kb.y, acc);
        acc = fmaf(qa.z, kb.z, acc);
        acc = fmaf(qa.w, kb.w, acc);
      }
#pragma unroll
      for (int o = LPB / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (B < nb && l == 0) {
        const float s = acc * rsd;
        if (scores_out) scores_out[rowoff + B] = s;
        s_key[B] = pref_key(s);
      }
    }
  }
  if (tid == 0) {
    s_prefix = 0;
    s_need = topk;  // rank (1-based) of the threshold among keys matching the prefix
  }
  __syncthreads();

  // --- radix select of the topk-th smallest key, 8 bits per round ----------
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SEL_T) s_hist[i] = 0;
    __syncthreads();
    const uint32_t pre = s_prefix;
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    for (int B = tid; B < nb; B += SEL_T) {
      const uint32_t k = s_key[B];
      if ((k & hmask) == pre) atomicAdd(&s_hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // inclusive scan of 256 bins, 4 per lane
      int c[4], run = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { run += s_hist[4 * lane + i]; c[i] = run; }
      int incl = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int base = incl - run;
      const int need = s_need;
      // the digit whose cumulative count first reaches `need`
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int before = base + (i ? c[i - 1] : 0);
        const int after = base + c[i];
        if (before < need && after >= need) {
          s_prefix = pre | ((uint32_t)(4 * lane + i) << shift);
          s_need = need - before;
        }
      }
    }
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int ties_needed = s_need;  // how many keys == thr to take, lowest B first

  // --- emit in ascending B: thread owns a contiguous range -------------------
  const int per = (nb + SEL_T - 1) / SEL_T;
  const int b0 = tid * per, b1 = min(nb, b0 + per);
  int n_less = 0, n_eq = 0;
  for (int B = b0; B < b1; ++B) {
    const uint32_t k = s_key[B];
    n_less += (k < thr);
    n_eq += (k == thr);
  }
  int tot_less, tot_eq;
  const int off_less = block_exscan(n_less, s_tmp, tot_less);
  const int off_eq = block_exscan(n_eq, s_tmp, tot_eq);
  (void)tot_less;
  (void)tot_eq;
  // output position of B = (#less before B) + min(#eq before B, ties_needed)
  int cl = off_less, ce = off_eq;
  int32_t* out = idx + ((long)h * nb + A) * topk;
  for (int B = b0; B < b1; ++B) {
    const uint32_t k = s_key[B];
    if (k < thr) {
      const int pos = cl + min(ce, ties_needed);
      if (pos < topk) out[pos] = B;
      ++cl;
    } else if (k == thr) {
      if (ce < ties_needed && cl + ce < topk) out[cl + ce] = B;
      ++ce;
    }
  }
}

int select_launch(int H, int N, int D, int BK, const float* qbar, const float* kbar,
                  const float* scores_in, int topk, int32_t* idx, float* scores_out,
                  hipStream_t st) {
  const int nb = cdiv(N, BK);
  const size_t lds = (size_t)nb * 4;
  if (lds > 128 * 1024)
    return spark_set_error(SPARK_E_SHAPE, "spark_select: %d blocks exceed the LDS row buffer", nb);
  const float rsd = 1.f / sqrtf((float)D);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)select_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    hipFuncSetAttribute((const void*)select_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    attr = true;
  }
  if (D == 128)
    hipLaunchKernelGGL(select_kernel<128>, dim3(H * nb), dim3(SEL_T), lds, st, qbar, kbar,
                       scores_in, topk, idx, scores_out, nb, rsd);
  else
    hipLaunchKernelGGL(select_kernel<64>, dim3(H * nb), dim3(SEL_T), lds, st, qbar, kbar,
                       scores_in, topk, idx, scores_out, nb, rsd);
  return spark_check_launch("select");
}

}  // namespace spark
