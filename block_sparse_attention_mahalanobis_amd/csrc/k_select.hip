// Block scoring and fixed Top-K routing ("Spark-H3" blog, Discussion: blocks
// are scored from block-level means and the Top-K selected blocks get exact
// attention; 01 / Method: Spark-Reblock: a fixed Top-K budget per query block).
//
// One workgroup per (head, 8 consecutive query blocks): the rows S[A, :] =
// qbar_A . kbar_B / sqrt(d) are computed into LDS (each lane scores four key
// blocks against all 8 query means, so every k_bar read serves 8 rows and
// every query-mean read 4 blocks; or read from scores_in); then one wave per
// row finds the k-th best order key (score desc, block asc) by a radix
// select over the 32-bit keys, held in registers, and writes the selected
// blocks in ascending order with ballot prefix sums.  Integer decisions
// only; bit-exact for given scores.
#include "common.hpp"

namespace spark {

constexpr int SEL_T = 512;

// Order key for "largest score first, NaN last": ascending key == preference.
__device__ __forceinline__ uint32_t pref_key(float s) {
  if (s != s) return 0xffffffffu;
  return ~float_key_asc(s);
}

constexpr int SEL_NC = 2;   // radix histogram copies per wave

// One row's top-k by one wave: the key of rank topk (radix select), then
// the blocks below it and the first ties_needed blocks equal to it, in
// ascending block order, each placed by a ballot prefix sum.  KPL > 0: the
// row's keys are first loaded into registers (block B in lane B % 64, slot
// B / 64; nb <= 64 KPL), so neither the radix rounds nor the emission read
// LDS per key; KPL = 0: the keys are read from LDS.
template <int KPL>
__device__ __forceinline__ void row_topk(const uint32_t* s_key, int nb, int topk, int* hist,
                                         int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  int ties_needed;
  uint32_t thr;
  uint32_t kr[KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int B = 64 * j + lane;
      kr[j] = (B < nb) ? s_key[B] : 0xffffffffu;
    }
    thr = wave_radix_select<SEL_NC>(topk, hist, &ties_needed, [&](uint32_t prefix, uint32_t hmask, int shift, int* h) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int B = 64 * j + lane;
        if (B < nb && (kr[j] & hmask) == prefix) atomicAdd(&h[(kr[j] >> shift) & 255], 1);
      }
    });
  } else {
    thr = wave_radix_kth(s_key, nb, topk, hist, &ties_needed);
  }
  int taken = 0, ties_seen = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto step = [&](int B, uint32_t k) {
    const bool tie = (B < nb) && (k == thr);
    const uint64_t tmask = __builtin_amdgcn_ballot_w64(tie);
    const int tie_rank = ties_seen + __builtin_popcountll(tmask & below);
    const bool sel = (B < nb) && (k < thr || (tie && tie_rank < ties_needed));
    const uint64_t smask = __builtin_amdgcn_ballot_w64(sel);
    const int pos = taken + __builtin_popcountll(smask & below);
    if (sel && pos < topk) out[pos] = B;
    taken += __builtin_popcountll(smask);
    ties_seen += __builtin_popcountll(tmask);
  };
  if constexpr (KPL > 0) {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (64 * j < nb) step(64 * j + lane, kr[j]);   // uniform
  } else {
    for (int B0 = 0; B0 < nb; B0 += 64) {
      const int B = B0 + lane;
      step(B, (B < nb) ? s_key[B] : 0xffffffffu);
    }
  }
}

constexpr int SEL_QB = 16;   // query blocks per workgroup (they share each k_bar read)
constexpr size_t SEL_LDS = 136 * 1024;   // dynamic LDS of a select workgroup

// Byte offset of the query means after the qb rows of nb keys, rounded up to
// 16 bytes.
__host__ __device__ __forceinline__ size_t sel_qoff(int qb, int nb) {
  return ((size_t)qb * nb * 4 + 15) & ~(size_t)15;
}
constexpr int SEL_KB = 4;   // key blocks per lane (they share each query-mean read)

template <int D>
__global__ __launch_bounds__(SEL_T) void select_kernel(const float* __restrict__ qbar,
                                                       const float* __restrict__ kbar,
                                                       const float* __restrict__ scores_in,
                                                       int topk, int32_t* __restrict__ idx,
                                                       float* __restrict__ scores_out, int nb,
                                                       int qb, float rsd) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(smem);  // [qb][nb]
  __shared__ int s_whist[SEL_T / 64][256 * SEL_NC];        // SEL_NC radix histograms per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqb = (nb + qb - 1) / qb;
  const int h = blockIdx.x / nqb, A0 = (blockIdx.x % nqb) * qb;
  const int nq = min(qb, nb - A0);

  // --- scores of rows A0 .. A0+nq-1 ----------------------------------------
  if (scores_in) {
    for (int q = 0; q < nq; ++q) {
      const long rowoff = ((long)h * nb + A0 + q) * nb;
      for (int B = tid; B < nb; B += SEL_T) {
        const float sc = scores_in[rowoff + B];
        if (scores_out) scores_out[rowoff + B] = sc;
        s_keys[q * nb + B] = pref_key(sc);
      }
    }
  } else {
    // SEL_KB key blocks per lane: the nq query means sit in LDS (broadcast
    // reads, each one used for SEL_KB blocks), the lane streams its k_bar
    // rows; no cross-lane reductions.  Every score is one fp32 FMA chain
    // over d in ascending order.  A lane's row reads are per-lane 16-byte
    // loads, 64 rows apart across the wave: the four loads that cover 64
    // bytes of a row are issued together, so they share the cache lines
    // they fetch instead of fetching them again on later steps.
    // [qb][D], 16-byte aligned for the float4 reads (qb * nb need not be a
    // multiple of 4)
    float* s_q = reinterpret_cast<float*>(smem + sel_qoff(qb, nb));
    for (int e = tid; e < nq * D; e += SEL_T) s_q[e] = qbar[((long)h * nb + A0) * D + e];
    __syncthreads();
    for (int B0 = 0; B0 < nb; B0 += SEL_T * SEL_KB) {
      const float* kr[SEL_KB];
#pragma unroll
      for (int r = 0; r < SEL_KB; ++r)
        kr[r] = kbar + ((long)h * nb + min(B0 + r * SEL_T + tid, nb - 1)) * D;   // tail lanes reread a row
      float acc[SEL_KB][SEL_QB];
#pragma unroll
      for (int r = 0; r < SEL_KB; ++r)
#pragma unroll
        for (int q = 0; q < SEL_QB; ++q) acc[r][q] = 0.f;
      for (int c0 = 0; c0 < D; c0 += 16) {
        float4 kv[SEL_KB][4];
#pragma unroll
        for (int r = 0; r < SEL_KB; ++r)
#pragma unroll
          for (int u = 0; u < 4; ++u) kv[r][u] = *reinterpret_cast<const float4*>(kr[r] + c0 + 4 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 4 * u;
#pragma unroll
          for (int q = 0; q < SEL_QB; ++q) {
            if (q < nq) {
              const float4 qv = *reinterpret_cast<const float4*>(s_q + q * D + c);
#pragma unroll
              for (int r = 0; r < SEL_KB; ++r) {
                acc[r][q] = fmaf(qv.x, kv[r][u].x, acc[r][q]);
                acc[r][q] = fmaf(qv.y, kv[r][u].y, acc[r][q]);
                acc[r][q] = fmaf(qv.z, kv[r][u].z, acc[r][q]);
                acc[r][q] = fmaf(qv.w, kv[r][u].w, acc[r][q]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < SEL_KB; ++r) {
        const int B = B0 + r * SEL_T + tid;
        if (B < nb) {
#pragma unroll
          for (int q = 0; q < SEL_QB; ++q) {
            if (q < nq) {
              const float sc = acc[r][q] * rsd;
              if (scores_out) scores_out[((long)h * nb + A0 + q) * nb + B] = sc;
              s_keys[q * nb + B] = pref_key(sc);
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // one wave per row: radix select of the threshold key, then ballot prefix
  // sums emit the selected blocks in ascending order (no barriers); rows of
  // up to 4096 blocks hold their keys in registers
  for (int q = wave; q < nq; q += SEL_T / 64) {
    const uint32_t* s_key = s_keys + q * nb;
    int32_t* out = idx + ((long)h * nb + A0 + q) * topk;
    if (nb <= 64 * 8)
      row_topk<8>(s_key, nb, topk, s_whist[wave], out);
    else if (nb <= 64 * 16)
      row_topk<16>(s_key, nb, topk, s_whist[wave], out);
    else if (nb <= 64 * 32)
      row_topk<32>(s_key, nb, topk, s_whist[wave], out);
    else if (nb <= 64 * 64)
      row_topk<64>(s_key, nb, topk, s_whist[wave], out);
    else
      row_topk<0>(s_key, nb, topk, s_whist[wave], out);
  }
}

int select_launch(int H, int N, int D, int BK, const float* qbar, const float* kbar,
                  const float* scores_in, int topk, int32_t* idx, float* scores_out,
                  hipStream_t st) {
  const int nb = cdiv(N, BK);
  // the 16 bytes cover the alignment padding of the query means
  if ((size_t)nb * 4 + 128 * 4 + 16 > SEL_LDS)
    return spark_set_error(SPARK_E_SHAPE, "spark_select: %d blocks exceed the LDS row buffer", nb);
  int qb = (int)std::min<size_t>(SEL_QB, (SEL_LDS - 16) / ((size_t)nb * 4 + (size_t)D * 4));
  qb = std::max(qb, 1);
  const size_t lds = sel_qoff(qb, nb) + (size_t)qb * D * 4;
  const float rsd = 1.f / sqrtf((float)D);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)select_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)SEL_LDS);
    hipFuncSetAttribute((const void*)select_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)SEL_LDS);
    attr = true;
  }
  const int grid = H * ((nb + qb - 1) / qb);
  if (D == 128)
    hipLaunchKernelGGL(select_kernel<128>, dim3(grid), dim3(SEL_T), lds, st, qbar, kbar,
                       scores_in, topk, idx, scores_out, nb, qb, rsd);
  else
    hipLaunchKernelGGL(select_kernel<64>, dim3(grid), dim3(SEL_T), lds, st, qbar, kbar,
                       scores_in, topk, idx, scores_out, nb, qb, rsd);
  return spark_check_launch("select");
}

}  // namespace spark
