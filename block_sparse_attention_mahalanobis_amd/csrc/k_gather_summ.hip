// Permutation gather + block pooling ("Spark-H3" blog, 01 / Method:
// Spark-Reblock: token IDs track membership through the tree, and blocks are
// scored from block-level means, Discussion section) and the compressed-branch
// summaries (02 / Method: Spark-Reweight: each block is scored once with the
// mean video query; the scores give weighted key/value summaries and a
// log-mass bias).  Both are HBM-streaming kernels: one workgroup per
// (head, block), 16-byte row loads, fp32 accumulation in a fixed order.
#include "common.hpp"

namespace spark {

// ---------------------------------------------------------------------------
// gather: x_p[h][p] = x[h][perm[h][p]] (rows past a block's real rows zero),
// x_pt the block-transposed layout [H, nbt, D, BK], xbar the fp32 block means.
// Blocks [0, nb) hold the Nv video tokens in permuted order, blocks
// [nb, nbt) the context tokens Nv..N-1 in original order (none unless the
// context mode is on: then Nv < N); xbar covers the video blocks only.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ perm,
                                                     T* __restrict__ xp, T* __restrict__ xpt,
                                                     float* __restrict__ xbar, int N, int Nv,
                                                     int BK, int nb, int nbt, int identity) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* tile = reinterpret_cast<T*>(smem);  // [BK][D + pad]
  constexpr int PAD = 16 / sizeof(T);
  constexpr int RS = D + PAD;
  constexpr int C16 = D * (int)sizeof(T) / 16;   // 16-byte chunks per row
  constexpr int MAXC = 128 * C16 / 256;          // chunks per thread for a 128-row block
  const int h = blockIdx.x / nbt, B = blockIdx.x % nbt;
  const int tid = threadIdx.x;
  const bool ctx = B >= nb;
  const long p0 = ctx ? (long)Nv + (long)(B - nb) * BK : (long)B * BK;  // first source position
  const int n_real = (int)min((long)BK, (ctx ? (long)N : (long)Nv) - p0);
  const long Np = (long)nbt * BK;
  // all of this thread's row loads are issued before any store, so up to
  // MAXC 16-byte loads per thread are in flight
  long src[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256, j = ch / C16;
    src[i] = -1;
    if (ch < BK * C16 && j < n_real)
      src[i] = (identity || ctx) ? p0 + j : (long)perm[(long)h * N + p0 + j];
  }
  uint4 buf[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256, cc = ch % C16;
    buf[i] = (src[i] >= 0)
                 ? *reinterpret_cast<const uint4*>(x + ((long)h * N + src[i]) * D + cc * (16 / (int)sizeof(T)))
                 : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = tid + i * 256, j = ch / C16, cc = ch % C16;
    if (ch < BK * C16) {
      if (xp)
        *reinterpret_cast<uint4*>(xp + ((long)h * Np + (long)B * BK + j) * D + cc * (16 / (int)sizeof(T))) = buf[i];
      if (xpt) *reinterpret_cast<uint4*>(tile + j * RS + cc * (16 / (int)sizeof(T))) = buf[i];
    }
  }
  if (xbar && !ctx) {
    // block means from the loaded chunks: a thread holds chunk column
    // tid % C16 of rows tid / C16 + (256 / C16) i, summed in i order, then
    // the lanes of a wave holding the same column (a fixed butterfly), then
    // the four waves in order
    __shared__ float s_part[4][D];
    constexpr int VE = 16 / (int)sizeof(T);
    float part[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) part[e] = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      if (src[i] >= 0) {
        const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            part[2 * e] += __uint_as_float(w[e] << 16);
            part[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) part[e] += __uint_as_float(w[e]);
        }
      }
    }
#pragma unroll
    for (int o = C16; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < VE; ++e) part[e] += __shfl_xor(part[e], o, 64);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < C16)
#pragma unroll
      for (int e = 0; e < VE; ++e) s_part[wave][lane * VE + e] = part[e];
    __syncthreads();
    for (int c = tid; c < D; c += blockDim.x)
      xbar[((long)h * nb + B) * D + c] = (((s_part[0][c] + s_part[1][c]) + s_part[2][c]) + s_part[3][c]) / (float)n_real;
  }
  if (xpt) {
    __syncthreads();
    // [D][BK]: a thread packs VE consecutive j of one column c into 16 bytes
    constexpr int VE = 16 / sizeof(T);
    if (BK % VE == 0) {
      const int runs = BK / VE;
      for (int e = tid; e < D * runs; e += blockDim.x) {
        const int c = e / runs, j0 = (e % runs) * VE;
        uint4 u;
        if constexpr (sizeof(T) == 2) {
          const uint16_t* tt = reinterpret_cast<const uint16_t*>(tile) + j0 * RS + c;
          u.x = (uint32_t)tt[0] | ((uint32_t)tt[RS] << 16);
          u.y = (uint32_t)tt[2 * RS] | ((uint32_t)tt[3 * RS] << 16);
          u.z = (uint32_t)tt[4 * RS] | ((uint32_t)tt[5 * RS] << 16);
          u.w = (uint32_t)tt[6 * RS] | ((uint32_t)tt[7 * RS] << 16);
        } else {
          const float* tt = reinterpret_cast<const float*>(tile) + j0 * RS + c;
          u.x = __float_as_uint(tt[0]);
          u.y = __float_as_uint(tt[RS]);
          u.z = __float_as_uint(tt[2 * RS]);
          u.w = __float_as_uint(tt[3 * RS]);
        }
        *reinterpret_cast<uint4*>(xpt + (((long)h * nbt + B) * D + c) * BK + j0) = u;
      }
    } else {
      for (int e = tid; e < D * BK; e += blockDim.x) {
        const int c = e / BK, j = e % BK;
        xpt[(((long)h * nbt + B) * D + c) * BK + j] = tile[j * RS + c];
      }
    }
  }
}

template <typename T, int D>
static int gather_t(int H, int N, int Nv, int BK, const void* x, const int32_t* perm, void* xp,
                    void* xpt, float* xbar, hipStream_t st) {
  const int nb = cdiv(Nv, BK), nbt = nb + cdiv(N - Nv, BK);
  constexpr int PAD = 16 / sizeof(T);
  const size_t lds = (size_t)BK * (D + PAD) * sizeof(T);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)gather_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    attr = true;
  }
  hipLaunchKernelGGL((gather_kernel<T, D>), dim3(H * nbt), dim3(256), xpt ? lds : 0, st, (const T*)x, perm,
                     (T*)xp, (T*)xpt, xbar, N, Nv, BK, nb, nbt, perm == nullptr ? 1 : 0);
  return spark_check_launch("gather");
}

// Nv = N: the plain layout; Nv < N: tokens [Nv, N) are context blocks.
int gather_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* x,
                  const int32_t* perm, void* xp, void* xpt, float* xbar, hipStream_t st) {
  if (dtype == SPARK_F32)
    return D == 128 ? gather_t<float, 128>(H, N, Nv, BK, x, perm, xp, xpt, xbar, st)
                    : gather_t<float, 64>(H, N, Nv, BK, x, perm, xp, xpt, xbar, st);
  return D == 128 ? gather_t<uint16_t, 128>(H, N, Nv, BK, x, perm, xp, xpt, xbar, st)
                  : gather_t<uint16_t, 64>(H, N, Nv, BK, x, perm, xp, xpt, xbar, st);
}

// 8 consecutive elements as loaded (16 bytes of bf16, 32 of fp32), widened
// to fp32 on use.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 q;
  __device__ __forceinline__ void load(const uint16_t* p) { q = *reinterpret_cast<const uint4*>(p); }
  // the first cnt (1..8) elements one by one, the rest zero: for rows whose
  // length is not a multiple of 8 (no read past the row, no 16-byte alignment)
  __device__ __forceinline__ void load_n(const uint16_t* p, int cnt) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (2 * i < cnt) ? p[2 * i] : 0u;
      const uint32_t hi = (2 * i + 1 < cnt) ? p[2 * i + 1] : 0u;
      w[i] = lo | (hi << 16);
    }
    q = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ __forceinline__ void zero() { q = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void widen(float (&v)[8]) const {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load_n(const float* p, int cnt) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (i < cnt) ? p[i] : 0.f;
    a = make_float4(v[0], v[1], v[2], v[3]);
    b = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void widen(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// ---------------------------------------------------------------------------
// summaries.  REWEIGHT:  t_j = anchor.k_j / sqrt(d);  w = softmax_B(t);
//   ksum = sum w_j k_j;  vsum = sum w_j v_j;
//   bias = max t + log sum exp(t - max t) - log n_B - anchor.ksum / sqrt(d)
// MEAN: w_j = 1 / n_B, bias = 0.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void summarize_kernel(const T* __restrict__ kp,
                                                        const T* __restrict__ vpt,
                                                        const float* __restrict__ anchor,
                                                        float* __restrict__ ksum,
                                                        float* __restrict__ vsum,
                                                        float* __restrict__ bias, int N, int BK,
                                                        int nb, int nbt, int mean_mode, float rsd) {
  __shared__ float s_anchor[D];
  __shared__ float s_w[128];
  __shared__ float s_t[128];
  __shared__ float s_part[16][D];
  __shared__ float s_red[2];
  const int h = blockIdx.x / nb, B = blockIdx.x % nb;
  const int tid = threadIdx.x;
  const int n_real = min(BK, N - B * BK);
  const long Np = (long)nbt * BK;   // k_p / v_pt may hold nbt - nb context blocks after these
  const T* kblk = kp + ((long)h * Np + (long)B * BK) * D;
  const T* vblk = vpt + ((long)h * nbt + B) * (long)D * BK;
  constexpr int CPR = D / 8;           // chunks per row
  constexpr int RPP = 256 / CPR;       // rows per pass
  constexpr int NR = 128 / RPP;        // row passes of a block of up to 128 tokens
  // the block's key chunks (rows rg + RPP i) and transposed value chunks
  // (rows c + 16 i, tokens jc .. jc + 7), all loaded up front: a workgroup
  // then has its whole block in flight, and the keys serve both key passes
  const int rg = tid / CPR, ck = (tid % CPR) * 8;
  const int rv = tid / 16, jc = (tid % 16) * 8;
  Raw8<T> kraw[NR], vraw[D / 16];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int j = rg + RPP * i;
    if (j < n_real) kraw[i].load(kblk + (long)j * D + ck);
    else kraw[i].zero();
  }
  // a transposed row holds BK tokens: with BK % 8 == 0 every 8-token chunk
  // is 16-byte aligned and inside the row; otherwise the chunk is read
  // element by element up to the block's last real token
  const bool vec_rows = (BK & 7) == 0;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const T* src = vblk + (long)(rv + 16 * i) * BK + jc;
    if (jc >= n_real) vraw[i].zero();
    else if (vec_rows) vraw[i].load(src);
    else vraw[i].load_n(src, min(8, n_real - jc));
  }
  auto widen8 = [](const Raw8<T>& q, float (&v)[8]) { q.widen(v); };

  if (!mean_mode) {
    for (int c = tid; c < D; c += 256) s_anchor[c] = anchor[(long)h * D + c];
    __syncthreads();
    // t_j: CPR lanes per row, reduced with shuffles (CPR is 8 or 16)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (RPP * i < n_real) {   // uniform
        const int j = rg + RPP * i;
        float acc = 0.f;
        if (j < n_real) {
          float v[8];
          widen8(kraw[i], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(v[e], s_anchor[ck + e], acc);
        }
        acc = group_sum<CPR>(acc);
        if (j < n_real && (tid % CPR) == 0) s_w[j] = acc * rsd;
      }
    }
    __syncthreads();
    if (tid < 64) {
      float m = -INFINITY;
      for (int j = tid; j < n_real; j += 64) m = fmaxf(m, s_w[j]);
      m = wave_max(m);
      float z = 0.f;
      for (int j = tid; j < n_real; j += 64) z += expf(s_w[j] - m);
      z = wave_sum(z);
      if (tid == 0) { s_red[0] = m; s_red[1] = z; }
    }
    __syncthreads();
    const float m = s_red[0], z = s_red[1];
    for (int j = tid; j < n_real; j += 256) {
      s_t[j] = s_w[j];
      s_w[j] = expf(s_w[j] - m) / z;
    }
    __syncthreads();
  } else {
    for (int j = tid; j < n_real; j += 256) s_w[j] = 1.f / (float)n_real;
    __syncthreads();
  }

  // ksum: row-chunk partials over RPP row groups, then a fixed-order reduce
  {
    const int c = ck;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = rg + RPP * i;
      if (j < n_real) {
        float v[8];
        widen8(kraw[i], v);
        const float w = s_w[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[e], acc[e]);
      }
    }
    if (rg < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_part[rg][c + e] = acc[e];
    }
    // RPP is 16 (D=128) or 32 (D=64): fold rows 16..31 in a second step
    __syncthreads();
    if (RPP > 16 && rg >= 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_part[rg - 16][c + e] += acc[e];
    }
    __syncthreads();
  }
  float kval = 0.f;
  if (tid < D) {
    for (int r = 0; r < 16; ++r) kval += s_part[r][tid];
    ksum[((long)h * nb + B) * D + tid] = kval;
  }
  // vsum from the transposed block: row c of vpt holds the block's values of
  // column c.  16 lanes per row, 8 consecutive tokens each (one 16-byte
  // load), then a fixed shuffle tree over the 16 lanes; tokens past n_real
  // are skipped.
  {
    float wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = (jc + e < n_real) ? s_w[jc + e] : 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int c = rv + 16 * i;
      float acc = 0.f;
      if (jc < n_real) {
        float v[8];
        widen8(vraw[i], v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (jc + e < n_real) acc = fmaf(wv[e], v[e], acc);
      }
      acc = group_sum<16>(acc);
      if ((tid & 15) == 0) vsum[((long)h * nb + B) * D + c] = acc;
    }
  }
  if (mean_mode) {
    if (tid == 0) bias[(long)h * nb + B] = 0.f;
    return;
  }
  // bias = m + log z - log n_B - anchor . ksum / sqrt(d).  Since
  // anchor . ksum / sqrt(d) = sum_j w_j t_j, this equals
  // log z - log n_B + sum_j w_j (m - t_j), which is exactly 0 for a
  // one-token block.  s_t holds the logits t_j (saved before w overwrote them).
  if (tid < 64) {
    const float m = s_red[0], z = s_red[1];
    float a = 0.f;
    for (int j = tid; j < n_real; j += 64) a = fmaf(s_w[j], m - s_t[j], a);
    a = wave_sum(a);
    if (tid == 0) bias[(long)h * nb + B] = logf(z) - logf((float)n_real) + a;
  }
}

template <typename T, int D>
static int summarize_t(int H, int N, int nbc, int BK, const void* kp, const void* vpt,
                       const float* anchor, float* ksum, float* vsum, float* bias, int mean_mode,
                       hipStream_t st) {
  const int nb = cdiv(N, BK);
  hipLaunchKernelGGL((summarize_kernel<T, D>), dim3(H * nb), dim3(256), 0, st, (const T*)kp,
                     (const T*)vpt, anchor, ksum, vsum, bias, N, BK, nb, nb + nbc, mean_mode,
                     1.f / sqrtf((float)D));
  return spark_check_launch("summarize");
}

// Summaries of the ceil(N / BK) blocks of N (video) tokens; k_p / v_pt carry
// nbc further (context) blocks per head, which are not summarised.
int summarize_launch(int H, int N, int nbc, int D, int BK, int dtype, const void* kp,
                     const void* vpt, const float* anchor, float* ksum, float* vsum, float* bias,
                     int mean_mode, hipStream_t st) {
  if (dtype == SPARK_F32)
    return D == 128 ? summarize_t<float, 128>(H, N, nbc, BK, kp, vpt, anchor, ksum, vsum, bias, mean_mode, st)
                    : summarize_t<float, 64>(H, N, nbc, BK, kp, vpt, anchor, ksum, vsum, bias, mean_mode, st);
  return D == 128 ? summarize_t<uint16_t, 128>(H, N, nbc, BK, kp, vpt, anchor, ksum, vsum, bias, mean_mode, st)
                  : summarize_t<uint16_t, 64>(H, N, nbc, BK, kp, vpt, anchor, ksum, vsum, bias, mean_mode, st);
}

// anchor[h] = mean of query rows [0, n_anchor) (column sums in row order)
// Anchor without the moments pass (IDENTITY / GIVEN layouts): per head, the
// mean of the first n_anchor query rows.  Pass 1: chunk c of every head sums
// its rows (16 row lanes x 8-column chunks per workgroup, batched loads),
// pass 2 adds the chunk sums in chunk order (deterministic).
constexpr int ANC_T = 256;

template <typename T, int D>
__global__ __launch_bounds__(ANC_T) void anchor_partial(const T* __restrict__ q, float* __restrict__ part,
                                                        int N, int n_anchor, int rows_per_chunk,
                                                        long part_head_stride) {
  constexpr int VE = 16 / (int)sizeof(T), CPR = D / VE, RL = ANC_T / CPR;
  __shared__ float sp[RL][D];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rl = tid / CPR, cc = (tid % CPR) * VE;
  const long r0 = (long)c * rows_per_chunk;
  const long r1 = min((long)n_anchor, r0 + rows_per_chunk);
  const T* qh = q + (long)h * N * D;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  for (long r = r0 + rl; r < r1; r += 4 * RL) {
    float v[4][VE];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long rr = r + (long)u * RL;
      if (rr < r1) {
        Chunk<T>::load(qh + rr * D + cc, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) v[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += v[u][e];
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) sp[rl][cc + e] = acc[e];
  __syncthreads();
  for (int col = tid; col < D; col += ANC_T) {
    float s = 0.f;
    for (int l = 0; l < RL; ++l) s += sp[l][col];
    part[(long)h * part_head_stride + (long)c * D + col] = s;
  }
}

__global__ void anchor_reduce(const float* __restrict__ part, float* __restrict__ anchor, int D,
                              int nchunk, long part_head_stride, int n_anchor) {
  const int h = blockIdx.x;
  for (int col = threadIdx.x; col < D; col += blockDim.x) {
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += part[(long)h * part_head_stride + (long)c * D + col];
    anchor[(long)h * D + col] = s / (float)n_anchor;
  }
}

template <typename T, int D>
static void anchor_t(int H, int N, const void* q, float* anchor, int n_anchor, float* scratch,
                     int nb, hipStream_t st) {
  // up to nb chunks, so the partials fit in a [H, nb, D] fp32 scratch
  const int nchunk = std::max(1, std::min(nb, cdiv(n_anchor, 512)));
  const int rpc = cdiv(n_anchor, nchunk);
  const long stride = (long)nb * D;
  hipLaunchKernelGGL((anchor_partial<T, D>), dim3(nchunk, H), dim3(ANC_T), 0, st, (const T*)q, scratch, N,
                     n_anchor, rpc, stride);
  hipLaunchKernelGGL(anchor_reduce, dim3(H), dim3(D), 0, st, scratch, anchor, D, nchunk, stride, n_anchor);
}

// scratch: [H, scratch_nb, D] fp32 (e.g. the qbar output, written later)
int anchor_launch(int H, int N, int D, int dtype, const void* q, float* anchor, int n_anchor,
                  float* scratch, int scratch_nb, hipStream_t st) {
  const int nb = scratch_nb;
  if (dtype == SPARK_F32) {
    if (D == 128) anchor_t<float, 128>(H, N, q, anchor, n_anchor, scratch, nb, st);
    else anchor_t<float, 64>(H, N, q, anchor, n_anchor, scratch, nb, st);
  } else {
    if (D == 128) anchor_t<uint16_t, 128>(H, N, q, anchor, n_anchor, scratch, nb, st);
    else anchor_t<uint16_t, 64>(H, N, q, anchor, n_anchor, scratch, nb, st);
  }
  return spark_check_launch("anchor");
}

}  // namespace spark
