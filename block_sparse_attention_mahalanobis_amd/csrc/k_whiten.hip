// Spark-Reblock's metric ("Spark-H3" blog, 01 / Method: Spark-Reblock, the
// d_Q equation): second moments M = E[x x^T] of each side, their symmetric
// square roots, and the whitened, unit-normalised rows x^ = W x / ||W x||,
// whose dot products are the Mahalanobis cosines 1 - d_Q.
//
//  * moments: bf16 rows go through v_mfma_f32_32x32x16_bf16 (X^T X with the
//    chunk staged transposed in LDS), fp32 rows through VALU; per-chunk
//    partials are summed in a fixed order (deterministic).  The anchor query
//    (mean of the video queries, 02 / Method: Spark-Reweight) is fused into
//    the query pass.
//  * msqrt: coupled Newton-Schulz iteration in fp32, one workgroup per matrix.
//  * whiten: X W on MFMA (bf16, W rounded to bf16) or VALU (fp32), row norms
//    in the epilogue.
#include "common.hpp"

namespace spark {

constexpr int MOM_TOK = 128;     // rows staged per LDS round

// Rows per moment partial: a function of N alone, so a head's moments (and
// everything computed from them) do not depend on how many heads are
// processed together.  At most 25 chunks per matrix: the 768p layer's 80
// matrices give 2000 workgroups, four full waves of the 512 that the chip
// holds at once (two per CU), so no wave runs a small remainder alone; a
// multiple of MOM_TOK, at least 256 rows.
struct MomPlan {
  int nchunk, rpc;
};
static MomPlan mom_plan(int N) {
  int rpc = std::max(256, cdiv(N, 25));
  rpc = cdiv(rpc, MOM_TOK) * MOM_TOK;
  return {cdiv(N, rpc), rpc};
}

// partial[t][c][D*D] (+ colsum partial[t][c][D] for anchors); trees t < H
// are the query side (xq), the others the key side (xk).  The next round's
// rows are loaded into registers while the current round's MFMAs run.
template <int D>
__global__ __launch_bounds__(256) void moments_mfma(const uint16_t* __restrict__ xq,
                                                    const uint16_t* __restrict__ xk,
                                                    float* __restrict__ part,
                                                    float* __restrict__ cpart, int H, int N,
                                                    int n_anchor, int nchunk, int rpc) {
  // X^T in LDS, one row per column of X.  d = 128: rows of MOM_TOK tokens
  // as 16 chunks of 8, chunk slot XOR-swizzled by (row + row / 8) mod 16, so
  // the transposed stores (16 rows 8 apart, 4 chunk groups per wave) and
  // the MFMA operand reads (32 consecutive rows, one chunk each) both spread
  // over all banks.  d = 64: rows padded by 8 tokens.
  constexpr bool SWZ = (D == 128);
  constexpr int RS = SWZ ? MOM_TOK : MOM_TOK + 8;   // LDS row stride (bf16) of X^T
  __shared__ __attribute__((aligned(16))) uint16_t sXT[D * RS];
  auto xt_sw = [](int r) { return SWZ ? ((r + (r >> 3)) & 15) : 0; };
  const int t = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const long r0 = (long)chunk * rpc;
  const long r1 = min((long)N, r0 + rpc);
  const uint16_t* xt = (t < H) ? xq + (long)t * N * D : xk + (long)(t - H) * N * D;
  constexpr int MT = D / 32;                 // output tiles per side
  constexpr int TPW = MT * MT / 4;           // output tiles per wave (4 or 1)
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  const bool want_cs = cpart != nullptr && t < H;
  float cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // column sums of rows < n_anchor

  // staging: thread -> (RPG-row group, 8-col chunk); the next round's rows
  // (32 KB per workgroup for d = 128) are in flight while this round runs
  constexpr int CPR = D / 8;                 // 16 or 8
  constexpr int RG = 256 / CPR;              // row groups per round: 16 or 32
  constexpr int RPG = MOM_TOK / RG;          // rows per group: 8 or 4
  static_assert(RPG == 8 || RPG == 4, "staging layout");
  const int g = tid / CPR, cc = (tid % CPR) * 8;
  constexpr bool stager = true;

  uint4 pf[RPG];
  auto fetch = [&](long rb) {
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      const long row = rb + g * RPG + rr;
      pf[rr] = (row < r1) ? *reinterpret_cast<const uint4*>(xt + row * D + cc) : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(r0);
  for (long rb = r0; rb < r1; rb += MOM_TOK) {
    __syncthreads();  // the previous round's MFMAs are done with sXT
    if (stager) {
      uint16_t vals[RPG][8];
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr) {
        const long row = rb + g * RPG + rr;
        const uint32_t w[4] = {pf[rr].x, pf[rr].y, pf[rr].z, pf[rr].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vals[rr][2 * e] = (uint16_t)(w[e] & 0xffff);
          vals[rr][2 * e + 1] = (uint16_t)(w[e] >> 16);
        }
        if (want_cs && row < r1 && row < n_anchor) {
#pragma unroll
          for (int e = 0; e < 8; ++e) cs[e] += bf2f(vals[rr][e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (RPG == 8) {
          uint4 p;
          p.x = (uint32_t)vals[0][e] | ((uint32_t)vals[1][e] << 16);
          p.y = (uint32_t)vals[2][e] | ((uint32_t)vals[3][e] << 16);
          p.z = (uint32_t)vals[4][e] | ((uint32_t)vals[5][e] << 16);
          p.w = (uint32_t)vals[6][e] | ((uint32_t)vals[7][e] << 16);
          *reinterpret_cast<uint4*>(sXT + (cc + e) * RS + ((g ^ xt_sw(cc + e)) * RPG)) = p;
        } else {
          uint2 p;
          p.x = (uint32_t)vals[0][e] | ((uint32_t)vals[1][e] << 16);
          p.y = (uint32_t)vals[2][e] | ((uint32_t)vals[3][e] << 16);
          *reinterpret_cast<uint2*>(sXT + (cc + e) * RS + g * RPG) = p;
        }
      }
    }
    __syncthreads();
    if (rb + MOM_TOK < r1) fetch(rb + MOM_TOK);
#pragma unroll
    for (int ks = 0; ks < MOM_TOK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tile = wave * TPW + i;
        const int mt = tile / MT, nt = tile % MT;
        if (tile >= MT * MT) continue;
        const int ra = 32 * mt + l32, rb2 = 32 * nt + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sXT + ra * RS + (((2 * ks + hf) ^ xt_sw(ra)) * 8));
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(sXT + rb2 * RS + (((2 * ks + hf) ^ xt_sw(rb2)) * 8));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      }
    }
  }
  float* pout = part + ((long)t * nchunk + chunk) * D * D;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wave * TPW + i;
    if (tile >= MT * MT) continue;
    const int mt = tile / MT, nt = tile % MT;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * mt + 8 * (v / 4) + 4 * hf + (v % 4);
      const int col = 32 * nt + l32;
      pout[row * D + col] = acc[i][v];
    }
  }
  if (want_cs) {
    // reduce the RG row groups' column sums through LDS (reuse sXT as floats)
    __syncthreads();
    float* sf = reinterpret_cast<float*>(sXT);
    if (stager)
#pragma unroll
      for (int e = 0; e < 8; ++e) sf[g * D + cc + e] = cs[e];
    __syncthreads();
    const int ng = RG;
    for (int c = tid; c < D; c += 256) {
      float s = 0.f;
      for (int gg = 0; gg < ng; ++gg) s += sf[gg * D + c];
      cpart[((long)t * nchunk + chunk) * D + c] = s;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void moments_f32(const float* __restrict__ xq,
                                                   const float* __restrict__ xk,
                                                   float* __restrict__ part,
                                                   float* __restrict__ cpart, int H, int N,
                                                   int n_anchor, int nchunk, int rpc) {
  constexpr int RPT = D * D / 256;  // outputs per thread: 64 (D=128) or 16 (D=64)
  constexpr int SUB = (D == 128) ? 8 : 4;  // output sub-block side
  __shared__ float sX[MOM_TOK][D];
  const int t = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const long r0 = (long)chunk * rpc;
  const long r1 = min((long)N, r0 + rpc);
  const float* xt = (t < H) ? xq + (long)t * N * D : xk + (long)(t - H) * N * D;
  const int bi = (tid / (D / SUB)) * SUB, bj = (tid % (D / SUB)) * SUB;
  float acc[SUB][SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j) acc[i][j] = 0.f;
  const bool want_cs = cpart != nullptr && t < H;
  float cs = 0.f;
  static_assert(RPT == SUB * SUB, "tiling");
  for (long rb = r0; rb < r1; rb += MOM_TOK) {
    __syncthreads();
    for (int e = tid; e < MOM_TOK * D; e += 256) {
      const long row = rb + e / D;
      sX[e / D][e % D] = (row < r1) ? xt[row * D + e % D] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < MOM_TOK; ++r) {
      float a[SUB], b[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) { a[i] = sX[r][bi + i]; b[i] = sX[r][bj + i]; }
#pragma unroll
      for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    if (want_cs && tid < D)
      for (int r = 0; r < MOM_TOK; ++r)
        if (rb + r < r1 && rb + r < n_anchor) cs += sX[r][tid];
  }
  float* pout = part + ((long)t * nchunk + chunk) * D * D;
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j) pout[(bi + i) * D + bj + j] = acc[i][j];
  if (want_cs && tid < D) cpart[((long)t * nchunk + chunk) * D + tid] = cs;
}

// M[t] = (sum over chunks in order) / N; anchor[t] = colsum / n_anchor
__global__ void moments_reduce(const float* __restrict__ part, const float* __restrict__ cpart,
                               float* __restrict__ MQ, float* __restrict__ MK,
                               float* __restrict__ anchor, int H, int D, int N, int n_anchor,
                               int nchunk) {
  const int t = blockIdx.y;  // 0..2H-1: q trees then k trees
  const long DD = (long)D * D;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < DD; e += (long)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += part[((long)t * nchunk + c) * DD + e];
    float* dst = (t < H) ? (MQ + (long)t * DD) : (MK + (long)(t - H) * DD);
    dst[e] = s / (float)N;
  }
  if (anchor != nullptr && t < H && blockIdx.x == 0) {
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
      float s = 0.f;
      for (int ch = 0; ch < nchunk; ++ch) s += cpart[((long)t * nchunk + ch) * D + c];
      anchor[(long)t * D + c] = s / (float)n_anchor;
    }
  }
}

size_t moments_ws_bytes(int H, int N, int D) {
  const int nchunk = mom_plan(N).nchunk;
  return (size_t)2 * H * nchunk * D * D * 4 + (size_t)2 * H * nchunk * D * 4 + 512;
}

// One launch over both sides: trees 0..H-1 are q, H..2H-1 are k (k, MK may
// be NULL: then only the query side, M_Q and the anchor).
int moments_launch(int H, int N, int D, int dtype, const void* q, const void* k, float* MQ,
                   float* MK, float* anchor, int n_anchor, void* ws, hipStream_t st) {
  const MomPlan mp = mom_plan(N);
  const int nchunk = mp.nchunk;
  float* part = (float*)ws;
  float* cpart = part + (size_t)2 * H * nchunk * D * D;
  const int trees = (k != nullptr) ? 2 * H : H;  // k == NULL: the query side only
  dim3 grid(nchunk, trees);
  if (dtype == SPARK_BF16) {
    if (D == 128)
      hipLaunchKernelGGL(moments_mfma<128>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k, part, cpart, H, N, n_anchor, nchunk, mp.rpc);
    else
      hipLaunchKernelGGL(moments_mfma<64>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k, part, cpart, H, N, n_anchor, nchunk, mp.rpc);
  } else {
    if (D == 128)
      hipLaunchKernelGGL(moments_f32<128>, grid, dim3(256), 0, st, (const float*)q, (const float*)k, part, cpart, H, N, n_anchor, nchunk, mp.rpc);
    else
      hipLaunchKernelGGL(moments_f32<64>, grid, dim3(256), 0, st, (const float*)q, (const float*)k, part, cpart, H, N, n_anchor, nchunk, mp.rpc);
  }
  int rc = spark_check_launch("moments");
  if (rc) return rc;
  hipLaunchKernelGGL(moments_reduce, dim3(16, trees), dim3(256), 0, st, part, cpart, MQ, MK,
                     anchor, H, D, N, n_anchor, nchunk);
  return spark_check_launch("moments_reduce");
}

// ---------------------------------------------------------------------------
// msqrt: Y0 = M / s + delta I with s = ||M||_F, Z0 = I;  T = (3I - Z Y) / 2;
// Y <- Y T;  Z <- T Z.  Y -> (M/s + delta I)^{1/2}, so W = sqrt(s) Y.  The
// ridge delta = 1e-6 bounds the smallest eigenvalue the iteration has to
// reach (and keeps rank-deficient moments from amplifying round-off in their
// null space); it moves W by at most sqrt(delta * s) in directions of zero
// energy.  Y, Z and T live in LDS (two D x D slots: see the loop).  Stops
// when max|ZY - I| < 3e-5, after at most 40 iterations.
// ---------------------------------------------------------------------------
constexpr int MSQ_T = 512;
template <int D>
__global__ __launch_bounds__(MSQ_T) void msqrt_kernel(const float* __restrict__ M,
                                                    float* __restrict__ W) {
  // each thread owns an SI x SJ block of every product: 8 x 4 (d = 128) or
  // 4 x 2 (d = 64) with MSQ_T threads, two waves per SIMD
  constexpr int SI = (D == 128) ? 8 : 4, SJ = SI / 2;
  constexpr int NW = MSQ_T / 64;
  __shared__ float sY[D * D];
  __shared__ float sZ[D * D];
  __shared__ float s_red[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long off = (long)blockIdx.x * D * D;
  const float* m = M + off;
  const int bi = (tid / (D / SJ)) * SI, bj = (tid % (D / SJ)) * SJ;

  // Frobenius norm (symmetrised input)
  float ss = 0.f;
  for (int e = tid; e < D * D; e += MSQ_T) {
    const int r = e / D, c = e % D;
    const float v = 0.5f * (m[r * D + c] + m[c * D + r]);
    sY[e] = v;
    ss += v * v;
  }
  ss = wave_sum(ss);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  float ssum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ssum += s_red[w];
  const float fro = sqrtf(ssum);
  if (!(fro > 0.f) || !isfinite(fro)) {
    for (int e = tid; e < D * D; e += MSQ_T) W[off + e] = (fro == 0.f) ? 0.f : NAN;
    return;
  }
  const float inv = 1.f / fro;
  constexpr float kRidge = 1e-6f;
  for (int e = tid; e < D * D; e += MSQ_T) {
    const bool diag = (e / D == e % D);
    sY[e] = sY[e] * inv + (diag ? kRidge : 0.f);
    sZ[e] = diag ? 1.f : 0.f;
  }
  __syncthreads();

  // Y in sA, Z in sB at the start of every iteration; T never leaves the
  // workgroup: each thread keeps its own block of Z in registers while T
  // takes Z's place for Y T, then Z takes Y's place for T Z
  float* sA = sY;
  float* sB = sZ;
  for (int it = 0; it < 40; ++it) {
    // P = Z Y (this thread's block)
    float acc[SI][SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) acc[i][j] = 0.f;
#pragma unroll 4
    for (int kx = 0; kx < D; ++kx) {
      float a[SI], b[SJ];
#pragma unroll
      for (int i = 0; i < SI; ++i) a[i] = sB[(bi + i) * D + kx];
#pragma unroll
      for (int j = 0; j < SJ; ++j) b[j] = sA[kx * D + bj + j];
#pragma unroll
      for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    float dev = 0.f;
    float zk[SI][SJ];   // this thread's block of Z
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        const float id = (bi + i == bj + j) ? 1.f : 0.f;
        dev = fmaxf(dev, fabsf(acc[i][j] - id));
        acc[i][j] = 0.5f * (3.f * id - acc[i][j]);   // T
        zk[i][j] = sB[(bi + i) * D + bj + j];
      }
    dev = wave_max(dev);
    if (lane == 0) s_red[wave] = dev;
    __syncthreads();  // s_red ready; every read of Z done
    float gdev = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) gdev = fmaxf(gdev, s_red[w]);
    if (gdev < 3e-5f) break;
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) sB[(bi + i) * D + bj + j] = acc[i][j];
    __syncthreads();  // T in sB
    // Ynew = Y T
    float ay[SI][SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) ay[i][j] = 0.f;
#pragma unroll 4
    for (int kx = 0; kx < D; ++kx) {
      float ya[SI], tb[SJ];
#pragma unroll
      for (int i = 0; i < SI; ++i) ya[i] = sA[(bi + i) * D + kx];
#pragma unroll
      for (int j = 0; j < SJ; ++j) tb[j] = sB[kx * D + bj + j];
#pragma unroll
      for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j) ay[i][j] = fmaf(ya[i], tb[j], ay[i][j]);
    }
    __syncthreads();  // every read of Y done
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) sA[(bi + i) * D + bj + j] = zk[i][j];
    __syncthreads();  // Z in sA
    // Znew = T Z
    float az[SI][SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) az[i][j] = 0.f;
#pragma unroll 4
    for (int kx = 0; kx < D; ++kx) {
      float ta[SI], zb[SJ];
#pragma unroll
      for (int i = 0; i < SI; ++i) ta[i] = sB[(bi + i) * D + kx];
#pragma unroll
      for (int j = 0; j < SJ; ++j) zb[j] = sA[kx * D + bj + j];
#pragma unroll
      for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j) az[i][j] = fmaf(ta[i], zb[j], az[i][j]);
    }
    __syncthreads();  // every read of T and Z done
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        sA[(bi + i) * D + bj + j] = ay[i][j];
        sB[(bi + i) * D + bj + j] = az[i][j];
      }
    __syncthreads();
  }
  const float sc = sqrtf(fro);
  for (int e = tid; e < D * D; e += MSQ_T) {
    const int r = e / D, c = e % D;
    W[off + e] = 0.5f * (sA[r * D + c] + sA[c * D + r]) * sc;
  }
}

int msqrt_launch(int count, int D, const float* M, float* W, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL(msqrt_kernel<128>, dim3(count), dim3(MSQ_T), 0, st, M, W);
  else
    hipLaunchKernelGGL(msqrt_kernel<64>, dim3(count), dim3(MSQ_T), 0, st, M, W);
  return spark_check_launch("msqrt");
}

// ---------------------------------------------------------------------------
// whiten: xhat = normalize(W x) row by row.  bf16: x^T-side MFMA with W (bf16)
// as the A operand: O^T[c][i] = sum_k W[c][k] x_i[k]; lane l32 owns row i.
// ---------------------------------------------------------------------------
constexpr int WH_ROWS = 4096;  // rows per workgroup: 32 rounds of 4 waves x 32 (the W setup is paid per workgroup)

// Each wave whitens 32 consecutive rows per round.  The rows (8 KB for
// d = 128, contiguous in HBM) come in with 16-byte lane loads, four rows per
// instruction, are staged in the wave's own LDS slice, and feed the MFMA B
// operand from there; the bf16 results go back through the same slice and
// out as coalesced 16-byte stores.  The next round's rows are loaded into
// registers while the current round runs.  A wave's LDS accesses are ordered
// by wave_lds_sync(), so past the W load there is no workgroup barrier.
template <int D>
__global__ __launch_bounds__(256, 2) void whiten_mfma(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ W,
                                                   uint16_t* __restrict__ xh, int N, int xrows,
                                                   float* __restrict__ cpart, int tree_off, int nb) {
  constexpr int RS = D + 8;            // LDS row stride (bf16), 16-byte pad
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int CPL = 32 * CPR / 64;   // chunks per lane per round (d = 128: 8)
  __shared__ __attribute__((aligned(16))) uint16_t sW[D * RS];
  __shared__ __attribute__((aligned(16))) uint16_t sX[4][32 * RS];
  __shared__ float s_cp[2][4][D];   // by round parity
  const int t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const float* w = W + (long)t * D * D;
  for (int e = tid; e < D * D; e += 256) sW[(e / D) * RS + e % D] = f2bf(w[e]);
  __syncthreads();
  uint16_t* sx = sX[wave];
  const uint16_t* xt = x + (long)t * xrows * D;
  uint16_t* ht = xh + (long)t * N * D;
  const long wbase = (long)blockIdx.x * WH_ROWS + wave * 32;   // this wave's first row, round 0

  uint4 pf[CPL];
  auto load = [&](long base) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane, rr = c / CPR, cc = c % CPR;
      pf[i] = (base + rr < N) ? *reinterpret_cast<const uint4*>(xt + (base + rr) * D + cc * 8)
                              : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (wbase < N) load(wbase);
  for (int r0 = 0; r0 < WH_ROWS; r0 += 128) {
    const long base = wbase + r0;
    // uniform across the workgroup (the partial sums below take barriers): a
    // wave whose rows all lie past N runs the round on ignored data, with
    // every load, store and sum guarded by row < N
    if ((long)blockIdx.x * WH_ROWS + r0 >= N) break;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane, rr = c / CPR, cc = c % CPR;
      *reinterpret_cast<uint4*>(sx + rr * RS + cc * 8) = pf[i];
    }
    if (r0 + 128 < WH_ROWS && base + 128 < N) load(base + 128);
    wave_lds_sync();
    bf16x8 xb[D / 16];
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2)
      xb[s2] = *reinterpret_cast<const bf16x8*>(sx + l32 * RS + 16 * s2 + 8 * hf);
    f32x16 acc[D / 32];
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ct][v] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < D / 16; ++s2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sW + (32 * ct + l32) * RS + 16 * s2 + 8 * hf);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[s2], acc[ct], 0, 0, 0);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) ss = fmaf(acc[ct][v], acc[ct][v], ss);
    ss = group_sum<64, 32>(ss);
    const float inv = (ss > 0.f) ? 1.f / sqrtf(ss) : 0.f;
    wave_lds_sync();   // every lane has read its B operand rows
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 p;
        p.x = pack_bf2(acc[ct][4 * a] * inv, acc[ct][4 * a + 1] * inv);
        p.y = pack_bf2(acc[ct][4 * a + 2] * inv, acc[ct][4 * a + 3] * inv);
        *reinterpret_cast<uint2*>(sx + l32 * RS + 32 * ct + 8 * a + 4 * hf) = p;
      }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane, rr = c / CPR, cc = c % CPR;
      if (base + rr < N)
        *reinterpret_cast<uint4*>(ht + (base + rr) * D + cc * 8) = *reinterpret_cast<const uint4*>(sx + rr * RS + cc * 8);
    }
    if (cpart) {
      // The round's 128 rows are one block of the split's first level (block
      // 128, identity order): its partial centroid sum in the split's own
      // centroid-pass order (wave w: lane (rl, chunk c) adds its slice rows
      // 4 it + rl, absent rows as +0; then the lanes of a chunk; then the
      // waves in order), so the sums are bit-identical to that pass's.
      const long row0 = (long)blockIdx.x * WH_ROWS + r0;
      const int rl = lane / CPR, c = (lane % CPR) * 8, par = (r0 >> 7) & 1;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int j = 4 * it + rl;   // this wave's slice row
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (base + j < N) raw = *reinterpret_cast<const uint4*>(sx + j * RS + c);
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          acc[2 * q2] += __uint_as_float(wv[q2] << 16);
          acc[2 * q2 + 1] += __uint_as_float(wv[q2] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = group_sum<64, CPR>(acc[e]);
      if (lane < CPR)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_cp[par][wave][c + e] = acc[e];
      __syncthreads();   // the four waves' sums (the other parity is free again)
      for (int cc2 = tid; cc2 < D; cc2 += 256) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) sum += s_cp[par][w2][cc2];
        cpart[((long)(tree_off + t) * nb + row0 / 128) * D + cc2] = sum;
      }
    }
    wave_lds_sync();   // the slice is free for the next round
  }
}

template <int D>
__global__ __launch_bounds__(256) void whiten_f32(const float* __restrict__ x,
                                                  const float* __restrict__ W,
                                                  float* __restrict__ xh, int N, int xrows) {
  __shared__ float sW[D * (D + 1)];
  const int t = blockIdx.y, tid = threadIdx.x;
  const float* w = W + (long)t * D * D;
  for (int e = tid; e < D * D; e += 256) sW[(e / D) * (D + 1) + e % D] = w[e];
  __syncthreads();
  // one thread per row
  const long row = (long)blockIdx.x * 256 + tid;
  if (row >= N) return;
  const float* xr = x + ((long)t * xrows + row) * D;
  float xv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) xv[c] = xr[c];
  float ss = 0.f;
  float* dst = xh + ((long)t * N + row) * D;
  for (int c = 0; c < D; ++c) {
    float acc = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < D; ++k2) acc = fmaf(sW[c * (D + 1) + k2], xv[k2], acc);
    dst[c] = acc;
    ss = fmaf(acc, acc, ss);
  }
  const float inv = (ss > 0.f) ? 1.f / sqrtf(ss) : 0.f;
  for (int c = 0; c < D; ++c) dst[c] *= inv;
}

// Rows [0, N) of each of the `count` input matrices, whose head stride is
// xrows >= N rows (xrows > N: the rows past N are context tokens, not
// whitened); xh is [count, N, D].
// cpart (bf16, d = 128 only; else NULL): also store the split's first-level
// partial centroid sums of 128-row blocks, for trees tree_off .. tree_off +
// count - 1 of a [trees][ceil(N / 128)][D] array.
int whiten_launch(int count, int N, int xrows, int D, int dtype, const void* x, const float* W,
                  void* xh, hipStream_t st, float* cpart, int tree_off) {
  if (dtype == SPARK_BF16) {
    dim3 grid(cdiv(N, WH_ROWS), count);
    const int nb = cdiv(N, 128);
    if (D == 128)
      hipLaunchKernelGGL(whiten_mfma<128>, grid, dim3(256), 0, st, (const uint16_t*)x, W, (uint16_t*)xh, N, xrows,
                         cpart, tree_off, nb);
    else
      hipLaunchKernelGGL(whiten_mfma<64>, grid, dim3(256), 0, st, (const uint16_t*)x, W, (uint16_t*)xh, N, xrows,
                         (float*)nullptr, 0, nb);
  } else {
    dim3 grid(cdiv(N, 256), count);
    if (D == 128)
      hipLaunchKernelGGL(whiten_f32<128>, grid, dim3(256), 0, st, (const float*)x, W, (float*)xh, N, xrows);
    else
      hipLaunchKernelGGL(whiten_f32<64>, grid, dim3(256), 0, st, (const float*)x, W, (float*)xh, N, xrows);
  }
  return spark_check_launch("whiten");
}

}  // namespace spark
