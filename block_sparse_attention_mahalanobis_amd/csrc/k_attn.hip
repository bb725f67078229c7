// Fused exact + compressed block-sparse attention with the inverse-permutation
// scatter ("Spark-H3" blog, 01 / Method: Spark-Reblock, the BSA(Q_A) equation
// and the concatenated effective keys/values K~_A, V~_A: one row-wise softmax
// over the exact rows of the selected blocks and, for every other block, its
// summary repeated |B| times; the summaries and log-mass bias come from
// 02 / Method: Spark-Reweight).
//
// Two kernels:
//  * attn_mfma: bf16, block size 32/64/128, d 64/128.  One workgroup per
//    (head, query block), one wave per 32 query rows.  S^T = K Q^T and
//    O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, an
//    online softmax in the log2 domain, K / V^T tiles staged through LDS with
//    a register prefetch of the next tile.  The compressed branch runs the
//    same loop over tiles of bf16 summaries, with the per-block bias
//    (+ log |B|) added to the logits and the selected blocks masked to -inf.
//  * attn_generic: fp32 or bf16, any block size 1..128; one thread per query
//    row, fp32 VALU arithmetic.  Small and slow; it exists for the fp32
//    workloads and odd block sizes.
#include "common.hpp"

namespace spark {

// ---------------------------------------------------------------------------
// Compressed-branch operands in the layout the MFMA kernel streams:
//   ks16  [H, nbp, D]          bf16 summary keys, rows >= n_b zero
//   vs16t [H, nbp/BK, D, BK]   bf16 summary values, tile-transposed
//   bias2 [H, nbp]             (bias + log n_B) * log2(e), -inf for padding
// ---------------------------------------------------------------------------
__global__ void attn_prep_summaries(const float* __restrict__ ksum, const float* __restrict__ vsum,
                                    const float* __restrict__ bias, uint16_t* __restrict__ ks16,
                                    uint16_t* __restrict__ vs16t, float* __restrict__ bias2, int H,
                                    int N, int D, int BK, int nb, int nbp) {
  const long total = (long)H * nbp * D;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total;
       e += (long)gridDim.x * blockDim.x) {
    const int c = (int)(e % D);
    const long hb = e / D;
    const int B = (int)(hb % nbp);
    const int h = (int)(hb / nbp);
    float kv = 0.f, vv = 0.f;
    if (B < nb) {
      kv = ksum[((long)h * nb + B) * D + c];
      vv = vsum[((long)h * nb + B) * D + c];
    }
    ks16[e] = f2bf(kv);
    const int tile = B / BK, j = B % BK;
    vs16t[(((long)h * (nbp / BK) + tile) * D + c) * BK + j] = f2bf(vv);
    if (c == 0) {
      float b2 = -INFINITY;
      if (B < nb) {
        const int nB = (B == nb - 1) ? (N - (nb - 1) * BK) : BK;
        b2 = (bias[(long)h * nb + B] + logf((float)nB)) * kLog2e;
      }
      bias2[(long)h * nbp + B] = b2;
    }
  }
}

// Workgroup -> (head, query block) so that consecutive query blocks of one
// head run on the same XCD (workgroups are dealt to the 8 XCDs round-robin),
// sharing that XCD's L2 for the key blocks they both select.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int q = G / 8, r = G % 8;
  const int xcd = bid % 8, pos = bid / 8;
  return (xcd < r) ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

// Position inside a 32-row tile at which K row j is stored, so that the
// S^T accumulator of lane half h holds keys 8h..8h+7 (and 16+8h..16+8h+7)
// in order -- exactly the B-operand layout the P^T of the PV product needs.
__device__ __forceinline__ int kslot32(int j) {
  const int a2 = j >> 4, hh = (j >> 3) & 1, a1 = (j >> 2) & 1, c = j & 3;
  return 8 * (2 * a2 + a1) + 4 * hh + c;
}

template <int D, int BK>
struct MfmaCfg {
  static constexpr int NW = BK / 32;     // waves per workgroup
  static constexpr int NT = NW * 64;     // threads
  static constexpr int RSK = D + 8;      // LDS row stride of K (bf16), +16 B pad
  static constexpr int RSV = BK + 8;     // LDS row stride of V^T
  static constexpr int K_CHUNKS = BK * D / 8;  // 16-byte chunks per tile
  static constexpr int V_CHUNKS = D * BK / 8;
  static constexpr int KPT = K_CHUNKS / NT;    // chunks per thread
  static constexpr int VPT = V_CHUNKS / NT;
  static constexpr int LDS_TILES = (BK * RSK + D * RSV) * 2;  // bytes
};

template <int D, int BK>
__global__ __launch_bounds__(2 * BK) void attn_mfma(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vpt, const int32_t* __restrict__ idx, int topk,
    const uint16_t* __restrict__ ks16, const uint16_t* __restrict__ vs16t,
    const float* __restrict__ bias2, const int32_t* __restrict__ perm_q,
    uint16_t* __restrict__ out, int H, int N, int nb, int nbp, float scale_log2) {
  using C = MfmaCfg<D, BK>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sV = sK + BK * C::RSK;
  float* sBias = reinterpret_cast<float*>(smem + C::LDS_TILES);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int h = logical / nb, A = logical % nb;
  const long Np = (long)nb * BK;
  const int nct = (topk < nb) ? nbp / BK : 0;   // compressed tiles
  const int ntiles = topk + nct;
  const int32_t* myidx = idx + ((long)h * nb + A) * topk;

  // --- summaries' bias in LDS, selected blocks masked --------------------
  if (nct > 0) {
    for (int i = tid; i < nbp; i += C::NT) sBias[i] = bias2[(long)h * nbp + i];
    __syncthreads();
    for (int t = tid; t < topk; t += C::NT) sBias[myidx[t]] = -INFINITY;
  }

  // --- Q operand (B of S^T = K Q^T): row l32 of this wave, d = 16s+8hf.. --
  const long qrow = (long)h * Np + (long)A * BK + wave * 32 + l32;
  bf16x8 qop[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qop[s] = *reinterpret_cast<const bf16x8*>(qp + qrow * D + 16 * s + 8 * hf);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // --- tile source addresses ----------------------------------------------
  // exact tile t < topk: key block idx[t]; compressed tile: summaries t - topk
#define SPARK_TILE_SRC(t, ksrc, vsrc)                                        \
  if ((t) < topk) {                                                          \
    const int B_ = myidx[(t)];                                               \
    ksrc = kp + ((long)h * Np + (long)B_ * BK) * D;                          \
    vsrc = vpt + ((long)h * nb + B_) * (long)D * BK;                         \
  } else {                                                                   \
    const int c_ = (t) - topk;                                               \
    ksrc = ks16 + ((long)h * nbp + (long)c_ * BK) * D;                       \
    vsrc = vs16t + ((long)h * (nbp / BK) + c_) * (long)D * BK;               \
  }
  for (int t = 0; t < ntiles; ++t) {
    const uint16_t *ksrc, *vsrc;
    SPARK_TILE_SRC(t, ksrc, vsrc)
    __syncthreads();  // previous tile fully consumed (and sBias ready)
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int ch = tid + i * C::NT;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      const int slot = (row & ~31) + kslot32(row & 31);
      *reinterpret_cast<uint4*>(sK + slot * C::RSK + col) =
          *reinterpret_cast<const uint4*>(ksrc + (long)ch * 8);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int ch = tid + i * C::NT;
      const int row = ch / (BK / 8), col = (ch % (BK / 8)) * 8;
      *reinterpret_cast<uint4*>(sV + row * C::RSV + col) =
          *reinterpret_cast<const uint4*>(vsrc + (long)ch * 8);
    }
    __syncthreads();

    // S^T = K Q^T for the BK keys of this tile
    f32x16 sacc[BK / 32];
#pragma unroll
    for (int jt = 0; jt < BK / 32; ++jt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sK + (32 * jt + l32) * C::RSK + 16 * s + 8 * hf);
        sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[s], sacc[jt], 0, 0, 0);
      }
    }

    // logits in the log2 domain; key of (jt, v) is 32jt + (v<8 ? 8hf+v : 16+8hf+v-8)
    float mx = -INFINITY;
    if (t < topk) {
      const int B = myidx[t];
      const int valid = (B == nb - 1) ? (N - (nb - 1) * BK) : BK;
#pragma unroll
      for (int jt = 0; jt < BK / 32; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float s2 = sacc[jt][v] * scale_log2;
          if (valid < BK) {
            const int j = 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
            if (j >= valid) s2 = -INFINITY;
          }
          sacc[jt][v] = s2;
          mx = fmaxf(mx, s2);
        }
    } else {
      const float* bb = sBias + (t - topk) * BK;
#pragma unroll
      for (int jt = 0; jt < BK / 32; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
          const float s2 = sacc[jt][v] * scale_log2 + bb[j];
          sacc[jt][v] = s2;
          mx = fmaxf(mx, s2);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pop[BK / 16];
#pragma unroll
    for (int jt = 0; jt < BK / 32; ++jt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[jt][8 * hh + e] - m_new);
          psum += p;
          pop[2 * jt + hh][e] = (__bf16)p;
        }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sV + (32 * dt + l32) * C::RSV + 16 * ks + 8 * hf);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[ks], oacc[dt], 0, 0, 0);
      }
  }

#undef SPARK_TILE_SRC
  // --- epilogue: normalise and scatter back to the original token order ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  const long prow = (long)A * BK + wave * 32 + l32;  // permuted row
  uint16_t* dst;
  if (perm_q != nullptr) {
    if (prow >= N) return;
    dst = out + ((long)h * N + perm_q[(long)h * N + prow]) * D;
  } else {
    dst = out + ((long)h * Np + prow) * D;
  }
  const bool pad = prow >= N;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = pad ? 0.f : oacc[dt][4 * a + c] * inv;
      uint2 w;
      w.x = pack_bf2(o[0], o[1]);
      w.y = pack_bf2(o[2], o[3]);
      *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * a + 4 * hf) = w;
    }
}

// ---------------------------------------------------------------------------
// attn_mfma_d128: the d = 128, block = 128 kernel.
//
// 8 waves per workgroup: wave w owns query rows 32*(w&3).. and keys
// 64*(w>>2).. of every tile, i.e. the two waves of a row group split each key
// tile and keep independent online-softmax states that are merged at the end.
// Two waves per SIMD let one wave's softmax (VALU, exp) run while the other
// issues MFMAs.  K and V^T tiles are double-buffered in LDS and filled by
// direct global->LDS loads (global_load_lds_dwordx4) issued one tile ahead,
// so no registers hold the prefetch.  Tiles are stored with 256-byte rows and
// the 16-byte chunk index XOR-swizzled by (row & 15), which keeps the
// MFMA-operand reads (16 rows x 16 B per quarter-wave) free of bank conflicts
// without padding (direct loads fill 1 KB contiguous per instruction).
// The running max is only raised when a tile's max exceeds it by more than
// 8 (log2 units); otherwise the stale max is kept and the O rescale skipped
// (exact: numerator and denominator use the same reference).
// ---------------------------------------------------------------------------
constexpr int V2_NT = 512;                 // 8 waves
constexpr int V2_TILE_BYTES = 2 * 128 * 256;   // K + V^T of one tile
constexpr int V2_LDS_TILES = 2 * V2_TILE_BYTES;  // double buffer: 128 KB

__device__ __forceinline__ int sw_off(int row, int lc) {  // byte offset in a 128x256 B tile
  return row * 256 + ((lc ^ (row & 15)) << 4);
}

// Head-major order with each head's query blocks split into 8 contiguous
// ranges, one per XCD: every XCD works on the same head at the same time
// (that head's K/V stays in the shared last-level cache), and each XCD walks
// tree-adjacent query blocks (similar selections, L2 reuse).
__device__ __forceinline__ bool v2_map(int bid, int nb, int& h, int& A) {
  const int nb8 = (nb + 7) & ~7;
  h = bid / nb8;
  const int r = bid - h * nb8;
  A = (r & 7) * (nb8 >> 3) + (r >> 3);
  return A < nb;
}

__global__ __launch_bounds__(V2_NT) void attn_mfma_d128(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vpt, const int32_t* __restrict__ idx, int topk,
    const uint16_t* __restrict__ ks16, const uint16_t* __restrict__ vs16t,
    const float* __restrict__ bias2, const int32_t* __restrict__ perm_q,
    uint16_t* __restrict__ out, int H, int N, int nb, int nbp, float scale_log2) {
  constexpr int D = 128, BK = 128;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* sBias = reinterpret_cast<float*>(smem + V2_LDS_TILES);

  int h, A;
  if (!v2_map(blockIdx.x, nb, h, A)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int rg = wave & 3, kh = wave >> 2;
  const long Np = (long)nb * BK;
  const int nct = (topk < nb) ? nbp / BK : 0;
  const int ntiles = topk + nct;
  const int32_t* myidx = idx + ((long)h * nb + A) * topk;

  if (nct > 0) {
    for (int i = tid; i < nbp; i += V2_NT) sBias[i] = bias2[(long)h * nbp + i];
    __syncthreads();
    for (int t = tid; t < topk; t += V2_NT) sBias[myidx[t]] = -INFINITY;
    // made visible by the first barrier of the tile loop
  }

  // direct-load plan of this wave: 8 x 1 KB per tile; instructions g = 8w..8w+7
  // (g < 32: K slots 4g..4g+3; g >= 32: V^T rows 4(g-32)..)
  const int p_row = lane >> 4, p_pc = lane & 15;
  auto issue_tile = [&](int t, int buf) {
    const uint16_t* ksrc;
    const uint16_t* vsrc;
    if (t < topk) {
      const int B = myidx[t];
      ksrc = kp + ((long)h * Np + (long)B * BK) * D;
      vsrc = vpt + ((long)h * nb + B) * (long)D * BK;
    } else {
      const int c = t - topk;
      ksrc = ks16 + ((long)h * nbp + (long)c * BK) * D;
      vsrc = vs16t + ((long)h * (nbp / BK) + c) * (long)D * BK;
    }
    unsigned char* base = smem + buf * V2_TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = wave * 8 + i;
      const int part = g >> 5, gg = g & 31;
      const int srow = 4 * gg + p_row;
      const int lc = p_pc ^ (srow & 15);
      const uint16_t* src;
      if (part == 0) {
        const int grow = (srow & ~31) + ((((srow & 31) >> 3) >> 1) << 4) + (((srow >> 2) & 1) << 3) +
                         ((((srow & 31) >> 3) & 1) << 2) + (srow & 3);
        src = ksrc + (long)grow * D + lc * 8;
      } else {
        src = vsrc + (long)srow * BK + lc * 8;
      }
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)src,
          (void __attribute__((address_space(3)))*)(base + part * (128 * 256) + gg * 1024), 16, 0, 0);
    }
  };

  // Q operand: rows 32rg + l32, d = 16s + 8hf ..
  const long qrow = (long)h * Np + (long)A * BK + rg * 32 + l32;
  bf16x8 qop[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qop[s] = *reinterpret_cast<const bf16x8*>(qp + qrow * D + 16 * s + 8 * hf);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m_ref = -1e30f, l_run = 0.f;

  if (ntiles > 0) issue_tile(0, 0);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t landed (all waves); buffer buf^1 free
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const unsigned char* tK = smem + buf * V2_TILE_BYTES;
    const unsigned char* tV = tK + 128 * 256;

    // S^T for keys 64kh .. 64kh+63 (two 32-key tiles)
    f32x16 sacc[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
      const int row = 32 * (2 * kh + jt) + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(tK + sw_off(row, 2 * s + hf));
        sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[s], sacc[jt], 0, 0, 0);
      }
    }

    float mx = -INFINITY;
    if (t < topk) {
      const int B = myidx[t];
      const int valid = (B == nb - 1) ? (N - (nb - 1) * BK) : BK;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float s2 = sacc[jt][v] * scale_log2;
          if (valid < BK) {
            const int j = 64 * kh + 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
            if (j >= valid) s2 = -INFINITY;
          }
          sacc[jt][v] = s2;
          mx = fmaxf(mx, s2);
        }
    } else {
      const float* bb = sBias + (t - topk) * BK + 64 * kh;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
          const float s2 = fmaf(sacc[jt][v], scale_log2, bb[j]);
          sacc[jt][v] = s2;
          mx = fmaxf(mx, s2);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // raise the reference max only when this tile exceeds it by > 8
    const bool need = mx > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    bf16x8 pop[4];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[jt][8 * hh + e] - m_ref);
          l_run += p;
          pop[2 * jt + hh][e] = (__bf16)p;
        }

    // O^T += V^T P^T over this wave's 64 keys
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ks = 4 * kh + kk;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(tV + sw_off(32 * dt + l32, 2 * ks + hf));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kk], oacc[dt], 0, 0, 0);
      }
  }

  // --- merge the two key halves of each row group, then scatter ---------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  __syncthreads();  // all waves done with the tile buffers
  float* sm = reinterpret_cast<float*>(smem);
  // per row group: [64 lanes][16 v][4 dt] O^T values + m, l per lane
  float* mo = sm + rg * (64 * 16 * 4 + 128);
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mo[(dt * 16 + v) * 64 + lane] = oacc[dt][v];
    mo[64 * 64 + lane] = m_ref;
    mo[64 * 64 + 64 + lane] = l_tot;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m2 = mo[64 * 64 + lane], l2 = mo[64 * 64 + 64 + lane];
  const float mm = fmaxf(m_ref, m2);
  const float f1 = __builtin_amdgcn_exp2f(m_ref - mm), f2 = __builtin_amdgcn_exp2f(m2 - mm);
  const float inv = 1.f / (l_tot * f1 + l2 * f2);
  const long prow = (long)A * BK + rg * 32 + l32;
  uint16_t* dst;
  if (perm_q != nullptr) {
    if (prow >= N) return;
    dst = out + ((long)h * N + perm_q[(long)h * N + prow]) * D;
  } else {
    dst = out + ((long)h * Np + prow) * D;
  }
  const bool pad = prow >= N;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int v = 4 * a + c;
        const float val = (oacc[dt][v] * f1 + mo[(dt * 16 + v) * 64 + lane] * f2) * inv;
        o[c] = pad ? 0.f : val;
      }
      uint2 w;
      w.x = pack_bf2(o[0], o[1]);
      w.y = pack_bf2(o[2], o[3]);
      *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * a + 4 * hf) = w;
    }
}

// ---------------------------------------------------------------------------
// Generic VALU kernel: one thread per query row of the block.
// ---------------------------------------------------------------------------
constexpr int GEN_CH = 32;  // keys per staged chunk

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_generic(
    const T* __restrict__ qp, const T* __restrict__ kp, const T* __restrict__ vpt,
    const int32_t* __restrict__ idx, int topk, const float* __restrict__ ksum,
    const float* __restrict__ vsum, const float* __restrict__ bias,
    const int32_t* __restrict__ perm_q, T* __restrict__ out, int H, int N, int BK, int nb,
    float scale) {
  __shared__ float sK[GEN_CH][D];
  __shared__ float sV[GEN_CH][D];
  __shared__ float sB[GEN_CH];
  extern __shared__ unsigned char smask[];  // nb bytes: 1 = selected

  const int tid = threadIdx.x;
  const int h = blockIdx.x / nb, A = blockIdx.x % nb;
  const long Np = (long)nb * BK;
  const int32_t* myidx = idx + ((long)h * nb + A) * topk;
  for (int i = tid; i < nb; i += blockDim.x) smask[i] = 0;
  __syncthreads();
  for (int t = tid; t < topk; t += blockDim.x) smask[myidx[t]] = 1;
  __syncthreads();

  const long prow = (long)A * BK + tid;
  const bool active = tid < BK;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = active ? Elem<T>::load(qp + ((long)h * Np + prow) * D + c) : 0.f;
    o[c] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;

  auto consume = [&](int cnt) {  // logits of sK[0..cnt) with sB weights
    float s[GEN_CH];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < GEN_CH; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], sK[j][c], acc);
      s[j] = (j < cnt) ? acc * scale + sB[j] : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = expf(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < GEN_CH; ++j) {
      const float p = expf(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, sV[j][c], o[c]);
    }
  };

  // exact branch
  for (int t = 0; t < topk; ++t) {
    const int B = myidx[t];
    const int valid = (B == nb - 1) ? (N - (nb - 1) * BK) : BK;
    for (int j0 = 0; j0 < valid; j0 += GEN_CH) {
      const int cnt = min(GEN_CH, valid - j0);
      __syncthreads();
      for (int e = tid; e < GEN_CH * D; e += blockDim.x) {
        const int j = e / D, c = e % D;
        float kv = 0.f, vv = 0.f;
        if (j < cnt) {
          kv = Elem<T>::load(kp + ((long)h * Np + (long)B * BK + j0 + j) * D + c);
          vv = Elem<T>::load(vpt + (((long)h * nb + B) * D + c) * BK + j0 + j);
        }
        sK[j][c] = kv;
        sV[j][c] = vv;
      }
      for (int j = tid; j < GEN_CH; j += blockDim.x) sB[j] = 0.f;
      __syncthreads();
      consume(cnt);
    }
  }
  // compressed branch: every unselected block, weight |B| through log|B|
  for (int B0 = 0; B0 < nb; B0 += GEN_CH) {
    const int cnt = min(GEN_CH, nb - B0);
    __syncthreads();
    for (int e = tid; e < GEN_CH * D; e += blockDim.x) {
      const int j = e / D, c = e % D;
      sK[j][c] = (j < cnt) ? ksum[((long)h * nb + B0 + j) * D + c] : 0.f;
      sV[j][c] = (j < cnt) ? vsum[((long)h * nb + B0 + j) * D + c] : 0.f;
    }
    for (int j = tid; j < GEN_CH; j += blockDim.x) {
      const int B = B0 + j;
      float bb = -INFINITY;
      if (j < cnt && !smask[B]) {
        const int nB = (B == nb - 1) ? (N - (nb - 1) * BK) : BK;
        bb = bias[(long)h * nb + B] + logf((float)nB);
      }
      sB[j] = bb;
    }
    __syncthreads();
    consume(cnt);
  }

  if (!active) return;
  const float inv = 1.f / l_run;
  T* dst;
  if (perm_q != nullptr) {
    if (prow >= N) return;
    dst = out + ((long)h * N + perm_q[(long)h * N + prow]) * D;
  } else {
    dst = out + ((long)h * Np + prow) * D;
  }
  const bool pad = prow >= N;
#pragma unroll
  for (int c = 0; c < D; ++c) Elem<T>::store(dst + c, pad ? 0.f : o[c] * inv);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t attn_ws_bytes(int H, int N, int D, int BK, int dtype) {
  if (dtype != SPARK_BF16 || (BK != 32 && BK != 64 && BK != 128)) return 0;
  const int nb = cdiv(N, BK);
  const int nbp = cdiv(nb, BK) * BK;
  const size_t a = (size_t)H * nbp * D * 2;  // ks16
  const size_t b = (size_t)H * nbp * D * 2;  // vs16t
  const size_t c = (size_t)H * nbp * 4;      // bias2
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(a) + up(b) + up(c);
}

bool attn_uses_mfma(int dtype, int BK) {
  return dtype == SPARK_BF16 && (BK == 32 || BK == 64 || BK == 128);
}

template <int D, int BK>
static int launch_mfma(const void* qp, const void* kp, const void* vpt, const int32_t* idx,
                       int topk, const uint16_t* ks16, const uint16_t* vs16t, const float* bias2,
                       const int32_t* perm_q, void* out, int H, int N, int nb, int nbp,
                       hipStream_t st) {
  using C = MfmaCfg<D, BK>;
  const size_t lds = C::LDS_TILES + (size_t)nbp * 4;
  if (lds > 160 * 1024)
    return spark_set_error(SPARK_E_SHAPE, "spark_attn: %d blocks need %zu B of LDS (max 163840)",
                           nb, lds);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma<D, BK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        160 * 1024);
    attr_set = true;
  }
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((attn_mfma<D, BK>), dim3(H * nb), dim3(C::NT), lds, st,
                     (const uint16_t*)qp, (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk,
                     ks16, vs16t, bias2, perm_q, (uint16_t*)out, H, N, nb, nbp, scale_log2);
  return spark_check_launch("attn_mfma");
}

static int launch_v2(const void* qp, const void* kp, const void* vpt, const int32_t* idx, int topk,
                     const uint16_t* ks16, const uint16_t* vs16t, const float* bias2,
                     const int32_t* perm_q, void* out, int H, int N, int nb, int nbp,
                     hipStream_t st) {
  const size_t lds = V2_LDS_TILES + (size_t)nbp * 4;
  if (lds > 160 * 1024)
    return spark_set_error(SPARK_E_SHAPE, "spark_attn: %d blocks need %zu B of LDS (max 163840)",
                           nb, lds);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma_d128, hipFuncAttributeMaxDynamicSharedMemorySize,
                        160 * 1024);
    attr_set = true;
  }
  const float scale_log2 = kLog2e / sqrtf(128.f);
  const int nb8 = (nb + 7) & ~7;
  hipLaunchKernelGGL(attn_mfma_d128, dim3(H * nb8), dim3(V2_NT), lds, st, (const uint16_t*)qp,
                     (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk, ks16, vs16t, bias2,
                     perm_q, (uint16_t*)out, H, N, nb, nbp, scale_log2);
  return spark_check_launch("attn_mfma_d128");
}

template <typename T, int D>
static int launch_generic(const void* qp, const void* kp, const void* vpt, const int32_t* idx,
                          int topk, const float* ksum, const float* vsum, const float* bias,
                          const int32_t* perm_q, void* out, int H, int N, int BK, int nb,
                          hipStream_t st) {
  if (nb > 64 * 1024)
    return spark_set_error(SPARK_E_SHAPE, "spark_attn: too many blocks (%d) for the generic kernel", nb);
  const float scale = 1.f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_generic<T, D>), dim3(H * nb), dim3(128), (size_t)nb, st,
                     (const T*)qp, (const T*)kp, (const T*)vpt, idx, topk, ksum, vsum, bias,
                     perm_q, (T*)out, H, N, BK, nb, scale);
  return spark_check_launch("attn_generic");
}

int attn_launch(int H, int N, int D, int BK, int dtype, const void* qp, const void* kp,
                const void* vpt, const int32_t* idx, int topk, const float* ksum,
                const float* vsum, const float* bias, const int32_t* perm_q, void* out, void* ws,
                hipStream_t st) {
  const int nb = cdiv(N, BK);
  if (attn_uses_mfma(dtype, BK)) {
    const int nbp = cdiv(nb, BK) * BK;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    uint16_t* ks16 = (uint16_t*)ws;
    uint16_t* vs16t = (uint16_t*)((char*)ws + up((size_t)H * nbp * D * 2));
    float* bias2 = (float*)((char*)ws + 2 * up((size_t)H * nbp * D * 2));
    const long total = (long)H * nbp * D;
    const int grid = (int)std::min<long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(attn_prep_summaries, dim3(grid), dim3(256), 0, st, ksum, vsum, bias, ks16,
                       vs16t, bias2, H, N, D, BK, nb, nbp);
    int rc = spark_check_launch("attn_prep_summaries");
    if (rc) return rc;
    if (D == 128) {
      if (BK == 128 && (size_t)V2_LDS_TILES + (size_t)nbp * 4 <= 160 * 1024)
        return launch_v2(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
      if (BK == 128) return launch_mfma<128, 128>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
      if (BK == 64) return launch_mfma<128, 64>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
      return launch_mfma<128, 32>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
    } else {
      if (BK == 128) return launch_mfma<64, 128>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
      if (BK == 64) return launch_mfma<64, 64>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
      return launch_mfma<64, 32>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, nb, nbp, st);
    }
  }
  if (dtype == SPARK_F32) {
    if (D == 128) return launch_generic<float, 128>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, BK, nb, st);
    return launch_generic<float, 64>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, BK, nb, st);
  }
  if (D == 128) return launch_generic<uint16_t, 128>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, BK, nb, st);
  return launch_generic<uint16_t, 64>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, BK, nb, st);
}

}  // namespace spark
