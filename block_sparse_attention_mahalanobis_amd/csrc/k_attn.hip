// Fused exact + compressed block-sparse attention with the inverse-permutation
// scatter ("Spark-H3" blog, 01 / Method: Spark-Reblock, the BSA(Q_A) equation
// and the concatenated effective keys/values K~_A, V~_A: one row-wise softmax
// over the exact rows of the selected blocks and, for every other block, its
// summary repeated |B| times; the summaries and log-mass bias come from
// 02 / Method: Spark-Reweight).
//
// Three kernels:
//  * attn_mfma_d128: bf16, d = 128, block 128 (the 768p layer shape); see its
//    own comment below.
//  * attn_mfma: bf16, block size 32/64/128, d 64/128.  One workgroup per
//    (head, query block), one wave per 32 query rows.  S^T = K Q^T and
//    O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, an
//    online softmax in the log2 domain, K / V^T tiles staged through LDS.
//    The compressed branch runs the same loop over tiles of bf16 summaries,
//    with the per-block bias (+ log |B|) added to the logits and the selected
//    blocks masked to -inf.
//  * attn_generic: fp32 or bf16, any block size 1..128; one thread per query
//    row, fp32 VALU arithmetic.  Small and slow; it exists for the fp32
//    workloads and odd block sizes.
//
// Context/sink tokens (01 / Method: Spark-Reblock: they stay exact, outside
// the video-block Top-K budget): with Nv < N video tokens, q_p / k_p / v_pt
// hold nb video blocks followed by nbc context blocks (nbt = nb + nbc).  A
// video query block's exact tiles are its topk selected blocks and then the
// nbc context blocks, followed by the compressed tiles; a context query block
// attends exactly to all nbt blocks and has no compressed branch.  With
// nbc = 0 this is the plain layer.
#include <type_traits>
#include "common.hpp"

namespace spark {

// Tiles of one (head, query block A) workgroup: exact tiles [0, nex) --
// tile t < nidx is key block idx[t], tile t >= nidx is block t + bofs --
// then nct compressed tiles.
struct TilePlan {
  int nidx, nex, bofs, nct;
};
__device__ __forceinline__ TilePlan tile_plan(int A, int nb, int nbc, int topk, int nct_all) {
  TilePlan p;
  if (A < nb) {
    p.nidx = topk;
    p.nex = topk + nbc;
    p.bofs = nb - topk;
    p.nct = (topk < nb) ? nct_all : 0;
  } else {
    p.nidx = 0;
    p.nex = nb + nbc;
    p.bofs = 0;
    p.nct = 0;
  }
  return p;
}

// Real rows of key block B (the last video block and the last context block
// may be short).
__device__ __forceinline__ int block_rows(int B, int nb, int nbt, int N, int Nv, int BK) {
  if (B == nb - 1) return Nv - (nb - 1) * BK;
  if (B == nbt - 1) return N - Nv - (nbt - nb - 1) * BK;
  return BK;
}

// Output row of query row r of block A: its position in the unpadded
// permuted order (video rows [0, Nv), then the context rows), or -1 for a
// padding row.  Context rows keep their original position.
__device__ __forceinline__ long out_pos(int A, int r, int nb, int N, int Nv, int BK) {
  const long p = (A < nb) ? (long)A * BK + r : (long)Nv + (long)(A - nb) * BK + r;
  return p < ((A < nb) ? Nv : N) ? p : -1;
}

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
    uint16_t* __restrict__ out, int H, int N, int Nv, int nb, int nbc, int nbp, float scale_log2) {
  using C = MfmaCfg<D, BK>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sV = sK + BK * C::RSK;
  float* sBias = reinterpret_cast<float*>(smem + C::LDS_TILES);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int nbt = nb + nbc;
  const int h = logical / nbt, Ar = logical % nbt;
  const int A = (Ar < nbc) ? nb + Ar : Ar - nbc;   // context query blocks first
  const long Np = (long)nbt * BK;
  const TilePlan tp = tile_plan(A, nb, nbc, topk, nbp / BK);
  const int nct = tp.nct;
  const int ntiles = tp.nex + nct;
  const int32_t* myidx = (A < nb) ? idx + ((long)h * nb + A) * topk : idx;

  // --- summaries' bias in LDS, selected blocks masked --------------------
  if (nct > 0) {
    for (int i = tid; i < nbp; i += C::NT) sBias[i] = bias2[(long)h * nbp + i];
    __syncthreads();
    for (int t = tid; t < tp.nidx; t += C::NT) sBias[myidx[t]] = -INFINITY;
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
  // exact tile t < tp.nex: key block B (see TilePlan); compressed tile:
  // summaries t - tp.nex
#define SPARK_TILE_SRC(t, ksrc, vsrc)                                        \
  if ((t) < tp.nex) {                                                        \
    const int B_ = ((t) < tp.nidx) ? myidx[(t)] : (t) + tp.bofs;             \
    ksrc = kp + ((long)h * Np + (long)B_ * BK) * D;                          \
    vsrc = vpt + ((long)h * nbt + B_) * (long)D * BK;                        \
  } else {                                                                   \
    const int c_ = (t) - tp.nex;                                             \
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
    if (t < tp.nex) {
      const int B = (t < tp.nidx) ? myidx[t] : t + tp.bofs;
      const int valid = block_rows(B, nb, nbt, N, Nv, BK);
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
      const float* bb = sBias + (t - tp.nex) * BK;
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
  const long pos = out_pos(A, wave * 32 + l32, nb, N, Nv, BK);
  uint16_t* dst;
  if (perm_q != nullptr) {
    if (pos < 0) return;
    dst = out + ((long)h * N + ((A < nb) ? perm_q[(long)h * N + pos] : pos)) * D;
  } else {
    dst = out + ((long)h * Np + (long)A * BK + wave * 32 + l32) * D;
  }
  const bool pad = pos < 0;
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
// Helpers of the d = 128 kernel.  Tiles sit in LDS as 128 rows of 256 bytes
// with the 16-byte chunk index XOR-swizzled by (row & 15): the MFMA operand
// reads (16 consecutive rows, one chunk each, per quarter-wave) then hit 16
// different bank groups, and the direct global->LDS loads, which write 1 KB
// contiguous per instruction, need no padding.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sw_off(int row, int lc) {  // byte offset in a 128x256 B tile
  return row * 256 + ((lc ^ (row & 15)) << 4);
}

// Head-major order with each head's video query blocks split into 8
// contiguous ranges, one per XCD (workgroup bid runs on XCD bid % 8): every
// XCD works on the same head at the same time (that head's K/V stays in the
// shared last-level cache), and each XCD walks tree-adjacent query blocks
// (similar selections, L2 reuse).  Context query blocks, which attend to
// every block and so run ~nbt/(topk+nbc) times longer, are dealt round-robin
// over the XCDs and placed first in each XCD's share of the head, so they
// start early and the short blocks fill in behind them.
__device__ __forceinline__ int d128_slots(int nb, int nbc) {  // workgroups per head
  return 8 * (((nbc + 7) >> 3) + ((nb + 7) >> 3));
}
__device__ __forceinline__ bool d128_map(int bid, int nb, int nbc, int& h, int& A, bool ctx_only = false) {
  const int cpx = (nbc + 7) >> 3, vpx = ctx_only ? 0 : (nb + 7) >> 3;
  const int R = 8 * (cpx + vpx);
  h = bid / R;
  const int r = bid - h * R;
  const int x = r & 7, j = r >> 3;
  if (j < cpx) {
    const int c = j * 8 + x;
    A = nb + c;
    return c < nbc;
  }
  A = x * vpx + (j - cpx);
  return A < nb;
}

// ---------------------------------------------------------------------------
// attn_mfma_d128: d = 128, block = 128, 4 waves x 32 query rows, full 128-key
// tiles per wave, and TWO workgroups per CU (72 KB of LDS each): while one
// workgroup waits on a barrier or a tile load the other one's waves issue
// MFMAs and softmax, so the two interleave on every SIMD.  K and V^T use one
// LDS buffer each, refilled by direct global->LDS loads in split phases:
// K(t+1) streams in during softmax(t) + PV(t), V(t+1) during QK(t+1) +
// softmax(t+1).
// ---------------------------------------------------------------------------
constexpr int D128_NT = 256;
constexpr int D128_PF = 2;   // operand prefetch distance, in 16-deep k steps

// Issue order of one 4-MFMA-per-step block (mask 0x100: LDS reads, 0x008:
// MFMAs): the operand reads of the first D128_PF steps, then for every step
// its 4 MFMAs, each followed by one read D128_PF steps ahead.
template <int STEPS>
__device__ __forceinline__ void d128_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * D128_PF, 0);
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s + D128_PF < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}
constexpr int D128_LDS_TILES = 2 * 128 * 256;   // K + V^T, 64 KB
// Workgroup barrier without a memory fence: the waves' own LDS reads are
// complete (lgkmcnt(0)) and the direct loads are waited for explicitly with
// vmcnt counts, so loads issued for a later tile stay in flight across it
// (a fenced barrier would wait for every outstanding direct load, which the
// compiler counts as an LDS write).  The asm memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void d128_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
}

// fp8 logits: issue order of the QK block (16 LDS reads of 16 bytes, 8
// 32x32x64 MFMAs): the first k step's reads, then each MFMA of that step
// followed by two reads of the second step, then the second step's MFMAs.
__device__ __forceinline__ void d128_pipeline_fp8() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Smallest power of two s with amax <= 448 s (the E4M3 group scale; 1 for
// amax = 0 or not finite).
__device__ __forceinline__ float attn_pow2_scale(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 1.f;
  int e;
  frexpf(amax, &e);
  e -= 9;
  while (amax > 448.f * ldexpf(1.f, e)) ++e;
  while (amax <= 448.f * ldexpf(1.f, e - 1)) --e;
  return ldexpf(1.f, e);
}
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 query row for the fp8 logits: lane (l32, hf) holds d = 64 s + 32 hf +
// 0..31 of its row (s = 0, 1), scaled by the row's power-of-two scale
// (the smallest s with max |q| <= 448 s, taken over the lane pair).
__device__ __forceinline__ void attn_q8(const uint16_t* __restrict__ qp, long qrow, int hf, i32x8 (&q8)[2],
                                        float& qscale) {
  constexpr int D = 128;
  bf16x8 raw[2][4];
  float amax = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      raw[s2][u] = *reinterpret_cast<const bf16x8*>(qp + qrow * D + 64 * s2 + 32 * hf + 8 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[s2][u][e]));
    }
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  qscale = attn_pow2_scale(amax);
  const float inv = 1.f / qscale;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const bf16x8 r = raw[s2][u];
        const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((float)r[4 * w] * inv,
                                                                       (float)r[4 * w + 1] * inv, 0, false) & 0xffffu;
        const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((float)r[4 * w + 2] * inv,
                                                                       (float)r[4 * w + 3] * inv, 0, false) & 0xffffu;
        q8[s2][2 * u + w] = (int)(lo | (hi << 16));
      }
}

// Sum of the 64 bf16 P values a lane holds, two bf16 per dot-product step
// (against (1, 1)), in two interleaved partial sums: the softmax denominator
// is summed from the same rounded P that multiplies V.
__device__ __forceinline__ float rowsum_bf16(const bf16x8 (&pop)[8]) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16x8 v = pop[i];
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, s1, false);
  }
  return s0 + s1;
}

// CTX = false (no context blocks) compiles the tile bookkeeping of the plain
// layer: one compare less per tile and the idx load unconditional.
// FP8: the logits come from E4M3 operands ([blog] Benchmark Results' FP8
// runs): kp / ks16 then point at E4M3 key tiles (16 KB, one power-of-two
// scale per tile in kscale / ksscale), each query row is rounded to E4M3
// with its own scale in registers, and S^T runs on 32x32x64 fp8 MFMAs;
// P V stays bf16.
template <bool CTX, bool FP8>
__global__ __launch_bounds__(D128_NT, 2) void attn_mfma_d128(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vpt, const int32_t* __restrict__ idx, int topk,
    const uint16_t* __restrict__ ks16, const uint16_t* __restrict__ vs16t,
    const float* __restrict__ bias2, const int32_t* __restrict__ perm_q,
    uint16_t* __restrict__ out, int H, int N, int Nv, int nb, int nbc, int nbp, float scale_log2,
    const float* __restrict__ kscale, const float* __restrict__ ksscale, int ctx_only) {
  constexpr int D = 128, BK = 128;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  unsigned char* sK = smem;
  unsigned char* sV = smem + 128 * 256;
  float* sBias = reinterpret_cast<float*>(smem + D128_LDS_TILES);

  if constexpr (!CTX) nbc = 0;
  int h, A;
  if (!d128_map(blockIdx.x, nb, nbc, h, A, ctx_only != 0)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index as a scalar: every LDS destination of a direct load is
  // then computed in SGPRs (M0 needs no v_readfirstlane, a VALU op that would
  // queue behind the other wave's MFMAs)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int nbt = nb + nbc;
  const long Np = (long)nbt * BK;
  TilePlan tp;
  if constexpr (CTX) {
    tp = tile_plan(A, nb, nbc, topk, nbp / BK);
  } else {
    tp.nidx = topk;
    tp.nex = topk;
    tp.bofs = 0;
    tp.nct = (topk < nb) ? nbp / BK : 0;
  }
  const int nct = tp.nct;
  const int ntiles = tp.nex + nct;
  const int32_t* myidx = (A < nb) ? idx + ((long)h * nb + A) * topk : idx;

  if (nct > 0) {
    for (int i = tid; i < nbp; i += D128_NT) sBias[i] = bias2[(long)h * nbp + i];
    __syncthreads();
    for (int t = tid; t < tp.nidx; t += D128_NT) sBias[myidx[t]] = -INFINITY;
  }

  // per-lane byte offsets (loop invariant) of this wave's 8 direct loads per
  // tensor: instruction i fills LDS rows 4*(8*wave+i) .. +3.  Loads i and i+4
  // fill rows 16 apart, which sit 16 rows (4096 bytes) apart in the source
  // tile for K and V^T alike, so only i = 0..3 need lane offsets; the 4096
  // goes into the scalar offset.
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int srow = 4 * (8 * wave + i) + (lane >> 4);
    const int lc = (lane & 15) ^ (srow & 15);
    const int grow = (srow & ~31) + ((((srow & 31) >> 3) >> 1) << 4) + (((srow >> 2) & 1) << 3) +
                     ((((srow & 31) >> 3) & 1) << 2) + (srow & 3);
    koff[i] = (uint32_t)(grow * D + lc * 8) * 2u;
    voff[i] = (uint32_t)(srow * BK + lc * 8) * 2u;
  }
  if constexpr (FP8) {
    // E4M3 K tile: 128 rows of 128 bytes; load i of this wave fills LDS rows
    // 32 wave + 8 i .. +7, the 16-byte chunk slot XOR-swizzled by (row >> 1) & 7
    // (16 consecutive rows then hit 16 distinct bank groups); rows in the
    // same permuted order as the bf16 tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int srow = 32 * wave + 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((srow >> 1) & 7);
      const int grow = (srow & ~31) + ((((srow & 31) >> 3) >> 1) << 4) + (((srow >> 2) & 1) << 3) +
                       ((((srow & 31) >> 3) & 1) << 2) + (srow & 3);
      koff[i] = (uint32_t)(grow * 128 + c * 16);
    }
  }
  constexpr int KES = FP8 ? 1 : 2;   // bytes per key element
  auto tile_base = [&](int t, const char*& kb, const char*& vb) {
    if (t < tp.nex) {
      const int B = (!CTX || t < tp.nidx) ? myidx[t] : t + tp.bofs;
      kb = reinterpret_cast<const char*>(kp) + ((long)h * Np + (long)B * BK) * D * KES;
      vb = reinterpret_cast<const char*>(vpt + ((long)h * nbt + B) * (long)D * BK);
    } else {
      const int c = t - tp.nex;
      kb = reinterpret_cast<const char*>(ks16) + ((long)h * nbp + (long)c * BK) * D * KES;
      vb = reinterpret_cast<const char*>(vs16t + ((long)h * (nbp / BK) + c) * (long)D * BK);
    }
  };
  // one 16 KB E4M3 key tile, four 1 KB direct loads per wave
  auto issue8 = [&](const char* base, unsigned char* dst) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 128 * 128, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (void __attribute__((address_space(3)))*)(dst + (4 * wave + i) * 1024), 16, koff[i], 0, 0, 0);
  };
  // one 32 KB tile through a buffer resource (scalar base, 32-bit lane
  // offsets; bytes past the tile would read as 0)
  auto issue = [&](const char* base, const uint32_t* off, unsigned char* dst) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 128 * 256, 0x00020000);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (void __attribute__((address_space(3)))*)(dst + (8 * wave + i) * 1024), 16, off[i & 3],
          (i >> 2) * 4096, 0, 0);
  };

  const long qrow = (long)h * Np + (long)A * BK + wave * 32 + l32;
  bf16x8 qop[FP8 ? 1 : D / 16];
  i32x8 q8[2];       // E4M3 query, lane (l32, hf): d = 64 s + 32 hf + 0..31
  float qscale = 1.f;
  if constexpr (FP8) {
    attn_q8(qp, qrow, hf, q8, qscale);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qop[s] = *reinterpret_cast<const bf16x8*>(qp + qrow * D + 16 * s + 8 * hf);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m_ref = -1e30f, l_run = 0.f;

  // per-lane LDS read offsets (loop invariant): row 32*jt + l32, logical
  // chunk 2s + hf; the 32-row tile index only adds the constant jt * 8 KB.
  int ro[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) ro[s] = sw_off(l32, 2 * s + hf);
  // E4M3 K operand reads: row 32 jt + l32, logical chunks 4 s + 2 hf + u
  int ro8[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int u = 0; u < 2; ++u) ro8[s2][u] = l32 * 128 + (((4 * s2 + 2 * hf + u) ^ ((l32 >> 1) & 7)) << 4);

  {
    const char *kb, *vb;
    tile_base(0, kb, vb);
    if constexpr (FP8) {
      issue8(kb, sK);
      issue(vb, voff, sV);
    } else {
      issue(kb, koff, sK);   // V(0) is issued during QK(0)
    }
  }
  auto rsrc32k = [&](const char* base) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 128 * 256, 0x00020000);
  };
  // load i (0..7) of this wave's share of a 32 KB tile
  auto load1 = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t* off, unsigned char* dst, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (void __attribute__((address_space(3)))*)(dst + (8 * wave + i) * 1024), 16, off[i & 3],
        (i >> 2) * 4096, 0, 0);
  };

  for (int t = 0; t < ntiles; ++t) {
    const bool exact = t < tp.nex;
    // K(t) landed (bf16: nothing else is in flight; fp8: V(t) may be)
    if constexpr (FP8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    d128_barrier();
    f32x16 sacc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
    }
    __builtin_amdgcn_s_setprio(2);  // favour the wave that feeds the matrix core
    if constexpr (FP8) {
      i32x8 kop8[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const uint4 lo = *reinterpret_cast<const uint4*>(sK + ro8[s2][0] + jt * 4096);
          const uint4 hi = *reinterpret_cast<const uint4*>(sK + ro8[s2][1] + jt * 4096);
          kop8[s2][jt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          sacc[jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop8[s2][jt], q8[s2], sacc[jt], 0, 0, 0,
                                                                     0, 0, 0);
      d128_pipeline_fp8();
    } else {
      // all 32 K operand reads and MFMAs are written out; the group barriers
      // below fix the issue order: the reads of steps 0..D128_PF-1 first,
      // then each MFMA of step s followed by one read of step s+D128_PF, so
      // every read has D128_PF steps of MFMAs to land in
      // V(t) streams in during this product, one direct load per k step
      const char *kbt, *vbt;
      tile_base(t, kbt, vbt);
      const __amdgpu_buffer_rsrc_t rsv = rsrc32k(vbt);
      bf16x8 kop[D / 16][4];
#pragma unroll
      for (int s = 0; s < D128_PF; ++s)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          kop[s][jt] = *reinterpret_cast<const bf16x8*>(sK + ro[s] + jt * 8192);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        if (s + D128_PF < D / 16) {
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            kop[s + D128_PF][jt] = *reinterpret_cast<const bf16x8*>(sK + ro[s + D128_PF] + jt * 8192);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s][jt], qop[s], sacc[jt], 0, 0, 0);
        load1(rsv, voff, sV, s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    d128_barrier();  // every wave is done reading sK
    const char *kb1 = nullptr, *vb1 = nullptr;
    // bf16: K(t+1) streams in during the softmax; the last tile reloads its
    // own K (unused) so that every tile issues the same loads
    tile_base(t + 1 < ntiles ? t + 1 : t, kb1, vb1);
    if constexpr (FP8) {
      if (t + 1 < ntiles) issue8(kb1, sK);
    }
    const __amdgpu_buffer_rsrc_t rsk = rsrc32k(kb1);

    // P against the lazy reference m_ref: p = 2^(logit * log2 e - m_ref).
    // Every p of a row half is at most that half's sum, so a sum <= 2^12
    // shows that no p exceeds 2^12 (bf16 P and the fp32 sums hold that with
    // room to spare) and m_ref can stay -- no per-tile maximum.  Otherwise
    // (the first tile, or logits that rose by more than ~12 in log2 units)
    // the exact tile maximum is taken, the running sums are rescaled and P
    // is recomputed.
    float lsc = scale_log2;   // logit -> log2 units (fp8: times the two group scales)
    if (exact) {
      const int B = (!CTX || t < tp.nidx) ? myidx[t] : t + tp.bofs;
      if constexpr (FP8) lsc = scale_log2 * qscale * kscale[(long)h * nbt + B];
      const int valid = CTX ? block_rows(B, nb, nbt, N, Nv, BK) : ((B == nb - 1) ? Nv - (nb - 1) * BK : BK);
      if (valid < BK) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
            if (j >= valid) sacc[jt][v] = -INFINITY;
          }
      }
    } else {
      const float* bb = sBias + (t - tp.nex) * BK;
      if constexpr (FP8) lsc = scale_log2 * qscale * ksscale[(long)h * (nbp / BK) + (t - tp.nex)];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + ((v < 8) ? 8 * hf + v : 16 + 8 * hf + v - 8);
          sacc[jt][v] = fmaf(sacc[jt][v], lsc, bb[j]);
        }
    }
    bf16x8 pop[8];
    float psum;
    // exact tiles hold raw logits (the scale is folded into the exp
    // argument), compressed tiles already-scaled, biased ones
#define SPARK_D128_P()                                                                   \
    {                                                                                   \
      const float nm = -m_ref;                                                          \
      const float sc = exact ? lsc : 1.f;                                               \
      _Pragma("unroll") for (int jt = 0; jt < 4; ++jt)                                  \
      _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                  \
      _Pragma("unroll") for (int e = 0; e < 8; ++e)                                     \
        pop[2 * jt + hh][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[jt][8 * hh + e], sc, nm)); \
      psum = rowsum_bf16(pop);                                                          \
    }
    if constexpr (FP8) {
      SPARK_D128_P()
    } else {
      const float nm = -m_ref;
      const float sc = exact ? lsc : 1.f;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pop[2 * jt + hh][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[jt][8 * hh + e], sc, nm));
          load1(rsk, koff, sK, 2 * jt + hh);
          __builtin_amdgcn_sched_barrier(0);
        }
      psum = rowsum_bf16(pop);
    }
    if (__builtin_amdgcn_ballot_w64(!(psum <= 4096.f)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[jt][v]);
      if (exact) mx *= lsc;
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
      SPARK_D128_P()
    }
#undef SPARK_D128_P
    l_run += psum;

    // V(t) landed: only this wave's K(t+1) loads (8 bf16 / 4 fp8) may be outstanding
    if constexpr (FP8) {
      if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // K(t+1) in flight
    }
    d128_barrier();
    __builtin_amdgcn_s_setprio(2);
    {
      bf16x8 vop[BK / 16][4];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          vop[ks][dt] = *reinterpret_cast<const bf16x8*>(sV + ro[ks] + dt * 8192);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[ks][dt], pop[ks], oacc[dt], 0, 0, 0);
      d128_pipeline<BK / 16>();
    }
    __builtin_amdgcn_s_setprio(0);
    d128_barrier();  // every wave is done reading sV
    if constexpr (FP8) {
      if (t + 1 < ntiles) issue(vb1, voff, sV);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last tile's K reload

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  const long pos = out_pos(A, wave * 32 + l32, nb, N, Nv, BK);
  uint16_t* dst;
  if (perm_q != nullptr) {
    if (pos < 0) return;
    dst = out + ((long)h * N + ((A < nb) ? perm_q[(long)h * N + pos] : pos)) * D;
  } else {
    dst = out + ((long)h * Np + (long)A * BK + wave * 32 + l32) * D;
  }
  const bool pad = pos < 0;
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
// Paired query blocks (bf16 logits, d = 128, block 128, no context blocks).
//
// One workgroup of 8 waves owns two adjacent query blocks of one head (leaf
// siblings of the split tree, whose top-k selections overlap the most):
// waves 0-3 (group 0) the even block, waves 4-7 (group 1) the odd one; wave
// w and wave w + 4 share a SIMD.  Each group visits nct + topk tiles in this
// order: the compressed tiles, the exact blocks both groups selected, then
// its own exact blocks.  Up to the end of the shared part one direct load of
// a tile serves both groups, which removes the L2 -> LDS traffic of the
// shared blocks' second copy (about a third of all tile bytes on the 768p
// routing) and the power it costs.
//
// The groups run one slot apart.  In a group's matrix slot it streams P V of
// its previous tile and then S^T of the current one (64 MFMAs); in its next
// slot it computes that tile's softmax.  So in every slot one wave of each
// SIMD feeds the matrix core while the other one runs its vector work, and
// the latter also issues all of the slot's direct loads (issuing them
// stalls a wave, which the matrix core cannot afford).  One workgroup
// barrier ends each slot.  Four 32 KB buffers (K and V^T, two each) hold the
// tiles; the slot in which each tile is loaded is fixed so that no buffer
// is overwritten while a group still reads it:
//   shared K(t) at slot 2t - 2 into K[t & 1]; shared V(t) at 2t + 1 into
//   V[t & 1]; own K(t) of group g at 2t + g - 1 and own V(t) at 2t + g + 1
//   into K/V[pb ^ g], pb the parity of the shared tile count.
// Every wave waits for its own loads at the end of the slot, before the
// barrier, so a tile loaded in slot s is complete in slot s + 1.  The row
// sums add the fp32 p (not the bf16-rounded P): v_dot2c shares the matrix
// core's issue and waits behind the other wave's MFMA stream.
// ---------------------------------------------------------------------------
constexpr int PAIR_NT = 512;
// the tiles loaded in a slot (eight 1 KB direct loads each per loading wave)
struct SlotLoads {
  __amdgpu_buffer_rsrc_t rsk, rsv;   // the K tile and the V^T tile
  int dk, dv;                        // their buffers (0/1)
  bool hk, hv;                       // whether they are loaded
};
constexpr int PAIR_TB = 128 * 256;   // bytes of one bf16 K or V^T tile

// LDS bytes of the paired kernel: 4 tiles, two bias rows, the slot table
// (and with fp8 logits the steps' key scales).
// The plan's scratch (two block bitmaps, the shared and the two own block
// lists, 32 counters) lives in the second K buffer, which no load touches
// before the slot table is built; a plan that would not fit there returns
// a size no workgroup gets.
__host__ __device__ inline size_t pair_lds_bytes(int nb, int nbc, int nbp, int topk, bool fp8) {
  const int ntiles = ((topk < nb) ? nbp / 128 : 0) + nbc + topk;
  const size_t plan = (size_t)2 * ((nb + 31) / 32) * 4 + (size_t)3 * topk * 4 + 32 * 4;
  if (plan > (size_t)PAIR_TB) return ~(size_t)0;
  return (size_t)4 * PAIR_TB + (size_t)2 * nbp * 4 + (size_t)2 * (2 * ntiles + 2) * 8 +
         (fp8 ? (size_t)2 * ntiles * 4 : 0);   // fp8: each step's key scale, per group
}

// FP8: E4M3 logits as in attn_mfma_d128 (kp / ks16 then hold 16 KB E4M3 key
// tiles with one power-of-two scale per tile in kscale / ksscale).
template <bool FP8>
__global__ __launch_bounds__(PAIR_NT, 1) void attn_pair_d128(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vpt, const int32_t* __restrict__ idx, int topk,
    const uint16_t* __restrict__ ks16, const uint16_t* __restrict__ vs16t,
    const float* __restrict__ bias2, const int32_t* __restrict__ perm_q,
    uint16_t* __restrict__ out, int H, int N, int Nv, int nb, int nbc, int nbp, float scale_log2,
    const float* __restrict__ kscale, const float* __restrict__ ksscale) {
  constexpr int D = 128, BK = 128;
  constexpr int KES = FP8 ? 1 : 2;   // bytes per key element
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int nwb = (nb + 31) >> 5;
  float* sBias0 = reinterpret_cast<float*>(smem + 4 * PAIR_TB);
  // per slot: the K tile and the V^T tile it loads
  uint64_t* sSlot = reinterpret_cast<uint64_t*>(sBias0 + 2 * nbp);
  float* sKsc = nullptr;   // fp8: key scale of step t of group g at [g * ntiles + t] (set below)
  // plan scratch, in K buffer 1 (first loaded in slot 0, after the plan)
  uint32_t* sMap = reinterpret_cast<uint32_t*>(smem + PAIR_TB);
  int* sS = reinterpret_cast<int*>(sMap + 2 * nwb);
  int* sP0 = sS + topk;
  int* sP1 = sP0 + topk;
  int* sCnt = sP1 + topk;

  const int tid = threadIdx.x;
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  const int w8 = 4 * grp + wave;
  const int tg = tid & 255, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

  // block pair: head-major, each head's pairs split into 8 contiguous ranges,
  // one per XCD (consecutive workgroups go to consecutive XCDs)
  const int npairs = (nb + 1) >> 1, ppx = (npairs + 7) >> 3;
  const int h = blockIdx.x / (8 * ppx);
  const int r = blockIdx.x - h * 8 * ppx;
  const int pr = (r & 7) * ppx + (r >> 3);
  if (pr >= npairs) return;   // the whole workgroup
  // group 1 of an odd last pair repeats group 0's block and writes nothing
  const bool idle = 2 * pr + grp >= nb;
  const int A = idle ? 2 * pr : 2 * pr + grp;
  const int nbt = nb + nbc;   // video blocks, then context blocks
  const long Np = (long)nbt * BK;
  const int nct = (topk < nb) ? nbp / BK : 0;
  const int cbase = nct + nbc;   // first exact video step
  const int ntiles = cbase + topk;
  const int32_t* myidx = idx + ((long)h * nb + A) * topk;
  // first list entry of this thread, loaded ahead of the query rows and step 0's K
  const int idx0 = (tg < topk) ? myidx[tg] : 0;

  // every K, V^T and summary tile is 32 contiguous KB: per-head bases
  const char* kb_h = reinterpret_cast<const char*>(kp) + (long)h * Np * D * KES;
  const char* vb_h = reinterpret_cast<const char*>(vpt + (long)h * nbt * D * BK);
  const char* ksb_h = reinterpret_cast<const char*>(ks16) + (long)h * nbp * D * KES;
  const char* vsb_h = reinterpret_cast<const char*>(vs16t + (long)h * nbp * D);

  // In every slot the group that is not in its matrix slot loads the slot's
  // tiles (a direct load stalls the issuing wave, which the matrix core
  // cannot afford).  Load j (0..7) of a tile by wave w of that group fills
  // LDS rows srow = 32 w + 4 j + (lane >> 4) (1 KB), the 16-byte chunk
  // XOR-swizzled by srow & 15.  V^T rows come in order; K rows in the
  // permuted order that makes the S^T accumulator the P^T operand, which
  // swaps bits 2 and 3 of the row: the source row is srow + ((j & 1) -
  // ((j >> 1) & 1)) * 4.  K and V share the lane offsets of j & 3; the 4096
  // of j >= 4 and the +-1024 of K go into the scalar offset, with load 2's
  // lane offset stored 1024 low (it is at least 2048).  (An immediate offset
  // would also move the LDS destination.)
  uint32_t loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r4 = 4 * i + (lane >> 4);
    const int lc = (lane & 15) ^ r4;
    loff[i] = (uint32_t)(8192 * wave + r4 * 256 + lc * 16) - (i == 2 ? 1024u : 0u);
  }
  // fp8 K tiles: 128 rows of 128 bytes, in the same permuted row order,
  // the 16-byte chunk slot XOR-swizzled by (row >> 1) & 7
  uint32_t koff8[4];
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int srow = 32 * wave + 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ ((srow >> 1) & 7);
      const int grow = (srow & ~31) + ((((srow & 31) >> 3) >> 1) << 4) + (((srow >> 2) & 1) << 3) +
                       ((((srow & 31) >> 3) & 1) << 2) + (srow & 3);
      koff8[j] = (uint32_t)(grow * 128 + c * 16);
    }
  }
  auto mk_rsrc = [&](const char* src) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, PAIR_TB, 0x00020000);
  };
  // load l (a constant) of a slot: 0..7 the K tile, 8..15 the V^T tile
  auto issue_load = [&](const SlotLoads& L, int l) {
    const int j = l & 7, i = j & 3;
    if (l < 8) {
      if (!L.hk) return;
      if constexpr (FP8) {   // a 16 KB E4M3 tile: loads 0..3 fill rows 32 w + 8 j .. +7
        if (j >= 4) return;
        auto lp = (void __attribute__((address_space(3)))*)(smem + L.dk * PAIR_TB + (4 * wave + j) * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsk, lp, 16, koff8[j], 0, 0, 0);
        return;
      }
      auto lp = (void __attribute__((address_space(3)))*)(smem + L.dk * PAIR_TB + (8 * wave + j) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsk, lp, 16, loff[i], 4096 * (j >> 2) + (i == 1 ? 1024 : 0), 0, 0);
    } else {
      if (!L.hv) return;
      auto lp = (void __attribute__((address_space(3)))*)(smem + (2 + L.dv) * PAIR_TB + (8 * wave + j) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsv, lp, 16, loff[i], 4096 * (j >> 2) + (i == 2 ? 1024 : 0), 0, 0);
    }
  };

  // step 0's K into buffer 0 (buffer 1 holds the plan's scratch until slot 0)
  auto issue_k0 = [&](const char* src) {
    SlotLoads L0;
    L0.rsk = L0.rsv = mk_rsrc(src);
    L0.dk = L0.dv = 0;
    L0.hk = true;
    L0.hv = false;
    if (grp == 1) {   // group 1 has no matrix slot before slot 1
#pragma unroll
      for (int l = 0; l < 8; ++l) issue_load(L0, l);
    }
  };
  if (nct > 0) issue_k0(ksb_h);   // step 0 is summary tile 0
  const long qrow = (long)h * Np + (long)A * BK + wave * 32 + l32;
  bf16x8 qop[FP8 ? 1 : D / 16];
  i32x8 q8[2];
  float qscale = 1.f;
  if constexpr (FP8) {
    attn_q8(qp, qrow, hf, q8, qscale);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qp + qrow * D + 16 * s + 8 * hf);
  }
  int ro8[2][2];   // fp8 K operand reads: row 32 jt + l32, logical chunks 4 s + 2 hf + u
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int u = 0; u < 2; ++u) ro8[s2][u] = l32 * 128 + (((4 * s2 + 2 * hf + u) ^ ((l32 >> 1) & 7)) << 4);
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m_ref = -1e30f, l_run = 0.f;
  int ro[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) ro[s] = sw_off(l32, 2 * s + hf);

  // ---- tile plan: shared blocks (in group 0's order) and each group's own
  float* sBias = sBias0 + grp * nbp;
  uint32_t* myMap = sMap + grp * nwb;
  const uint32_t* otMap = sMap + (1 - grp) * nwb;
  for (int i = tg; i < nwb; i += 256) myMap[i] = 0u;
  for (int i = tid; i < 3 * topk; i += PAIR_NT) sS[i] = 0;   // block 0 where a list is short (bad input)
  if (tid < 3) sCnt[18 + tid] = -1;   // list positions of the last block nb - 1
  if (nct > 0)
    for (int i = tg; i < nbp; i += 256) sBias[i] = bias2[(long)h * nbp + i];
  __syncthreads();
  for (int i = tg; i < topk; i += 256) {
    const int B = min(max((i == tg) ? idx0 : myidx[i], 0), nb - 1);
    atomicOr(&myMap[B >> 5], 1u << (B & 31));
    if (nct > 0) sBias[B] = -INFINITY;
  }
  __syncthreads();
  int cs = 0, cp = 0;
  for (int c0 = 0; c0 < topk; c0 += 256) {
    const int i = c0 + tg;
    const bool valid = i < topk;
    int B = 0;
    bool sh = false;
    if (valid) {
      B = min(max((c0 == 0) ? idx0 : myidx[i], 0), nb - 1);
      sh = (otMap[B >> 5] >> (B & 31)) & 1u;
    }
    const uint64_t bs = __builtin_amdgcn_ballot_w64(valid && sh);
    const uint64_t bp = __builtin_amdgcn_ballot_w64(valid && !sh);
    if (lane == 0) {
      sCnt[grp * 8 + wave] = __builtin_popcountll(bs);
      sCnt[grp * 8 + 4 + wave] = __builtin_popcountll(bp);
    }
    __syncthreads();
    int os = cs, op = cp, ts = 0, tq = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int a = sCnt[grp * 8 + w], b = sCnt[grp * 8 + 4 + w];
      if (w < wave) {
        os += a;
        op += b;
      }
      ts += a;
      tq += b;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int ps_ = os + __builtin_popcountll(bs & lt), pp_ = op + __builtin_popcountll(bp & lt);
    if (valid && sh && grp == 0) {
      sS[ps_] = B;
      if (B == nb - 1) sCnt[18] = ps_;
    }
    if (valid && !sh && pp_ < topk) {
      sS[(1 + grp) * topk + pp_] = B;
      if (B == nb - 1) sCnt[19 + grp] = pp_;
    }
    cs += ts;
    cp += tq;
    __syncthreads();
  }
  if (tid == 0) sCnt[16] = cs;   // both groups go by group 0's count
  __syncthreads();
  const int ns = min(__builtin_amdgcn_readfirstlane(sCnt[16]), topk);
  const int Tsh = cbase + ns;   // shared tiles: summaries, context blocks, common video blocks
  const int pb = Tsh & 1;

  // step of this group's last block nb - 1 (its padded keys get -inf), or -1
  const int tlast = __builtin_amdgcn_readfirstlane(
      (sCnt[18] >= 0) ? cbase + sCnt[18] : ((sCnt[19 + grp] >= 0) ? Tsh + sCnt[19 + grp] : -1));
  // step of the last context block and its valid rows (context tokens are
  // exact for every video query, outside the top-k budget)
  const int tctx = (nbc > 0) ? cbase - 1 : -1;
  const int validc = (N - Nv) - (nbc - 1) * BK;
  // buffer (0/1) of step t of group g; K at smem + buf * TB, V^T at smem + (2 + buf) * TB
  auto buf_of = [&](int g, int t) -> int { return (t < Tsh) ? (t & 1) : (pb ^ g); };

  // ---- slot table: the K tile and the V^T tile each slot loads, as the
  // tile's address with its buffer (0/1) in bit 48; 0 if none.  Built once,
  // so the loop needs no tile bookkeeping.
  const int nslots = 2 * ntiles + 2;
  {
    // address of the K (v = 0) or V^T (v = 1) tile of step t of group g
    auto step_src = [&](int g, int t, int v) -> uint64_t {
      const int sh = v ? 15 : (FP8 ? 14 : 15);   // log2 of the tile bytes
      if (t < nct) return (uint64_t)((v ? vsb_h : ksb_h) + ((long)t << sh));
      if (t < cbase) return (uint64_t)((v ? vb_h : kb_h) + ((long)(nb + t - nct) << sh));
      const int o = (t < Tsh) ? t - cbase : (g + 1) * topk + t - Tsh;
      return (uint64_t)((v ? vb_h : kb_h) + ((long)sS[o] << sh));
    };
    for (int sl = tid; sl < nslots; sl += PAIR_NT) {
      uint64_t rk = 0, rv = 0;
      if ((sl & 1) == 0) {
        const int ta = (sl >> 1) + 1;   // shared K(ta)
        const int td = sl >> 1;         // group 1's own K(td)
        const int tf = (sl >> 1) - 1;   // group 1's own V(tf)
        if (ta < Tsh && ta < ntiles) rk = ((uint64_t)(ta & 1) << 48) | step_src(0, ta, 0);
        else if (td >= Tsh && td < ntiles) rk = ((uint64_t)(pb ^ 1) << 48) | step_src(1, td, 0);
        if (tf >= Tsh && tf >= 0 && tf < ntiles) rv = ((uint64_t)(pb ^ 1) << 48) | step_src(1, tf, 1);
      } else {
        const int tb = (sl - 1) >> 1;   // shared V(tb), or group 0's own V(tb)
        const int tc = (sl + 1) >> 1;   // group 0's own K(tc)
        if (tb < ntiles) rv = ((uint64_t)buf_of(0, tb) << 48) | step_src(0, tb, 1);
        if (tc >= Tsh && tc < ntiles) rk = ((uint64_t)pb << 48) | step_src(0, tc, 0);
      }
      sSlot[2 * sl] = rk;
      sSlot[2 * sl + 1] = rv;
    }
    if constexpr (FP8) {
      sKsc = reinterpret_cast<float*>(sSlot + 2 * nslots);
      for (int i = tid; i < 2 * ntiles; i += PAIR_NT) {
        const int g = i / ntiles, t = i - g * ntiles;
        float sc;
        if (t < nct) {
          sc = ksscale[(long)h * (nbp / BK) + t];
        } else {
          const int B = (t < cbase) ? nb + t - nct : sS[(t < Tsh) ? t - cbase : (g + 1) * topk + t - Tsh];
          sc = kscale[(long)h * nbt + B];
        }
        sKsc[i] = sc;
      }
    }
  }
  // step 0's K of group 0 (shared, or its own when nothing is shared)
  const char* k0src = (nct > 0) ? ksb_h
                      : kb_h + ((long)((nbc > 0) ? nb : sS[(Tsh > 0) ? 0 : topk]) << (FP8 ? 14 : 15));
  __syncthreads();

  // the tiles loaded in slot s, from the slot table
  auto plan_loads = [&](int s) {
    const uint64_t rk = sSlot[2 * s], rv = sSlot[2 * s + 1];
    const uint32_t klo = __builtin_amdgcn_readfirstlane((uint32_t)rk);
    const uint32_t khi = __builtin_amdgcn_readfirstlane((uint32_t)(rk >> 32));
    const uint32_t vlo = __builtin_amdgcn_readfirstlane((uint32_t)rv);
    const uint32_t vhi = __builtin_amdgcn_readfirstlane((uint32_t)(rv >> 32));
    SlotLoads L;
    L.hk = (klo | khi) != 0;
    L.hv = (vlo | vhi) != 0;
    L.dk = (khi >> 16) & 1;
    L.dv = (vhi >> 16) & 1;
    L.rsk = mk_rsrc(reinterpret_cast<const char*>(((uint64_t)(khi & 0xffffu) << 32) | klo));
    L.rsv = mk_rsrc(reinterpret_cast<const char*>(((uint64_t)(vhi & 0xffffu) << 32) | vlo));
    return L;
  };
  if (nct == 0) issue_k0(k0src);   // step 0 is an exact block: known only now
  f32x16 sacc[4];
  bf16x8 pop[8];
  // every slot starts when all its tiles have landed and every wave is done
  // with the previous slot's LDS reads
  auto slot_begin = [&](int s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    d128_barrier();
    return plan_loads(s);
  };
  auto issue_all = [&](const SlotLoads& L) {
#pragma unroll
    for (int l = 0; l < 16; ++l) issue_load(L, l);
  };
  // matrix slot of step t: P V of step t - 1 (PV), then S^T of step t (QK)
  auto matrix_slot = [&](auto pv_tag, auto qk_tag, int t, const SlotLoads&) {
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
    __builtin_amdgcn_s_setprio(2);
    if constexpr (PV && QK && !FP8) {
      // P V(t-1) then S^T(t) as one stream of 16 k-steps with one operand
      // pipeline: the first K operands are read under the last P V MFMAs
      const unsigned char* sV = smem + (2 + buf_of(grp, t - 1)) * PAIR_TB;
      const unsigned char* sK = smem + buf_of(grp, t) * PAIR_TB;
      auto opnd = [&](int i, int x) {
        return *reinterpret_cast<const bf16x8*>(((i < 8) ? sV : sK) + ro[i & 7] + x * 8192);
      };
      bf16x8 op[16][4];
#pragma unroll
      for (int i = 0; i < D128_PF; ++i)
#pragma unroll
        for (int x = 0; x < 4; ++x) op[i][x] = opnd(i, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + D128_PF < 16) {
#pragma unroll
          for (int x = 0; x < 4; ++x) op[i + D128_PF][x] = opnd(i + D128_PF, x);
        }
        if (i < 8) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i][dt], pop[i], oacc[dt], 0, 0, 0);
        } else {
          if (i == 8) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
              for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
          }
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i][jt], qop[i - 8], sacc[jt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    if constexpr (PV && QK && FP8) {
      // P V(t-1), then S^T(t) on fp8 operands; the first half of the K reads
      // is issued under the last P V step's MFMAs
      const unsigned char* sV = smem + (2 + buf_of(grp, t - 1)) * PAIR_TB;
      const unsigned char* sK = smem + buf_of(grp, t) * PAIR_TB;
      bf16x8 vop[BK / 16][4];
      i32x8 kop8[2][4];
      auto read_k8 = [&](int s2) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const uint4 lo = *reinterpret_cast<const uint4*>(sK + ro8[s2][0] + jt * 4096);
          const uint4 hi = *reinterpret_cast<const uint4*>(sK + ro8[s2][1] + jt * 4096);
          kop8[s2][jt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      };
#pragma unroll
      for (int k = 0; k < D128_PF; ++k)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vop[k][dt] = *reinterpret_cast<const bf16x8*>(sV + ro[k] + dt * 8192);
#pragma unroll
      for (int k = 0; k < BK / 16; ++k) {
        if (k + D128_PF < BK / 16) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            vop[k + D128_PF][dt] = *reinterpret_cast<const bf16x8*>(sV + ro[k + D128_PF] + dt * 8192);
        }
        if (k == BK / 16 - 1) read_k8(0);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k][dt], pop[k], oacc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
      read_k8(1);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          sacc[jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop8[s2][jt], q8[s2], sacc[jt], 0, 0, 0,
                                                                     0, 0, 0);
      // each MFMA of the first half followed by two reads of the second
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    if constexpr (PV) {
      const unsigned char* sV = smem + (2 + buf_of(grp, t - 1)) * PAIR_TB;
      bf16x8 vop[BK / 16][4];
#pragma unroll
      for (int k = 0; k < D128_PF; ++k)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vop[k][dt] = *reinterpret_cast<const bf16x8*>(sV + ro[k] + dt * 8192);
#pragma unroll
      for (int k = 0; k < BK / 16; ++k) {
        if (k + D128_PF < BK / 16) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            vop[k + D128_PF][dt] = *reinterpret_cast<const bf16x8*>(sV + ro[k + D128_PF] + dt * 8192);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k][dt], pop[k], oacc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (QK && FP8) {
      const unsigned char* sK = smem + buf_of(grp, t) * PAIR_TB;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
      i32x8 kop8[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const uint4 lo = *reinterpret_cast<const uint4*>(sK + ro8[s2][0] + jt * 4096);
          const uint4 hi = *reinterpret_cast<const uint4*>(sK + ro8[s2][1] + jt * 4096);
          kop8[s2][jt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          sacc[jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop8[s2][jt], q8[s2], sacc[jt], 0, 0, 0,
                                                                     0, 0, 0);
      d128_pipeline_fp8();
    } else if constexpr (QK) {
      const unsigned char* sK = smem + buf_of(grp, t) * PAIR_TB;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[jt][v] = 0.f;
      bf16x8 kop[D / 16][4];
#pragma unroll
      for (int k = 0; k < D128_PF; ++k)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) kop[k][jt] = *reinterpret_cast<const bf16x8*>(sK + ro[k] + jt * 8192);
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        if (k + D128_PF < D / 16) {
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            kop[k + D128_PF][jt] = *reinterpret_cast<const bf16x8*>(sK + ro[k + D128_PF] + jt * 8192);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[k][jt], qop[k], sacc[jt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // keys past the end of the last block get -inf logits (in the matrix
  // slot, where P is dead); the valid row count is opaque to the compiler so
  // that the compares stay in this rarely taken branch
  auto mask_tail = [&](int t) {
    if (t == tlast || (t == tctx && validc < BK)) {
      int valid;
      asm volatile("s_mov_b32 %0, %1" : "=s"(valid) : "s"((t == tlast) ? Nv - (nb - 1) * BK : validc));
      const int vb = valid - 8 * hf;   // key j = 8 hf + c, c a constant per element
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * jt + ((v < 8) ? v : 8 + v);
          if (c >= vb) sacc[jt][v] = -INFINITY;
        }
    }
  };
  // softmax slot of step t, against the lazy reference m_ref (as in
  // attn_mfma_d128: no per-tile maximum unless a row half's sum exceeds 2^12).
  // Exact tiles hold raw logits (the scale goes into the exp argument),
  // compressed tiles scaled and biased ones.
  auto softmax_slot = [&](auto exact_tag, int t, const SlotLoads& L) {
    constexpr bool EXACT = decltype(exact_tag)::value;
    // logit -> log2 units (fp8: times the query's and the key tile's scales)
    float lsc = scale_log2;
    if constexpr (FP8) lsc = scale_log2 * qscale * sKsc[grp * ntiles + t];
    if constexpr (!EXACT) {
      // element v of 32-key group jt is key 32 jt + 8 hf + v (v < 8) or
      // 32 jt + 16 + 8 hf + v - 8: four runs of 8 consecutive biases
      const float* bb = sBias + t * BK + 8 * hf;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        float4 b4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) b4[u] = *reinterpret_cast<const float4*>(bb + 32 * jt + 16 * (u >> 1) + 4 * (u & 1));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float4 q4 = b4[v >> 2];
          const float bv = ((v & 3) == 0) ? q4.x : ((v & 3) == 1) ? q4.y : ((v & 3) == 2) ? q4.z : q4.w;
          sacc[jt][v] = fmaf(sacc[jt][v], lsc, bv);
        }
      }
    }
    const float sc = EXACT ? lsc : 1.f;
    // the row sums add the fp32 p with plain adds: v_dot2c shares the matrix
    // core's issue and stalls behind the other wave's MFMA stream
    float psum;
    {
      const float nm = -m_ref;
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[jt][8 * hh + e], sc, nm));
            pop[2 * jt + hh][e] = (__bf16)pv;
            ps[e & 1] += pv;
          }
          if constexpr (EXACT) {
            // The slot's 16 loads go out 4 per group over the first half of
            // the exps: late enough that the wave does not stall on a burst
            // before its first exp, early enough that the last ones land
            // before the slot ends (2 per group, to the end, is slower).  The
            // empty asm takes this group's P and sums ahead of its loads;
            // without it the compiler sinks every exp below the last
            // (conditional) load block, so all 16 loads go out first.
            asm volatile("" : "+v"(pop[2 * jt + hh]), "+v"(ps[0]), "+v"(ps[1]));
            if (2 * jt + hh < 4) {
#pragma unroll
              for (int u = 0; u < 4; ++u) issue_load(L, 4 * (2 * jt + hh) + u);
            }
          } else {
            issue_load(L, 2 * (2 * jt + hh));
            issue_load(L, 2 * (2 * jt + hh) + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      psum = ps[0] + ps[1];
    }
    if (__builtin_amdgcn_ballot_w64(!(psum <= 4096.f)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[jt][v]);
      if (EXACT) mx *= sc;
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
      const float nm = -m_ref;
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[jt][8 * hh + e], sc, nm));
            pop[2 * jt + hh][e] = (__bf16)pv;
            ps[e & 1] += pv;
          }
      psum = ps[0] + ps[1];
    }
    l_run += psum;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // group g runs matrix(t) in slot 2t + g and softmax(t) in slot 2t + 1 + g;
  // group 1 starts with an empty slot 0, group 0 ends with an empty slot
  // 2 ntiles + 1, so both pass the same 2 ntiles + 2 barriers.  Step 0 and
  // the last matrix slot are peeled, and the compressed and exact steps run
  // in loops of their own, so the steady loops carry no step tests.
  if (grp == 1) issue_all(slot_begin(0));
  matrix_slot(F_{}, T_{}, 0, slot_begin(grp));
  if (nct > 0) {
    softmax_slot(F_{}, 0, slot_begin(1 + grp));
  } else {
    mask_tail(0);
    softmax_slot(T_{}, 0, slot_begin(1 + grp));
  }
  for (int t = 1; t < nct; ++t) {
    matrix_slot(T_{}, T_{}, t, slot_begin(2 * t + grp));
    softmax_slot(F_{}, t, slot_begin(2 * t + 1 + grp));
  }
  for (int t = max(nct, 1); t < ntiles; ++t) {
    matrix_slot(T_{}, T_{}, t, slot_begin(2 * t + grp));
    mask_tail(t);
    softmax_slot(T_{}, t, slot_begin(2 * t + 1 + grp));
  }
  matrix_slot(T_{}, F_{}, ntiles, slot_begin(2 * ntiles + grp));
  if (grp == 0) issue_all(slot_begin(2 * ntiles + 1));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (idle) return;

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  const long pos = out_pos(A, wave * 32 + l32, nb, N, Nv, BK);
  uint16_t* dst;
  if (perm_q != nullptr) {
    if (pos < 0) return;
    dst = out + ((long)h * N + perm_q[(long)h * N + pos]) * D;
  } else {
    dst = out + ((long)h * Np + (long)A * BK + wave * 32 + l32) * D;
  }
  const bool pad = pos < 0;
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
// Generic VALU kernel: one thread per query row of the block.
// ---------------------------------------------------------------------------
constexpr int GEN_CH = 32;  // keys per staged chunk

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_generic(
    const T* __restrict__ qp, const T* __restrict__ kp, const T* __restrict__ vpt,
    const int32_t* __restrict__ idx, int topk, const float* __restrict__ ksum,
    const float* __restrict__ vsum, const float* __restrict__ bias,
    const int32_t* __restrict__ perm_q, T* __restrict__ out, int H, int N, int Nv, int BK, int nb,
    int nbc, float scale) {
  __shared__ float sK[GEN_CH][D];
  __shared__ float sV[GEN_CH][D];
  __shared__ float sB[GEN_CH];
  extern __shared__ unsigned char smask[];  // nb bytes: 1 = selected

  const int tid = threadIdx.x;
  const int nbt = nb + nbc;
  const int h = blockIdx.x / nbt, Ar = blockIdx.x % nbt;
  const int A = (Ar < nbc) ? nb + Ar : Ar - nbc;   // context query blocks first
  const long Np = (long)nbt * BK;
  const TilePlan tp = tile_plan(A, nb, nbc, topk, 1);
  const int32_t* myidx = (A < nb) ? idx + ((long)h * nb + A) * topk : idx;
  for (int i = tid; i < nb; i += blockDim.x) smask[i] = 0;
  __syncthreads();
  for (int t = tid; t < tp.nidx; t += blockDim.x) smask[myidx[t]] = 1;
  __syncthreads();

  const long qrow = (long)A * BK + tid;   // row in the padded layout of q_p
  const bool active = tid < BK;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = active ? Elem<T>::load(qp + ((long)h * Np + qrow) * D + c) : 0.f;
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

  // exact branch: selected blocks, then the context blocks (video query
  // blocks); every block (context query blocks)
  for (int t = 0; t < tp.nex; ++t) {
    const int B = (t < tp.nidx) ? myidx[t] : t + tp.bofs;
    const int valid = block_rows(B, nb, nbt, N, Nv, BK);
    for (int j0 = 0; j0 < valid; j0 += GEN_CH) {
      const int cnt = min(GEN_CH, valid - j0);
      __syncthreads();
      for (int e = tid; e < GEN_CH * D; e += blockDim.x) {
        const int j = e / D, c = e % D;
        float kv = 0.f, vv = 0.f;
        if (j < cnt) {
          kv = Elem<T>::load(kp + ((long)h * Np + (long)B * BK + j0 + j) * D + c);
          vv = Elem<T>::load(vpt + (((long)h * nbt + B) * D + c) * BK + j0 + j);
        }
        sK[j][c] = kv;
        sV[j][c] = vv;
      }
      for (int j = tid; j < GEN_CH; j += blockDim.x) sB[j] = 0.f;
      __syncthreads();
      consume(cnt);
    }
  }
  // compressed branch: every unselected video block, weight |B| through
  // log|B| (none for a context query block)
  for (int B0 = 0; B0 < (A < nb ? nb : 0); B0 += GEN_CH) {
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
        const int nB = (B == nb - 1) ? (Nv - (nb - 1) * BK) : BK;
        bb = bias[(long)h * nb + B] + logf((float)nB);
      }
      sB[j] = bb;
    }
    __syncthreads();
    consume(cnt);
  }

  if (!active) return;
  const float inv = 1.f / l_run;
  const long pos = out_pos(A, tid, nb, N, Nv, BK);
  T* dst;
  if (perm_q != nullptr) {
    if (pos < 0) return;
    dst = out + ((long)h * N + ((A < nb) ? perm_q[(long)h * N + pos] : pos)) * D;
  } else {
    dst = out + ((long)h * Np + qrow) * D;
  }
  const bool pad = pos < 0;
#pragma unroll
  for (int c = 0; c < D; ++c) Elem<T>::store(dst + c, pad ? 0.f : o[c] * inv);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Workspace of attn_launch: the bf16 summary tiles, and in fp8 mode the E4M3
// key tiles (all nbt blocks) and summary tiles with their scales.
struct AttnWs {
  size_t ks16, vs16t, bias2, k8, kscale, ks8, ksscale, total;
};
static AttnWs attn_ws_plan(int H, int N, int Nv, int D, int BK, bool fp8) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int nb = cdiv(Nv, BK), nbt = nb + cdiv(N - Nv, BK);
  const int nbp = cdiv(nb, BK) * BK;
  AttnWs w;
  size_t o = 0;
  w.ks16 = o;    o += up((size_t)H * nbp * D * 2);
  w.vs16t = o;   o += up((size_t)H * nbp * D * 2);
  w.bias2 = o;   o += up((size_t)H * nbp * 4);
  w.k8 = o;      o += fp8 ? up((size_t)H * nbt * BK * D) : 0;
  w.kscale = o;  o += fp8 ? up((size_t)H * nbt * 4) : 0;
  w.ks8 = o;     o += fp8 ? up((size_t)H * nbp * D) : 0;
  w.ksscale = o; o += fp8 ? up((size_t)H * (nbp / BK) * 4) : 0;
  w.total = o;
  return w;
}

// Nv video tokens of N (Nv = N without context tokens).
size_t attn_ws_bytes(int H, int N, int Nv, int D, int BK, int dtype, bool fp8) {
  if (dtype != SPARK_BF16 || (BK != 32 && BK != 64 && BK != 128)) return 0;
  return attn_ws_plan(H, N, Nv, D, BK, fp8).total;
}

bool attn_fp8_supported(int H, int N, int Nv, int D, int BK, int dtype) {
  const int nb = cdiv(Nv, BK), nbp = cdiv(nb, BK) * BK;
  return dtype == SPARK_BF16 && D == 128 && BK == 128 &&
         (size_t)D128_LDS_TILES + (size_t)nbp * 4 <= 80 * 1024;
}

bool attn_uses_mfma(int dtype, int BK) {
  return dtype == SPARK_BF16 && (BK == 32 || BK == 64 || BK == 128);
}

template <int D, int BK>
static int launch_mfma(const void* qp, const void* kp, const void* vpt, const int32_t* idx,
                       int topk, const uint16_t* ks16, const uint16_t* vs16t, const float* bias2,
                       const int32_t* perm_q, void* out, int H, int N, int Nv, int nb, int nbc,
                       int nbp, hipStream_t st) {
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
  hipLaunchKernelGGL((attn_mfma<D, BK>), dim3(H * (nb + nbc)), dim3(C::NT), lds, st,
                     (const uint16_t*)qp, (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk,
                     ks16, vs16t, bias2, perm_q, (uint16_t*)out, H, N, Nv, nb, nbc, nbp, scale_log2);
  return spark_check_launch("attn_mfma");
}

// kp / ks16: bf16 tiles, or (fp8) E4M3 tiles with their scales kscale / ksscale
static int launch_d128(const void* qp, const void* kp, const void* vpt, const int32_t* idx, int topk,
                     const uint16_t* ks16, const uint16_t* vs16t, const float* bias2,
                     const int32_t* perm_q, void* out, int H, int N, int Nv, int nb, int nbc,
                     int nbp, bool fp8, bool paired, const float* kscale, const float* ksscale, hipStream_t st) {
  const size_t lds = D128_LDS_TILES + (size_t)nbp * 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma_d128<false, false>, hipFuncAttributeMaxDynamicSharedMemorySize, 80 * 1024);
    hipFuncSetAttribute((const void*)attn_mfma_d128<true, false>, hipFuncAttributeMaxDynamicSharedMemorySize, 80 * 1024);
    hipFuncSetAttribute((const void*)attn_mfma_d128<false, true>, hipFuncAttributeMaxDynamicSharedMemorySize, 80 * 1024);
    hipFuncSetAttribute((const void*)attn_mfma_d128<true, true>, hipFuncAttributeMaxDynamicSharedMemorySize, 80 * 1024);
    attr_set = true;
  }
  const float scale_log2 = kLog2e / sqrtf(128.f);
  if (paired && pair_lds_bytes(nb, nbc, nbp, topk, fp8) <= 160 * 1024) {
    static bool pair_attr_set = false;
    if (!pair_attr_set) {
      hipFuncSetAttribute((const void*)attn_pair_d128<false>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      hipFuncSetAttribute((const void*)attn_pair_d128<true>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      pair_attr_set = true;
    }
    const long pslots = 8L * (((nb + 1) / 2 + 7) / 8);
    if ((long)H * pslots > 0x7fffffffL) return spark_set_error(SPARK_E_SHAPE, "spark_attn: grid too large");
    const size_t plds = pair_lds_bytes(nb, nbc, nbp, topk, fp8);
    const dim3 pgrid((unsigned)(H * pslots)), pblock(PAIR_NT);
#define SPARK_PAIR_LAUNCH(F)                                                                       \
    hipLaunchKernelGGL((attn_pair_d128<F>), pgrid, pblock, plds, st, (const uint16_t*)qp, (const uint16_t*)kp, \
                       (const uint16_t*)vpt, idx, topk, ks16, vs16t, bias2, perm_q, (uint16_t*)out, H, N, Nv, nb, \
                       nbc, nbp, scale_log2, kscale, ksscale)
    if (fp8) SPARK_PAIR_LAUNCH(true);
    else SPARK_PAIR_LAUNCH(false);
#undef SPARK_PAIR_LAUNCH
    int rc = spark_check_launch("attn_pair_d128");
    if (rc || nbc == 0) return rc;
    // the context query blocks (dense rows over all n_b + n_c tiles)
    const long cslots = 8L * ((nbc + 7) >> 3);
    if (fp8)
      hipLaunchKernelGGL((attn_mfma_d128<true, true>), dim3((unsigned)(H * cslots)), dim3(D128_NT), lds, st,
                         (const uint16_t*)qp, (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk, ks16, vs16t,
                         bias2, perm_q, (uint16_t*)out, H, N, Nv, nb, nbc, nbp, scale_log2, kscale, ksscale, 1);
    else
      hipLaunchKernelGGL((attn_mfma_d128<true, false>), dim3((unsigned)(H * cslots)), dim3(D128_NT), lds, st,
                         (const uint16_t*)qp, (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk, ks16, vs16t,
                         bias2, perm_q, (uint16_t*)out, H, N, Nv, nb, nbc, nbp, scale_log2, kscale, ksscale, 1);
    return spark_check_launch("attn_mfma_d128 (context blocks)");
  }
  const long slots = 8L * (((nbc + 7) >> 3) + ((nb + 7) >> 3));   // d128_slots
  if ((long)H * slots > 0x7fffffffL) return spark_set_error(SPARK_E_SHAPE, "spark_attn: grid too large");
  const dim3 grid((unsigned)(H * slots)), block(D128_NT);
#define SPARK_D128_LAUNCH(C, F)                                                                    \
  hipLaunchKernelGGL((attn_mfma_d128<C, F>), grid, block, lds, st, (const uint16_t*)qp,             \
                     (const uint16_t*)kp, (const uint16_t*)vpt, idx, topk, ks16, vs16t, bias2, perm_q, \
                     (uint16_t*)out, H, N, Nv, nb, nbc, nbp, scale_log2, kscale, ksscale, 0)
  if (nbc > 0) {
    if (fp8) SPARK_D128_LAUNCH(true, true);
    else SPARK_D128_LAUNCH(true, false);
  } else {
    if (fp8) SPARK_D128_LAUNCH(false, true);
    else SPARK_D128_LAUNCH(false, false);
  }
#undef SPARK_D128_LAUNCH
  return spark_check_launch("attn_mfma_d128");
}

template <typename T, int D>
static int launch_generic(const void* qp, const void* kp, const void* vpt, const int32_t* idx,
                          int topk, const float* ksum, const float* vsum, const float* bias,
                          const int32_t* perm_q, void* out, int H, int N, int Nv, int BK, int nb,
                          int nbc, hipStream_t st) {
  if (nb > 64 * 1024)
    return spark_set_error(SPARK_E_SHAPE, "spark_attn: too many blocks (%d) for the generic kernel", nb);
  const float scale = 1.f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_generic<T, D>), dim3(H * (nb + nbc)), dim3(128), (size_t)nb, st,
                     (const T*)qp, (const T*)kp, (const T*)vpt, idx, topk, ksum, vsum, bias,
                     perm_q, (T*)out, H, N, Nv, BK, nb, nbc, scale);
  return spark_check_launch("attn_generic");
}

int quant_e4m3_launch(int H, long in_rows, long out_rows, int D, int G, int dtype, const void* x,
                      uint8_t* x8, float* scales, hipStream_t st);

// Nv = N: the plain layer; Nv < N: tokens [Nv, N) are context tokens.  fp8:
// E4M3 logits (the caller has checked attn_fp8_supported).  paired: the bf16
// d = 128 / block 128 layer may run two query blocks per workgroup.
int attn_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* qp, const void* kp,
                const void* vpt, const int32_t* idx, int topk, const float* ksum,
                const float* vsum, const float* bias, const int32_t* perm_q, void* out, void* ws,
                bool fp8, bool paired, hipStream_t st) {
  const int nb = cdiv(Nv, BK), nbc = cdiv(N - Nv, BK);
  if (attn_uses_mfma(dtype, BK)) {
    const int nbp = cdiv(nb, BK) * BK;
    const AttnWs w = attn_ws_plan(H, N, Nv, D, BK, fp8);
    char* wb = (char*)ws;
    uint16_t* ks16 = (uint16_t*)(wb + w.ks16);
    uint16_t* vs16t = (uint16_t*)(wb + w.vs16t);
    float* bias2 = (float*)(wb + w.bias2);
    const long total = (long)H * nbp * D;
    const int grid = (int)std::min<long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(attn_prep_summaries, dim3(grid), dim3(256), 0, st, ksum, vsum, bias, ks16,
                       vs16t, bias2, H, Nv, D, BK, nb, nbp);
    int rc = spark_check_launch("attn_prep_summaries");
    if (rc) return rc;
    if (fp8) {
      uint8_t* k8 = (uint8_t*)(wb + w.k8);
      uint8_t* ks8 = (uint8_t*)(wb + w.ks8);
      float* kscale = (float*)(wb + w.kscale);
      float* ksscale = (float*)(wb + w.ksscale);
      const long rows = (long)(nb + nbc) * BK;
      rc = quant_e4m3_launch(H, rows, rows, D, BK, SPARK_BF16, kp, k8, kscale, st);
      if (rc) return rc;
      rc = quant_e4m3_launch(H, nb, nbp, D, BK, SPARK_F32, ksum, ks8, ksscale, st);
      if (rc) return rc;
      return launch_d128(qp, k8, vpt, idx, topk, (const uint16_t*)ks8, vs16t, bias2, perm_q, out, H, N, Nv,
                         nb, nbc, nbp, true, paired, kscale, ksscale, st);
    }
    if (D == 128) {
      if (BK == 128 && (size_t)D128_LDS_TILES + (size_t)nbp * 4 <= 80 * 1024)
        return launch_d128(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp,
                           false, paired, nullptr, nullptr, st);
      if (BK == 128) return launch_mfma<128, 128>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
      if (BK == 64) return launch_mfma<128, 64>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
      return launch_mfma<128, 32>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
    } else {
      if (BK == 128) return launch_mfma<64, 128>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
      if (BK == 64) return launch_mfma<64, 64>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
      return launch_mfma<64, 32>(qp, kp, vpt, idx, topk, ks16, vs16t, bias2, perm_q, out, H, N, Nv, nb, nbc, nbp, st);
    }
  }
  if (dtype == SPARK_F32) {
    if (D == 128) return launch_generic<float, 128>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, Nv, BK, nb, nbc, st);
    return launch_generic<float, 64>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, Nv, BK, nb, nbc, st);
  }
  if (D == 128) return launch_generic<uint16_t, 128>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, Nv, BK, nb, nbc, st);
  return launch_generic<uint16_t, 64>(qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, H, N, Nv, BK, nb, nbc, st);
}

}  // namespace spark
