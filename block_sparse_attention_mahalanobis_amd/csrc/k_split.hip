// Spark-Reblock's iterative hierarchical partitioner ("Spark-H3" blog,
// 01 / Method: Spark-Reblock: starting from the full token set, every group
// is split level by level according to the distance while enforcing the
// assigned child capacities, until every leaf holds one block; token IDs
// track membership through the tree).
//
// Rule implemented (two-pole capacity bisection), per group g with nb_g >= 2
// blocks:  left capacity c_L = ceil(nb_g / 2) * block;  centroid c = sum x^_i;
// pole A = argmin (x^_i . c, id);  pole B = argmin (x^_i . x^_A, id);
// s_i = x^_i . x^_A - x^_i . x^_B;  left child = the c_L members first in
// (s descending, id ascending) order (NaN last), right child = the rest, both
// keeping ascending ids.  Leaves end up in depth-first left-first order.
//
// Every tree (head x side) has the same shape, which depends only on
// (N, block), so a group is found from a block index (or a slot number = its
// left/right path) by walking down from the root; no tables are needed.
//
// Large groups (global levels) use level-synchronous passes over all trees:
//   cent_partial  -> per-block partial centroid sums (rows gathered by id;
//                    below the root only the left children's blocks)
//   cent_reduce   -> per-group centroid sum in fp64 (fixed chunk order:
//                    deterministic); a right child's is parent - left
//   argmin_partial/argmin_reduce (twice: pole A, pole B; 64-bit (key, id) mins)
//   groups of more than 64 blocks:
//     score       -> s_i for every position, to memory
//     capacity select: the exact c_L-th key by radix_hist /
//                 radix_pick_groups rounds over many workgroups, then
//                 seg_count / seg_partition, one workgroup per 8192
//                 positions (a stable partition of the ids)
//   groups of at most 64 blocks: score_select_small, one workgroup per
//     group: scores into LDS, the same radix select and stable partition
//     there, and the next level's centroid sums (that level then skips
//     cent_partial / cent_reduce).
// The capacity select is exact: the c_L-th key and how many of its ties go
// left, so every form gives the same permutation.
// Once every group fits in LDS (<= FIN_MAX tokens) one workgroup per group
// loads its rows once and finishes all remaining levels in LDS.
#include "common.hpp"

namespace spark {

constexpr int SPL_T = 256;
constexpr int FIN_MAX = 1024;         // tokens per finisher group
constexpr int FIN_LDS = 136 * 1024;   // bytes of rows in the finisher

// ---- tree navigation --------------------------------------------------------
// Group containing block cb at `level`; false if that block is already in a
// leaf (a group of one block) at an earlier level.  slot = path bits.
__device__ __forceinline__ bool group_of_block(int cb, int level, int nb, int& start, int& nbg,
                                               int& slot) {
  start = 0;
  nbg = nb;
  slot = 0;
  for (int l = 0; l < level; ++l) {
    if (nbg <= 1) return false;
    const int nl = (nbg + 1) >> 1;
    if (cb < start + nl) {
      nbg = nl;
      slot = slot << 1;
    } else {
      start += nl;
      nbg -= nl;
      slot = (slot << 1) | 1;
    }
  }
  return nbg >= 2;
}

__device__ __forceinline__ bool group_of_slot(int slot, int level, int nb, int& start, int& nbg) {
  start = 0;
  nbg = nb;
  for (int l = level - 1; l >= 0; --l) {
    if (nbg <= 1) return false;
    const int nl = (nbg + 1) >> 1;
    if ((slot >> l) & 1) {
      start += nl;
      nbg -= nl;
    } else {
      nbg = nl;
    }
  }
  return true;
}

__device__ __forceinline__ uint32_t pref_key_desc(float s) {
  if (s != s) return 0xffffffffu;
  return ~float_key_asc(s);
}

__device__ __forceinline__ uint64_t argmin_key(float v, int id) {
  return ((uint64_t)float_key_asc(v) << 32) | (uint32_t)id;
}

// ---- global-level passes ----------------------------------------------------
// ids[t][from + i] = from + i for i < n, rows of ld entries; trees
// t >= split_at go to hi (offset by split_at trees).
__global__ void iota_kernel(int32_t* __restrict__ lo, int32_t* __restrict__ hi, int split_at,
                            int n, long ld, int from, long total) {
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total;
       e += (long)gridDim.x * blockDim.x) {
    const long t = e / n;
    const int i = from + (int)(e % n);
    int32_t* row = (t < split_at) ? lo + t * ld : hi + (t - split_at) * ld;
    row[i] = i;
  }
}

// Rows of one block (chunk) of the current order, gathered by id: every lane
// loads its NIT row chunks up front (ids staged in LDS first), so all the
// row reads of the block are in flight together.  The chunks stay as loaded
// (16 bytes: 8 bf16 or 4 fp32) and are widened to fp32 where they are used,
// which halves the registers a bf16 pass holds and lets 8 waves per SIMD
// keep their reads in flight.
template <typename T, int D>
struct ChunkRows {
  static constexpr int VE = Chunk<T>::VE, CPR = D / VE, RPP = SPL_T / CPR, NIT = 128 / RPP;
  uint4 raw[NIT];
  __device__ __forceinline__ void load(const T* __restrict__ xt, const int32_t* s_ids, int n_real,
                                       int rg, int c) {
    load_rows(xt, s_ids, n_real, rg, RPP, c);
  }
  // chunk `it` holds row j0 + it * step
  __device__ __forceinline__ void load_rows(const T* __restrict__ xt, const int32_t* s_ids, int n_real,
                                            int j0, int step, int c) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = j0 + it * step;
      raw[it] = (j < n_real) ? *reinterpret_cast<const uint4*>(xt + (long)s_ids[j] * D + c)
                             : uint4{0u, 0u, 0u, 0u};
    }
  }
  // chunk `it` as fp32 (absent rows are zero)
  __device__ __forceinline__ void get(int it, float (&v)[VE]) const {
    const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
};

__device__ __forceinline__ void stage_ids(int32_t* s_ids, const int32_t* __restrict__ idr,
                                          int n_real) {
  for (int i = threadIdx.x; i < n_real; i += SPL_T) s_ids[i] = idr[i];
  __syncthreads();
}

// Per block (chunk) of the current order: partial centroid sum.
template <typename T, int D>
__global__ __launch_bounds__(SPL_T) void cent_partial(const T* __restrict__ xh,
                                                      const int32_t* __restrict__ ids,
                                                      float* __restrict__ cpart, int N, int BK,
                                                      int nb, int level) {
  using CR = ChunkRows<T, D>;
  constexpr int VE = CR::VE, CPR = CR::CPR, RPP = CR::RPP;
  __shared__ float s_p[SPL_T / 64][D];
  __shared__ int32_t s_ids[128];
  const int cb = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  int start, nbg, slot;
  if (!group_of_block(cb, level, nb, start, nbg, slot)) return;
  if (level > 0 && (slot & 1)) return;   // a right child: parent - left (cent_reduce)
  const int n_real = min(BK, N - cb * BK);
  // wave w sums rows [32 w, 32 w + 32) of the 128-row block: lane (rl, chunk
  // c) rows 32 w + RGW it + rl (the whitening pass, which holds each wave's
  // 32 rows, reproduces this order for the root)
  constexpr int RGW = 64 / CPR;   // row groups per wave
  const int lane = tid & 63, rl = lane / CPR, c = (tid % CPR) * VE;
  stage_ids(s_ids, ids + (long)t * N + (long)cb * BK, n_real);
  CR rows;
  rows.load_rows(xh + (long)t * N * D, s_ids, n_real, 32 * (tid >> 6) + rl, RGW, c);
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < CR::NIT; ++it) {
    float v[VE];
    rows.get(it, v);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += v[e];
  }
  // lanes holding the same chunk: fold within the wave, then across waves
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = group_sum<64, CPR>(acc[e]);
  if ((tid & 63) < CPR)
#pragma unroll
    for (int e = 0; e < VE; ++e) s_p[tid >> 6][c + e] = acc[e];
  __syncthreads();
  for (int cc = tid; cc < D; cc += SPL_T) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < SPL_T / 64; ++w) sum += s_p[w][cc];
    cpart[((long)t * nb + cb) * D + cc] = sum;
  }
}

// Per group: centroid sum, in fp64.  At the root, the sum of its blocks'
// partials.  Below it, one workgroup per parent: the left child's sum comes
// from its blocks' partials and the right child's is the parent's sum minus
// the left's, which is the same sum in exact arithmetic and saves reading the
// right half's rows; in fp64 the subtraction stays far below fp32 rounding.
// The left child holds ceil(nb_g / 2) blocks, so whenever the right child
// still splits (>= 2 blocks) the left has been summed.  NT threads: column
// c = tid % D, block stride G = NT / D; each thread keeps 8 partial sums
// (8 loads in flight), then the G partials are added in a fixed order
// (deterministic).  The top levels have few groups with thousands of blocks
// (NT = 1024); the deep levels many groups of a few dozen (NT = D).
template <int D, int NT>
__global__ __launch_bounds__(NT) void cent_reduce(const float* __restrict__ cpart,
                                                    const double* __restrict__ cen_up,
                                                    double* __restrict__ cen, int nb, int level,
                                                    int S) {
  constexpr int G = NT / D;
  __shared__ double s_p[G][D];
  const int par = blockIdx.x, t = blockIdx.y;
  const int lslot = level == 0 ? 0 : 2 * par;   // the root, or the parent's left child
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  int start, nbg;
  if (!group_of_slot(lslot, level, nb, start, nbg) || nbg < 2) return;
  const int end = start + nbg;
  const float* src = cpart + (long)t * nb * D + c;
  double a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = 0.0;
  int b = start + g;
  for (; b + 7 * G < end; b += 8 * G) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(long)(b + u * G) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] += (double)v[u];
  }
  for (; b < end; b += G) a[0] += (double)src[(long)b * D];
  s_p[g][c] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (g == 0) {
    double sl = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) sl += s_p[i][c];
    cen[((long)t * S + lslot) * D + c] = sl;
    if (level > 0) {
      int rstart, rnb;
      if (group_of_slot(lslot + 1, level, nb, rstart, rnb) && rnb >= 2)
        cen[((long)t * S + lslot + 1) * D + c] = cen_up[((long)t * S + par) * D + c] - sl;
    }
  }
}

// Per chunk: min over rows of (x^_i . vec_g, id), vec_g = cen[slot] (mode 0)
// or x^[poleA[slot]] (mode 1).
template <typename T, int D>
__global__ __launch_bounds__(SPL_T) void argmin_partial(const T* __restrict__ xh,
                                                        const int32_t* __restrict__ ids,
                                                        const double* __restrict__ cen,
                                                        const int32_t* __restrict__ poleA,
                                                        uint64_t* __restrict__ mpart, int N,
                                                        int BK, int nb, int level, int S,
                                                        int mode) {
  using CR = ChunkRows<T, D>;
  constexpr int VE = CR::VE, CPR = CR::CPR, RPP = CR::RPP;
  __shared__ uint64_t s_min[SPL_T / 64];
  __shared__ int32_t s_ids[128];
  const int cb = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  int start, nbg, slot;
  if (!group_of_block(cb, level, nb, start, nbg, slot)) return;
  const int n_real = min(BK, N - cb * BK);
  const int rg = tid / CPR, c = (tid % CPR) * VE;
  const T* xt = xh + (long)t * N * D;
  float vec[VE];
  if (mode == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) vec[e] = (float)cen[((long)t * S + slot) * D + c + e];
  } else {
    Chunk<T>::load(xt + (long)poleA[(long)t * S + slot] * D + c, vec);
  }
  stage_ids(s_ids, ids + (long)t * N + (long)cb * BK, n_real);
  CR rows;
  rows.load(xt, s_ids, n_real, rg, c);
  uint64_t best = ~0ull;
#pragma unroll
  for (int it = 0; it < CR::NIT; ++it) {
    const int j = it * RPP + rg;
    float v[VE];
    rows.get(it, v);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc = fmaf(v[e], vec[e], acc);
    acc = group_sum<CPR>(acc);
    if (j < n_real) {
      const uint64_t k = argmin_key(acc, s_ids[j]);
      best = k < best ? k : best;
    }
  }
  best = group_min_u64<64>(best);
  if ((tid & 63) == 0) s_min[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = s_min[0];
    for (int w = 1; w < SPL_T / 64; ++w) b = s_min[w] < b ? s_min[w] : b;
    mpart[(long)t * nb + cb] = b;
  }
}

// Per group: min over its chunks' partials -> pole id.  mode 1 also writes
// diff = x^_A - x^_B.
template <typename T, int D>
__global__ __launch_bounds__(64) void argmin_reduce(const uint64_t* __restrict__ mpart,
                                                    const T* __restrict__ xh,
                                                    int32_t* __restrict__ poleA,
                                                    int32_t* __restrict__ poleB,
                                                    float* __restrict__ diff, int N, int nb,
                                                    int level, int S, int mode) {
  const int slot = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg) || nbg < 2) return;
  uint64_t best = ~0ull;
  for (int b = start + lane; b < start + nbg; b += 64) {
    const uint64_t k = mpart[(long)t * nb + b];
    best = k < best ? k : best;
  }
  best = group_min_u64<64>(best);
  const int id = (int)(uint32_t)(best & 0xffffffffu);
  if (mode == 0) {
    if (lane == 0) poleA[(long)t * S + slot] = id;
    return;
  }
  if (lane == 0) poleB[(long)t * S + slot] = id;
  const T* xt = xh + (long)t * N * D;
  const int ia = poleA[(long)t * S + slot];
  for (int c = lane; c < D; c += 64)
    diff[((long)t * S + slot) * D + c] =
        Elem<T>::load(xt + (long)ia * D + c) - Elem<T>::load(xt + (long)id * D + c);
}

// s at every position of groups with >= 2 blocks: x^_i . diff_g
template <typename T, int D>
__global__ __launch_bounds__(SPL_T) void score_kernel(const T* __restrict__ xh,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ diff,
                                                      float* __restrict__ s, int N, int BK,
                                                      int nb, int level, int S) {
  using CR = ChunkRows<T, D>;
  constexpr int VE = CR::VE, CPR = CR::CPR, RPP = CR::RPP;
  __shared__ int32_t s_ids[128];
  const int cb = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  int start, nbg, slot;
  if (!group_of_block(cb, level, nb, start, nbg, slot)) return;
  const int n_real = min(BK, N - cb * BK);
  const int rg = tid / CPR, c = (tid % CPR) * VE;
  float vec[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) vec[e] = diff[((long)t * S + slot) * D + c + e];
  const long pos0 = (long)t * N + (long)cb * BK;
  stage_ids(s_ids, ids + pos0, n_real);
  CR rows;
  rows.load(xh + (long)t * N * D, s_ids, n_real, rg, c);
#pragma unroll
  for (int it = 0; it < CR::NIT; ++it) {
    const int j = it * RPP + rg;
    float v[VE];
    rows.get(it, v);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc = fmaf(v[e], vec[e], acc);
    acc = group_sum<CPR>(acc);
    if (j < n_real && (tid % CPR) == 0) s[pos0 + j] = acc;
  }
}

// ---- workgroup helpers (radix select + stable partition) ---------------------
// Exclusive scan of one int per thread over NT threads; returns the total.
template <int NT = SPL_T>
__device__ __forceinline__ int wg_exscan(int v, int* s_tmp, int& total) {
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
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) base += s_tmp[i];
    tot += s_tmp[i];
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Exclusive scan of one int per thread over FIN_T (512) threads.
__device__ __forceinline__ int fin_exscan(int v, int* s_tmp, int& total) {
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
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < w) base += s_tmp[i];
    tot += s_tmp[i];
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Exclusive scan over the NT threads of one team (waves w0 .. w0 + NT/64 - 1
// of the workgroup; s_tmp is indexed by workgroup wave).  Every thread of the
// workgroup must call it (two barriers).
template <int NT>
__device__ __forceinline__ int team_exscan(int v, int* s_tmp, int w0, int& total) {
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
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (w0 + i < w) base += s_tmp[w0 + i];
    tot += s_tmp[w0 + i];
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// After a histogram round: find the digit where the running count reaches
// *need (wave 0 only), updating *prefix and *need.
__device__ __forceinline__ void radix_pick(const int* s_hist, uint32_t* s_prefix, int* s_need,
                                           int shift) {
  const int lane = threadIdx.x & 63;
  int c[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += s_hist[4 * lane + i];
    c[i] = run;
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const int base = incl - run;
  const int need = *s_need;
  const uint32_t pre = *s_prefix;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int before = base + (i ? c[i - 1] : 0);
    const int after = base + c[i];
    if (before < need && after >= need) {
      *s_prefix = pre | ((uint32_t)(4 * lane + i) << shift);
      *s_need = need - before;
    }
  }
}

// Capacity select of the large groups by many workgroups, four radix rounds
// of two launches each, synchronised by the launch boundaries alone (no
// cross-workgroup fences or atomics, which cost an L2 write-back per
// workgroup on this multi-XCD part).  radix_hist: every workgroup takes
// RG_SEG positions of its group, counts the keys that match the prefix so
// far into per-wave LDS histograms and stores its 256 counts in its own
// slot of hpart.  radix_pick: one workgroup per group adds its segments'
// counts in segment order and picks the digit exactly as the one-workgroup
// form does (hpart is indexed by the level's groups, rec by the deepest
// level's slot count S, as select_partition reads it).  Per (tree, group)
// the record rec[RG_REC] holds the prefix and
// the rank still needed; after the last round it holds the c_L-th key and
// the number of ties that go left, which seg_count / seg_partition take.
constexpr int RG_REC = 2;
constexpr int RG_SEG = 8192;
constexpr int RG_T = 256;

__global__ __launch_bounds__(RG_T) void radix_hist(const float* __restrict__ s, const int* __restrict__ rec,
                                                  int* __restrict__ hpart, int N, int BK, int nb, int level,
                                                  int S, int nseg_max, int shift) {
  constexpr int NH = 4 * (RG_T / 64);   // four histograms per wave, by lane & 3
  __shared__ int s_whist[NH][256];
  const int slot = blockIdx.x / nseg_max, seg = blockIdx.x % nseg_max, t = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, hsel = 4 * wave + (tid & 3);
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg) || nbg < 2) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const int i0 = seg * RG_SEG;
  if (i0 >= n) return;
  const int i1 = min(n, i0 + RG_SEG);
  const uint32_t pre = (shift == 24) ? 0u : (uint32_t)rec[((long)t * S + slot) * RG_REC];
  for (int i = tid; i < NH * 256; i += RG_T) (&s_whist[0][0])[i] = 0;
  __syncthreads();
  const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
  const long base = (long)t * N + g0;
  constexpr int U = 8;
  for (int j0 = i0; j0 < i1; j0 += U * RG_T) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = j0 + u * RG_T + tid;
      v[u] = (i < i1) ? s[base + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = j0 + u * RG_T + tid;
      const uint32_t k = pref_key_desc(v[u]);
      if (i < i1 && (k & hmask) == pre) atomicAdd(&s_whist[hsel][(k >> shift) & 255], 1);
    }
  }
  __syncthreads();
  int* hp = hpart + (((long)t * (1 << level) + slot) * nseg_max + seg) * 256;   // this level's groups
  for (int b = tid; b < 256; b += RG_T) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < NH; ++w) c += s_whist[w][b];
    hp[b] = c;
  }
}

__global__ __launch_bounds__(RG_T) void radix_pick_groups(int* __restrict__ rec, const int* __restrict__ hpart,
                                                         int N, int BK, int nb, int level, int S,
                                                         int nseg_max, int shift) {
  __shared__ int s_hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int slot = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg) || nbg < 2) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const int nseg = (n + RG_SEG - 1) / RG_SEG;
  int* r = rec + ((long)t * S + slot) * RG_REC;
  const int* hp = hpart + ((long)t * (1 << level) + slot) * nseg_max * 256;
  for (int b = tid; b < 256; b += RG_T) {
    int c = 0;
    for (int g = 0; g < nseg; ++g) c += hp[g * 256 + b];
    s_hist[b] = c;
  }
  if (tid == 0) {
    s_prefix = (shift == 24) ? 0u : (uint32_t)r[0];
    s_need = (shift == 24) ? ((nbg + 1) >> 1) * BK : r[1];
  }
  __syncthreads();
  if (tid < 64) radix_pick(s_hist, &s_prefix, &s_need, shift);
  __syncthreads();
  if (tid == 0) {
    r[0] = (int)s_prefix;
    r[1] = s_need;
  }
}

// The levels whose groups exceed WIDE_MIN blocks take the threshold from the
// many-workgroup rounds and partition one segment per workgroup.
constexpr int WIDE_MIN = 64;
static bool wide_select(int nb, int lev) { return (nb >> lev) > WIDE_MIN; }

// Largest radix_hist grid (groups x segments) over the levels that use it.
static long radix_hist_slots(int N, int BK, int nb, int Lf) {
  long mx = 0;
  for (int lev = 0; lev < Lf; ++lev) {
    if (!wide_select(nb, lev)) continue;
    const long gmax = (nb + (1L << lev) - 1) >> lev;
    mx = std::max(mx, (1L << lev) * ((gmax * BK + RG_SEG - 1) / RG_SEG));
  }
  return mx;
}

// Keys (descending-order keys of the scores) and ids of the 8 positions
// q .. q + 7 of a group's rows [base, base + n); past n: key 0xffffffff, id 0.
__device__ __forceinline__ void fetch8(const float* __restrict__ s, const int32_t* __restrict__ ids_in,
                                       long base, int n, int q, bool vec_ok, uint32_t (&kn)[8],
                                       int32_t (&idn)[8]) {
  if (vec_ok && q + 8 <= n) {   // two 16-byte loads per array
    const float4 s0 = *reinterpret_cast<const float4*>(s + base + q);
    const float4 s1 = *reinterpret_cast<const float4*>(s + base + q + 4);
    const int4 i0 = *reinterpret_cast<const int4*>(ids_in + base + q);
    const int4 i1 = *reinterpret_cast<const int4*>(ids_in + base + q + 4);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const int32_t iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kn[e] = pref_key_desc(sv[e]);
      idn[e] = iv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = q + e;
      kn[e] = (p < n) ? pref_key_desc(s[base + p]) : 0xffffffffu;
      idn[e] = (p < n) ? ids_in[base + p] : 0;
    }
  }
}

// One tile of the stable capacity partition: positions p0 .. p0 + 8 NT - 1
// of a group of n (this thread's keys k and ids idv at p0 + 8 tid ..), the
// c_L-th key thr and the number of its ties that go left.  Before position
// p, lt(p) keys are below thr and eq(p) equal to it; a tie goes left iff its
// rank among ties is < ties_needed, so the lefts before p number lt(p) +
// min(eq(p), ties_needed): one scan of the packed (lt, eq) counts places
// every element.  run_lt / run_eq: those counts before the tile, advanced
// past it.  lds_left (optional): an LDS copy of the left child's ids at
// their output positions (each at most its own position, so it may alias
// keys of this and earlier tiles, already read).  The tile's lefts land in one run of out, its rights in another:
// the ids are staged in LDS in output order and both runs written with
// contiguous stores.  Every thread of the workgroup calls it (three
// barriers, the stage reusable on return).
template <int NT>
__device__ __forceinline__ void partition_tile(const uint32_t (&k)[8], const int32_t (&idv)[8], int p0, int n,
                                               uint32_t thr, int ties_needed, int cL, int& run_lt,
                                               int& run_eq, int* s_tmp, int32_t* s_stage,
                                               int32_t* __restrict__ out, int32_t* lds_left = nullptr) {
  constexpr int E = 8;
  const int tid = threadIdx.x;
  int lt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool valid = p0 + tid * E + e < n;
    lt += (valid && k[e] < thr);
    eq += (valid && k[e] == thr);
  }
  int tot;
  const int packed = wg_exscan<NT>((lt << 16) | eq, s_tmp, tot);   // tile counts < 2^16
  int lt_c = run_lt + (packed >> 16), eq_c = run_eq + (packed & 0xffff);
  const int tile_n = min(NT * E, n - p0);
  const int lb_tile = run_lt + min(run_eq, ties_needed);               // lefts before the tile
  const int la_tile = run_lt + (tot >> 16) + min(run_eq + (tot & 0xffff), ties_needed);
  const int nl_tile = la_tile - lb_tile;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = p0 + tid * E + e;
    if (p >= n) continue;
    const int left_before = lt_c + min(eq_c, ties_needed);
    bool l;
    if (k[e] < thr) {
      l = true;
      ++lt_c;
    } else if (k[e] == thr) {
      l = eq_c < ties_needed;
      ++eq_c;
    } else {
      l = false;
    }
    // position in the tile's output: lefts first, then rights, both in order
    const int j = l ? left_before - lb_tile : nl_tile + (p - left_before) - (p0 - lb_tile);
    s_stage[j] = idv[e];
  }
  __syncthreads();
  const int rb_tile = p0 - lb_tile;                                     // rights before the tile
  for (int j = tid; j < tile_n; j += NT) {
    const int dst = (j < nl_tile) ? lb_tile + j : cL + rb_tile + (j - nl_tile);
    if (dst < n) out[dst] = s_stage[j];
    if (lds_left != nullptr && j < nl_tile) lds_left[dst] = s_stage[j];
  }
  __syncthreads();   // the stage is rewritten by the next tile
  run_lt += tot >> 16;
  run_eq += tot & 0xffff;
}

// The partition of the large groups, one workgroup per RG_SEG positions of a
// group, after the many-workgroup radix rounds (thr and the ties that go left
// in rec).  seg_count stores each segment's keys below and equal to thr,
// packed (below << 16 | equal); seg_partition takes the counts before its
// segment as the sums over the earlier segments and places the segment as
// one tile of the one-workgroup partition: the same positions for every id.
constexpr int SEG_T = RG_SEG / 8;   // 1024 threads, 8 positions each

__global__ __launch_bounds__(RG_T) void seg_count(const float* __restrict__ s, const int* __restrict__ rec,
                                                  int* __restrict__ segcnt, int N, int BK, int nb, int level,
                                                  int S, int nseg_max) {
  __shared__ int s_red[2][RG_T / 64];
  const int slot = blockIdx.x / nseg_max, seg = blockIdx.x % nseg_max, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg) || nbg < 2) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const int i0 = seg * RG_SEG;
  if (i0 >= n) return;
  const int i1 = min(n, i0 + RG_SEG);
  const uint32_t thr = (uint32_t)rec[((long)t * S + slot) * RG_REC];
  const long base = (long)t * N + g0;
  int lt = 0, eq = 0;
  constexpr int U = 8;
  for (int j0 = i0; j0 < i1; j0 += U * RG_T) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = j0 + u * RG_T + tid;
      v[u] = (i < i1) ? s[base + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = j0 + u * RG_T + tid;
      const uint32_t k = pref_key_desc(v[u]);
      lt += (i < i1 && k < thr);
      eq += (i < i1 && k == thr);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lt += __shfl_xor(lt, o, 64);
    eq += __shfl_xor(eq, o, 64);
  }
  if (lane == 0) {
    s_red[0][wave] = lt;
    s_red[1][wave] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, b = 0;
#pragma unroll
    for (int w = 0; w < RG_T / 64; ++w) {
      a += s_red[0][w];
      b += s_red[1][w];
    }
    segcnt[((long)t * (1 << level) + slot) * nseg_max + seg] = (a << 16) | b;   // each <= RG_SEG
  }
}

__global__ __launch_bounds__(SEG_T) void seg_partition(const float* __restrict__ s,
                                                      const int32_t* __restrict__ ids_in,
                                                      int32_t* __restrict__ ids_out, int N, int BK, int nb,
                                                      int level, const int* __restrict__ rec,
                                                      const int* __restrict__ segcnt, int S, int nseg_max) {
  __shared__ int s_tmp[SEG_T / 64];
  __shared__ int32_t s_stage[RG_SEG];
  __shared__ int s_before[2];
  const int slot = blockIdx.x / nseg_max, seg = blockIdx.x % nseg_max, t = blockIdx.y;
  const int tid = threadIdx.x;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg)) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const int i0 = seg * RG_SEG;
  if (i0 >= n) return;
  const long base = (long)t * N + g0;
  if (nbg < 2) {  // a leaf carried through this level: copy
    for (int i = i0 + tid; i < min(n, i0 + RG_SEG); i += SEG_T) ids_out[base + i] = ids_in[base + i];
    return;
  }
  const int cL = ((nbg + 1) >> 1) * BK;
  const int* r = rec + ((long)t * S + slot) * RG_REC;
  const uint32_t thr = (uint32_t)r[0];
  const int ties_needed = r[1];
  if (tid < 64) {   // keys below / equal to thr in the earlier segments
    const int* sc = segcnt + ((long)t * (1 << level) + slot) * nseg_max;
    int bl = 0, be = 0;
    for (int g = tid; g < seg; g += 64) {
      const int c = sc[g];
      bl += c >> 16;
      be += c & 0xffff;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      bl += __shfl_xor(bl, o, 64);
      be += __shfl_xor(be, o, 64);
    }
    if (tid == 0) {
      s_before[0] = bl;
      s_before[1] = be;
    }
  }
  uint32_t k[8];
  int32_t idv[8];
  fetch8(s, ids_in, base, n, i0 + tid * 8, (base & 3) == 0, k, idv);
  __syncthreads();
  int run_lt = s_before[0], run_eq = s_before[1];
  partition_tile<SEG_T>(k, idv, i0, n, thr, ties_needed, cL, run_lt, run_eq, s_tmp, s_stage, ids_out + base);
}

// Groups of at most 64 blocks, score pass and capacity select fused: one
// SPL_T workgroup per group gathers the group's rows block by block (ids
// staged in LDS, the same lane layout and FMA order as score_kernel),
// keeps every score's order key in LDS, radix-selects the c_L-th key there
// and stable-partitions the ids: the scores never go to memory (the score
// pass's small writes cost ~10% of its time) and are never re-read.
template <typename T, int D>
__global__ __launch_bounds__(SPL_T) void score_select_small(const T* __restrict__ xh,
                                                            const int32_t* __restrict__ ids_in,
                                                            int32_t* __restrict__ ids_out,
                                                            const float* __restrict__ diff,
                                                            const double* __restrict__ cen_par,
                                                            double* __restrict__ cen_next, int N, int BK,
                                                            int nb, int level, int S) {
  using CR = ChunkRows<T, D>;
  constexpr int NT = SPL_T, E = 8, VE = CR::VE, CPR = CR::CPR, RPP = CR::RPP;
  extern __shared__ uint32_t s_keys[];   // [n] descending-order keys
  __shared__ int32_t s_ids[128];
  __shared__ int s_hist[256];
  __shared__ int s_whist[NT / 64][256];
  __shared__ int s_tmp[NT / 64];
  __shared__ int32_t s_stage[NT * E];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ float s_p[NT / 64][D];
  const int slot = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg)) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const long base = (long)t * N + g0;
  if (nbg < 2) {  // a leaf carried through this level: copy
    for (int i = tid; i < n; i += NT) ids_out[base + i] = ids_in[base + i];
    return;
  }
  const int cL = ((nbg + 1) >> 1) * BK;
  // scores, one block of the group at a time
  {
    const int rg = tid / CPR, c = (tid % CPR) * VE;
    float vec[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) vec[e] = diff[((long)t * S + slot) * D + c + e];
    const T* xt = xh + (long)t * N * D;
    for (int b0 = 0; b0 < n; b0 += BK) {
      const int n_real = min(BK, n - b0);
      stage_ids(s_ids, ids_in + base + b0, n_real);
      CR rows;
      rows.load(xt, s_ids, n_real, rg, c);
#pragma unroll
      for (int it = 0; it < CR::NIT; ++it) {
        const int j = it * RPP + rg;
        float v[VE];
        rows.get(it, v);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc = fmaf(v[e], vec[e], acc);
        acc = group_sum<CPR>(acc);
        if (j < n_real && (tid % CPR) == 0) s_keys[b0 + j] = pref_key_desc(acc);
      }
      __syncthreads();   // s_ids is restaged by the next block
    }
  }
  if (tid == 0) {
    s_prefix = 0u;
    s_need = cL;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < (NT / 64) * 256; i += NT) (&s_whist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t pre = s_prefix;
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = s_keys[i];
      if ((k & hmask) == pre) atomicAdd(&s_whist[wave][(k >> shift) & 255], 1);
    }
    __syncthreads();
    for (int i = tid; i < 256; i += NT) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) c += s_whist[w][i];
      s_hist[i] = c;
    }
    __syncthreads();
    if (tid < 64) radix_pick(s_hist, &s_prefix, &s_need, shift);
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int ties_needed = s_need;
  const bool vec_ok = (base & 3) == 0;
  int run_lt = 0, run_eq = 0;
  for (int p0 = 0; p0 < n; p0 += NT * E) {
    const int q = p0 + tid * E;
    uint32_t k[E];
    int32_t idv[E];
    if (vec_ok && q + E <= n) {
      const int4 i0 = *reinterpret_cast<const int4*>(ids_in + base + q);
      const int4 i1 = *reinterpret_cast<const int4*>(ids_in + base + q + 4);
      const int32_t iv[E] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        k[e] = s_keys[q + e];
        idv[e] = iv[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        k[e] = (q + e < n) ? s_keys[q + e] : 0xffffffffu;
        idv[e] = (q + e < n) ? ids_in[base + q + e] : 0;
      }
    }
    partition_tile<NT>(k, idv, p0, n, thr, ties_needed, cL, run_lt, run_eq, s_tmp, s_stage, ids_out + base,
                       cen_next != nullptr ? reinterpret_cast<int32_t*>(s_keys) : nullptr);
  }
  if (cen_next == nullptr) return;
  // the next level's centroid sums of the two children, exactly as the
  // centroid pass and its reduce would give them: each block of the left
  // child summed in fp32 in cent_partial's lane order and wave order, the
  // blocks added in fp64 in cent_reduce's eight chains, the right child's
  // sum the parent's minus the left's
  // the left child's ids, in order, are in LDS (over the keys); the last
  // tile's barrier made them visible
  const int32_t* left_ids = reinterpret_cast<const int32_t*>(s_keys);
  using CR = ChunkRows<T, D>;
  constexpr int RGW = 64 / CPR;
  const int lane = tid & 63, rl = lane / CPR, cc = (tid % CPR) * VE;
  const T* xt = xh + (long)t * N * D;
  const int nL = (nbg + 1) >> 1;   // left child's blocks
  double a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = 0.0;
  const int nfull8 = nL & ~7;
  for (int lb = 0; lb < nL; ++lb) {
    const int cb = start + lb;
    const int n_real = min(BK, N - cb * BK);
    CR rows;
    rows.load_rows(xt, left_ids + lb * BK, n_real, 32 * wave + rl, RGW, cc);
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
    for (int it = 0; it < CR::NIT; ++it) {
      float v[VE];
      rows.get(it, v);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = group_sum<64, CPR>(acc[e]);
    if (lane < CPR)
#pragma unroll
      for (int e = 0; e < VE; ++e) s_p[wave][cc + e] = acc[e];
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) sum += s_p[w][c];
      // cent_reduce's chains: blocks in full runs of 8 go to chain lb % 8,
      // the rest to chain 0 (a thread owns one column: a[] per column)
      if (c == tid) {
        const int u = (lb < nfull8) ? (lb & 7) : 0;
#pragma unroll
        for (int uu = 0; uu < 8; ++uu)
          if (uu == u) a[uu] += (double)sum;
      }
    }
    __syncthreads();   // s_p is reused by the next block
  }
  if (tid < D) {
    const double sl = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    const int lslot = 2 * slot;   // the children's slots at the next level
    cen_next[((long)t * S + lslot) * D + tid] = sl;
    int rstart, rnb;
    if (group_of_slot(lslot + 1, level + 1, nb, rstart, rnb) && rnb >= 2)
      cen_next[((long)t * S + lslot + 1) * D + tid] = cen_par[((long)t * S + slot) * D + tid] - sl;
  }
}

// Groups of at most 64 blocks: one workgroup per group radix-selects the
// c_L-th key of the group's scores (streamed from global; L2-resident at
// these sizes), then stable-partitions the ids tile by tile.
template <int NT>
__global__ __launch_bounds__(NT) void select_partition(const float* __restrict__ s,
                                                       const int32_t* __restrict__ ids_in,
                                                       int32_t* __restrict__ ids_out, int N,
                                                       int BK, int nb, int level) {
  __shared__ int s_hist[256];
  __shared__ int s_whist[NT / 64][256];  // one histogram per wave (less atomic contention)
  __shared__ int s_tmp[NT / 64];
  __shared__ int32_t s_stage[NT * 8];     // one partition tile's ids in output order
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int slot = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg)) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const long base = (long)t * N + g0;
  if (nbg < 2) {  // a leaf carried through this level: copy
    for (int i = tid; i < n; i += NT) ids_out[base + i] = ids_in[base + i];
    return;
  }
  const int cL = ((nbg + 1) >> 1) * BK;
  if (tid == 0) {
    s_prefix = 0u;
    s_need = cL;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < (NT / 64) * 256; i += NT) (&s_whist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t pre = s_prefix;
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    constexpr int U = 8;  // independent loads in flight per thread
    for (int i0 = 0; i0 < n; i0 += U * NT) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT + tid;
        v[u] = (i < n) ? s[base + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT + tid;
        const uint32_t k = pref_key_desc(v[u]);
        if (i < n && (k & hmask) == pre) atomicAdd(&s_whist[wave][(k >> shift) & 255], 1);
      }
    }
    __syncthreads();
    for (int i = tid; i < 256; i += NT) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) c += s_whist[w][i];
      s_hist[i] = c;
    }
    __syncthreads();
    if (tid < 64) radix_pick(s_hist, &s_prefix, &s_need, shift);
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int ties_needed = s_need;
  // stable partition in tiles of NT * 8 positions, 8 consecutive per
  // thread; each tile's keys and ids are loaded one tile ahead
  constexpr int E = 8;
  int run_lt = 0, run_eq = 0;  // below / equal before this tile
  uint32_t kn[E];
  int32_t idn[E];
  const bool vec_ok = (base & 3) == 0;   // 16-byte aligned rows of this group
  fetch8(s, ids_in, base, n, tid * E, vec_ok, kn, idn);
  for (int p0 = 0; p0 < n; p0 += NT * E) {
    uint32_t k[E];
    int32_t idv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      k[e] = kn[e];
      idv[e] = idn[e];
    }
    if (p0 + NT * E < n) fetch8(s, ids_in, base, n, p0 + NT * E + tid * E, vec_ok, kn, idn);
    partition_tile<NT>(k, idv, p0, n, thr, ties_needed, cL, run_lt, run_eq, s_tmp, s_stage, ids_out + base);
  }
}

// ---- LDS finisher -----------------------------------------------------------
// One workgroup (FIN_T threads) per group of <= FIN_MAX tokens at level L:
// the rows are loaded into LDS once, every remaining split of the subtree runs
// in place, and the final permutation is written.  Row dots use CPR lanes per
// row (one 16-byte chunk each) reduced with shuffles; the centroid sums
// independent rows per lane; all reductions run in a fixed order.
constexpr int FIN_T = 512;
constexpr int FIN_KR = 16;   // rows per lane slot a split holds in registers (host-checked)

template <typename T, int D>
__global__ __launch_bounds__(FIN_T) void finisher(const T* __restrict__ xh,
                                                  const int32_t* __restrict__ ids_in,
                                                  int32_t* __restrict__ perm_lo,
                                                  int32_t* __restrict__ perm_hi, int split_at,
                                                  int N, int BK, int nb, int level, long perm_ld) {
  constexpr int VE = Chunk<T>::VE, CPR = D / VE, RPP = FIN_T / CPR, NW = FIN_T / 64;
  constexpr int RS = D + 16 / (int)sizeof(T);  // padded row stride (elements)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sX = reinterpret_cast<T*>(smem);                          // [n][RS]
  __shared__ int32_t s_oid[FIN_MAX];    // original id of local row r
  __shared__ int16_t s_lid[FIN_MAX];    // current local order (row indices)
  __shared__ int16_t s_tmp_lid[FIN_MAX];
  __shared__ float s_val[FIN_MAX];      // score of local position (group-relative)
  // per team: below the first level the two independent splits of a level
  // run side by side, one in each half of the workgroup
  __shared__ int s_hist[2][256];
  __shared__ float s_vec[2][D];
  __shared__ float s_part[NW][D];       // by workgroup wave
  __shared__ uint64_t s_min[NW];        // by workgroup wave
  __shared__ int s_tmp[NW];             // by workgroup wave
  __shared__ uint32_t s_prefix[2];
  __shared__ int s_need[2];
  __shared__ int s_minr[NW];           // by workgroup wave

  const int slot = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int start, nbg;
  if (!group_of_slot(slot, level, nb, start, nbg)) return;
  const long g0 = (long)start * BK;
  const int n = (int)(min((long)N, (long)(start + nbg) * BK) - g0);
  const long base = (long)t * N + g0;
  const T* xt = xh + (long)t * N * D;

  // ids, then rows: every load of a batch is issued before the first store,
  // so a batch costs one memory latency, not one per load
  {
    constexpr int IB = FIN_MAX / FIN_T;
    int32_t idv[IB];
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      const int i = min(tid + j * FIN_T, n - 1);
      idv[j] = ids_in ? ids_in[base + i] : (int32_t)(g0 + i);
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      const int i = tid + j * FIN_T;
      if (i < n) {
        s_oid[i] = idv[j];
        s_lid[i] = (int16_t)i;
      }
    }
  }
  __syncthreads();
  // rows -> LDS with direct 4-byte-per-lane loads: one instruction moves
  // 256 bytes of one row to LDS (lane i -> row start + 4 i), so the padded
  // row stride is kept and a wave's loads all issue back to back; the row's
  // global offset is a scalar (readlane of its id).
  {
    constexpr int RB = D * (int)sizeof(T);  // row bytes
    constexpr int IPR = (RB + 255) / 256;   // instructions per row
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)xt, (short)0, 0x7fffffff, 0x00020000);
    for (int r0 = __builtin_amdgcn_readfirstlane(wave) * 64; r0 < n; r0 += NW * 64) {
      const int myid = (r0 + lane < n) ? s_oid[r0 + lane] : 0;
      const int cnt = min(64, n - r0);
      for (int j = 0; j < cnt; ++j) {
        const int id = __builtin_amdgcn_readlane(myid, j);
#pragma unroll
        for (int qq = 0; qq < IPR; ++qq) {
          if (qq * 256 + lane * 4 < RB)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs,
                (void __attribute__((address_space(3)))*)(reinterpret_cast<unsigned char*>(sX + (r0 + j) * RS) +
                                                          qq * 256),
                4, (uint32_t)(lane * 4), id * RB + qq * 256, 0, 0);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  // One split of the local positions [a, a + len) (capacity cL to the left)
  // by a team of NT threads (team 0 = the whole workgroup when NT = FIN_T).
  // Every barrier is a workgroup barrier: both teams run this with the same
  // NT and pass the same barriers (a team without a split runs it with
  // len = 0).
  auto split = [&](auto ntc, int team, int a, int len, int cL) {
    constexpr int NT = decltype(ntc)::value;
    constexpr int TW = NT / 64, RPT = NT / CPR;
    const int ttid = tid - team * NT, w0 = team * TW;
    const int rslot = ttid / CPR, cc = (ttid % CPR) * VE;
    int* hist = s_hist[team];
    float* vecs = s_vec[team];
    // this lane's 16-byte chunk of the rows at positions a + rslot + k RPT:
    // read from LDS once for the four row passes below
    uint4 rw[FIN_KR];
    {
      int rid[FIN_KR];
#pragma unroll
      for (int k = 0; k < FIN_KR; ++k) {
        const int i = rslot + k * RPT;
        rid[k] = (i < len) ? (int)s_lid[a + i] : 0;
      }
#pragma unroll
      for (int k = 0; k < FIN_KR; ++k) rw[k] = *reinterpret_cast<const uint4*>(sX + rid[k] * RS + cc);
    }
    // after a row's dot is summed over its CPR lanes every one of them holds
    // it; lane c of the row's lanes keeps the dot of slot k = c (lanes c >=
    // FIN_KR keep none), so each row's dot ends on one lane: its local row
    // number and original id are looked up once per split
    const int own_k = ttid % CPR;
    const int own_i = rslot + own_k * RPT;
    const bool own_ok = own_k < FIN_KR && own_i < len;
    const int own_rid = own_ok ? (int)s_lid[a + own_i] : 0;
    const int own_oid = s_oid[own_rid];
    auto widen = [&](const uint4& q, float (&v)[VE]) {
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
      }
    };
    // dot of every row of [a, a+len) with a vector: chunk_dot(x) is this
    // lane's partial over its chunk; returns the dot of the row this lane
    // keeps (garbage where !own_ok)
    auto rows_dot = [&](auto&& chunk_dot) -> float {
      float mine = 0.f;
#pragma unroll
      for (int k = 0; k < FIN_KR; ++k) {
        if (k * RPT < len) {   // uniform
          const float acc = group_sum<CPR>(chunk_dot(rw[k]));
          mine = (own_k == k) ? acc : mine;
        }
      }
      return mine;
    };
    // partial dot with the fp32 vector in vecs (widened chunk, one FMA chain)
    auto dot_f32 = [&]() -> float {
      float vec[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) vec[e] = vecs[cc + e];
      return rows_dot([&](const uint4& x) {
        // widened afresh (opaque copy): sharing the centroid pass's widened
        // chunks would keep all of them live between the two passes
        uint32_t w0 = x.x, w1 = x.y, w2 = x.z, w3 = x.w;
        asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
        float v[VE];
        widen(make_uint4(w0, w1, w2, w3), v);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc = fmaf(v[e], vec[e], acc);
        return acc;
      });
    };
    // bf16 rows against a bf16 row: both operands exact, two products per
    // v_dot2_f32_bf16, no widening
    auto dot2_chunk = [](const uint4& x, const uint4& y) -> float {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[i]),
                                              __builtin_bit_cast(bf16x2_t, yw[i]), acc, false);
      return acc;
    };
    // argmin over [a, a+len) of (the kept dot, original id) -> local row: the
    // winning row rides along the reduction, so one barrier suffices
    auto argmin_range = [&](float dv) -> int {
      const uint64_t best = own_ok ? argmin_key(dv, own_oid) : ~0ull;
      const uint64_t wb = group_min_u64<64>(best);
      const uint64_t holders = __builtin_amdgcn_ballot_w64(best == wb);
      const int wrow = __builtin_amdgcn_readlane(own_rid, __builtin_ctzll(holders));
      if (lane == 0) {
        s_min[wave] = wb;
        s_minr[wave] = wrow;
      }
      __syncthreads();
      uint64_t b = s_min[w0];
      int r = s_minr[w0];
#pragma unroll
      for (int w = 1; w < TW; ++w)
        if (s_min[w0 + w] < b) {
          b = s_min[w0 + w];
          r = s_minr[w0 + w];
        }
      return r;
    };
    // centroid: per-lane partial sums over independent rows, then lanes with
    // the same chunk (shuffles), then the team's waves (LDS), all in a fixed
    // order
    {
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.f;
      // rows in a fixed order (k ascending, in groups of 4), absent rows of a
      // started group add +0
#pragma unroll
      for (int k0 = 0; k0 < FIN_KR; k0 += 4) {
        if (rslot + k0 * RPT < len) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k = k0 + u;
            float v[VE];
            widen(rw[k], v);
            const bool in = rslot + k * RPT < len;
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] += in ? v[e] : 0.f;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = group_sum<64, CPR>(acc[e]);
      if (lane < CPR)
#pragma unroll
        for (int e = 0; e < VE; ++e) s_part[wave][cc + e] = acc[e];
      __syncthreads();
      for (int c = ttid; c < D; c += NT) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < TW; ++w) sum += s_part[w0 + w][c];
        vecs[c] = sum;
      }
      __syncthreads();
    }
    // pole A: the row least aligned with the centroid sum (fp32 vector)
    const int rA = argmin_range(dot_f32());
    float sv;
    if constexpr (sizeof(T) == 2) {
      // pole B and the score against the pole rows themselves (bf16, exact):
      // s = x . x_A - x . x_B, each lane's two partials differenced before
      // the lane sum
      const uint4 xa = *reinterpret_cast<const uint4*>(sX + rA * RS + cc);
      const int rB = argmin_range(rows_dot([&](const uint4& x) { return dot2_chunk(x, xa); }));
      const uint4 xb = *reinterpret_cast<const uint4*>(sX + rB * RS + cc);
      sv = rows_dot([&](const uint4& x) { return dot2_chunk(x, xa) - dot2_chunk(x, xb); });
    } else {
      for (int c = ttid; c < D; c += NT) vecs[c] = Elem<T>::load(sX + rA * RS + c);
      __syncthreads();
      const int rB = argmin_range(dot_f32());
      for (int c = ttid; c < D; c += NT)
        vecs[c] = Elem<T>::load(sX + rA * RS + c) - Elem<T>::load(sX + rB * RS + c);
      __syncthreads();
      sv = dot_f32();
    }
    if (own_ok) s_val[a + own_i] = sv;
    __syncthreads();
    // the cL-th key: radix select, 8 bits per round, the team's threads
    // counting into its LDS histogram, its first wave picking the digit
    if (ttid == 0) {
      s_prefix[team] = 0;
      s_need[team] = cL;
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = ttid; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
      const uint32_t pre = s_prefix[team];
      const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
      for (int i = ttid; i < len; i += NT) {
        const uint32_t k = pref_key_desc(s_val[a + i]);
        if ((k & hmask) == pre) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (ttid < 64) radix_pick(hist, &s_prefix[team], &s_need[team], shift);
      __syncthreads();
    }
    const uint32_t thr = s_prefix[team];
    const int ties_needed = s_need[team];
    // stable partition: E consecutive positions per thread.  Before position
    // p, lt(p) keys are below the threshold and eq(p) equal to it; a tie
    // goes left iff its rank among ties is < ties_needed, so the lefts before
    // p number lt(p) + min(eq(p), ties_needed): one scan of the packed
    // (lt, eq) counts places every position.
    constexpr int EMAX = FIN_MAX / NT;
    const int E = (len + NT - 1) / NT;
    uint32_t kk[EMAX];
    int lt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int p = ttid * E + e;
      kk[e] = (e < E && p < len) ? pref_key_desc(s_val[a + p]) : 0xffffffffu;
      lt += (e < E && p < len && kk[e] < thr);
      eq += (e < E && p < len && kk[e] == thr);
    }
    int tot;
    const int packed = team_exscan<NT>((lt << 16) | eq, s_tmp, w0, tot);   // counts < 2^16
    int lt_c = packed >> 16, eq_c = packed & 0xffff;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int p = ttid * E + e;
      if (e >= E || p >= len) continue;
      const int left_before = lt_c + min(eq_c, ties_needed);
      bool l;
      if (kk[e] < thr) {
        l = true;
        ++lt_c;
      } else if (kk[e] == thr) {
        l = eq_c < ties_needed;
        ++eq_c;
      } else {
        l = false;
      }
      const int dst = l ? left_before : cL + (p - left_before);
      if (dst < len) s_tmp_lid[a + dst] = s_lid[a + p];
    }
    __syncthreads();
    for (int i = ttid; i < len; i += NT) s_lid[a + i] = s_tmp_lid[a + i];
    __syncthreads();
  };

  // group geometry of `path` at sub-level `sub` below this group: false if
  // that subgroup is a single block (or does not exist)
  auto sub_group = [&](int sub, int path, int& a, int& len, int& cL) {
    int sstart = 0, snb = nbg;
    for (int l = sub - 1; l >= 0; --l) {
      if (snb <= 1) return false;
      const int nl = (snb + 1) >> 1;
      if ((path >> l) & 1) { sstart += nl; snb -= nl; } else snb = nl;
    }
    if (snb < 2) return false;
    a = sstart * BK;
    len = min(n, (sstart + snb) * BK) - a;
    cL = ((snb + 1) >> 1) * BK;
    return true;
  };
  {
    int a, len, cL;
    if (sub_group(0, 0, a, len, cL)) split(std::integral_constant<int, FIN_T>{}, 0, a, len, cL);
  }
  const int team = tid / (FIN_T / 2);
  for (int sub = 1;; ++sub) {
    bool any = false;
    for (int p2 = 0; p2 < (1 << sub); p2 += 2) {
      int a0, len0, cL0, a1, len1, cL1;
      const bool e0 = sub_group(sub, p2, a0, len0, cL0);
      const bool e1 = sub_group(sub, p2 + 1, a1, len1, cL1);
      if (!e0 && !e1) continue;
      any = true;
      int a = 0, len = 0, cL = 0;
      if (team == 0 && e0) { a = a0; len = len0; cL = cL0; }
      if (team == 1 && e1) { a = a1; len = len1; cL = cL1; }
      split(std::integral_constant<int, FIN_T / 2>{}, team, a, len, cL);
    }
    if (!any) break;
  }
  int32_t* perm = (t < split_at) ? perm_lo + (long)t * perm_ld : perm_hi + (long)(t - split_at) * perm_ld;
  for (int i = tid; i < n; i += FIN_T) perm[g0 + i] = s_oid[s_lid[i]];
}

// ---- host side ---------------------------------------------------------------
struct SplitPlan {
  int nb, F, Lf, S;
};

static SplitPlan split_plan(int N, int D, int BK, int esz) {
  SplitPlan p;
  p.nb = cdiv(N, BK);
  int fb = FIN_LDS / (BK * (D * esz + 16));
  fb = std::min(fb, FIN_MAX / BK);
  int F = 1;
  while (F * 2 <= fb) F *= 2;
  // a split keeps at most FIN_KR rows per lane slot in registers: FIN_T
  // threads on the group, FIN_T / 2 on each group of the levels below
  const int rpt = FIN_T / (D / (16 / esz));
  while (F > 1 && (F * BK > FIN_KR * rpt || ((F + 1) / 2) * BK > FIN_KR * (rpt / 2))) F >>= 1;
  p.F = std::max(F, 1);
  // first level whose largest group has <= F blocks
  int L = 0, mx = p.nb;
  while (mx > p.F) {
    mx = (mx + 1) / 2;
    ++L;
  }
  p.Lf = L;
  p.S = L > 0 ? (1 << (L - 1)) : 1;  // slots at the deepest global level
  return p;
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t split_ws_bytes(int count, int N, int D, int BK, int dtype) {
  const int esz = dtype == SPARK_BF16 ? 2 : 4;
  const SplitPlan p = split_plan(N, D, BK, esz);
  size_t b = 0;
  b += 2 * up256((size_t)count * N * 4);            // ids ping-pong
  b += up256((size_t)count * N * 4);                // s
  b += up256((size_t)count * p.nb * D * 4);         // cpart
  b += up256((size_t)count * p.nb * 8);             // mpart
  b += 2 * up256((size_t)count * p.S * D * 8);      // cen (fp64), one per level parity
  b += up256((size_t)count * p.S * D * 4);          // diff
  b += 2 * up256((size_t)count * p.S * 4);          // poleA, poleB
  b += up256((size_t)count * p.S * RG_REC * 4);     // capacity-select records
  b += up256((size_t)count * radix_hist_slots(N, BK, p.nb, p.Lf) * 256 * 4);   // their segment histograms
  b += up256((size_t)count * radix_hist_slots(N, BK, p.nb, p.Lf) * 4);         // segment (below, equal) counts
  return b;
}

template <typename T, int D>
static int split_t(int count, int N, int BK, const void* xhv, int32_t* perm_lo,
                   int32_t* perm_hi, int split_at, long perm_ld, void* ws, hipStream_t st,
                   bool level0_given) {
  const T* xh = (const T*)xhv;
  const SplitPlan p = split_plan(N, D, BK, sizeof(T));
  char* w = (char*)ws;
  int32_t* ids_a = (int32_t*)w; w += up256((size_t)count * N * 4);
  int32_t* ids_b = (int32_t*)w; w += up256((size_t)count * N * 4);
  float* s = (float*)w; w += up256((size_t)count * N * 4);
  float* cpart = (float*)w; w += up256((size_t)count * p.nb * D * 4);
  uint64_t* mpart = (uint64_t*)w; w += up256((size_t)count * p.nb * 8);
  double* cen_ab[2];
  cen_ab[0] = (double*)w; w += up256((size_t)count * p.S * D * 8);
  cen_ab[1] = (double*)w; w += up256((size_t)count * p.S * D * 8);
  float* diff = (float*)w; w += up256((size_t)count * p.S * D * 4);
  int32_t* poleA = (int32_t*)w; w += up256((size_t)count * p.S * 4);
  int32_t* poleB = (int32_t*)w; w += up256((size_t)count * p.S * 4);
  int* rec = (int*)w; w += up256((size_t)count * p.S * RG_REC * 4);
  int* hpart = (int*)w; w += up256((size_t)count * radix_hist_slots(N, BK, p.nb, p.Lf) * 256 * 4);
  int* segcnt = (int*)w;
  const long total = (long)count * N;
  if (p.nb <= 1) {
    hipLaunchKernelGGL(iota_kernel, dim3((int)std::min<long>((total + 255) / 256, 8192)), dim3(256), 0, st, perm_lo, perm_hi, split_at, N, perm_ld, 0, total);
    return spark_check_launch("split iota");
  }
  int32_t* cur = nullptr;
  if (p.Lf > 0) {
    hipLaunchKernelGGL(iota_kernel, dim3((int)std::min<long>((total + 255) / 256, 8192)), dim3(256), 0, st, ids_a, ids_a, count, N, (long)N, 0, total);
    cur = ids_a;
    int32_t* nxt = ids_b;
    for (int lev = 0; lev < p.Lf; ++lev) {
      const int S = 1 << lev;
      dim3 gc(p.nb, count), gs(S, count), gp(lev == 0 ? 1 : S / 2, count);
      double* cen = cen_ab[lev & 1];             // this level's sums; the parents' in the other
      // below a small level its fused kernel has already stored these sums
      const bool sums_given = lev > 0 && !wide_select(p.nb, lev - 1);
      if (!sums_given) {
        if (lev > 0 || !level0_given)   // else the whitening pass stored the root's partials
          hipLaunchKernelGGL((cent_partial<T, D>), gc, dim3(SPL_T), 0, st, xh, cur, cpart, N, BK, p.nb, lev);
        if ((p.nb >> lev) > 64)
          hipLaunchKernelGGL((cent_reduce<D, 1024>), gp, dim3(1024), 0, st, cpart, cen_ab[(lev + 1) & 1], cen, p.nb, lev, p.S);
        else
          hipLaunchKernelGGL((cent_reduce<D, D>), gp, dim3(D), 0, st, cpart, cen_ab[(lev + 1) & 1], cen, p.nb, lev, p.S);
      }
      hipLaunchKernelGGL((argmin_partial<T, D>), gc, dim3(SPL_T), 0, st, xh, cur, cen, poleA, mpart, N, BK, p.nb, lev, p.S, 0);
      hipLaunchKernelGGL((argmin_reduce<T, D>), gs, dim3(64), 0, st, mpart, xh, poleA, poleB, diff, N, p.nb, lev, p.S, 0);
      hipLaunchKernelGGL((argmin_partial<T, D>), gc, dim3(SPL_T), 0, st, xh, cur, cen, poleA, mpart, N, BK, p.nb, lev, p.S, 1);
      hipLaunchKernelGGL((argmin_reduce<T, D>), gs, dim3(64), 0, st, mpart, xh, poleA, poleB, diff, N, p.nb, lev, p.S, 1);
      // groups of more than 64 blocks: scores to memory, then the threshold
      // and the partition by many workgroups per group; smaller ones: one
      // workgroup per group scores, selects and partitions
      if (wide_select(p.nb, lev)) {
        hipLaunchKernelGGL((score_kernel<T, D>), gc, dim3(SPL_T), 0, st, xh, cur, diff, s, N, BK, p.nb, lev, p.S);
        const int gmax = (p.nb + (1 << lev) - 1) >> lev;   // largest group, blocks
        const int nseg_max = (int)(((long)gmax * BK + RG_SEG - 1) / RG_SEG);
        for (int shift = 24; shift >= 0; shift -= 8) {
          hipLaunchKernelGGL(radix_hist, dim3(S * nseg_max, count), dim3(RG_T), 0, st, s, rec, hpart, N, BK,
                             p.nb, lev, p.S, nseg_max, shift);
          hipLaunchKernelGGL(radix_pick_groups, gs, dim3(RG_T), 0, st, rec, hpart, N, BK, p.nb, lev, p.S,
                             nseg_max, shift);
        }
        hipLaunchKernelGGL(seg_count, dim3(S * nseg_max, count), dim3(RG_T), 0, st, s, rec, segcnt, N, BK, p.nb,
                           lev, p.S, nseg_max);
        hipLaunchKernelGGL(seg_partition, dim3(S * nseg_max, count), dim3(SEG_T), 0, st, s, cur, nxt, N, BK,
                           p.nb, lev, (const int*)rec, (const int*)segcnt, p.S, nseg_max);
      } else {
        const int gmax = (p.nb + (1 << lev) - 1) >> lev;   // largest group, blocks
        hipLaunchKernelGGL((score_select_small<T, D>), gs, dim3(SPL_T), (size_t)std::min(N, gmax * BK) * 4, st, xh,
                           cur, nxt, diff, (const double*)cen, lev + 1 < p.Lf ? cen_ab[(lev + 1) & 1] : nullptr, N,
                           BK, p.nb, lev, p.S);
      }
      int rc = spark_check_launch("split level");
      if (rc) return rc;
      std::swap(cur, nxt);
    }
  }
  const int SF = 1 << p.Lf;
  constexpr int RS = D + 16 / (int)sizeof(T);
  const size_t lds = (size_t)std::min(N, p.F * BK) * RS * sizeof(T);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)finisher<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, FIN_LDS);
    attr = true;
  }
  hipLaunchKernelGGL((finisher<T, D>), dim3(SF, count), dim3(FIN_T), lds, st, xh, cur, perm_lo, perm_hi, split_at, N, BK, p.nb, p.Lf, perm_ld);
  return spark_check_launch("split finisher");
}

__global__ void copy_perm_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

int copy_perm_launch(long count, const int32_t* src, int32_t* dst, hipStream_t st) {
  hipLaunchKernelGGL(copy_perm_kernel, dim3((int)std::min<long>((count + 255) / 256, 8192)), dim3(256), 0, st,
                     src, dst, count);
  return spark_check_launch("copy_perm");
}

// rows of ld entries: row[from + i] = from + i for i < n (the identity on
// positions [from, from + n))
int iota_launch(int count, int n, long ld, int from, int32_t* lo, int32_t* hi, int split_at,
                hipStream_t st) {
  const long total = (long)count * n;
  if (total == 0) return SPARK_OK;
  hipLaunchKernelGGL(iota_kernel, dim3((int)std::min<long>((total + 255) / 256, 8192)), dim3(256), 0, st, lo, hi, split_at, n, ld, from, total);
  return spark_check_launch("iota");
}

// Trees [0, split_at) write to perm_lo, trees [split_at, count) to perm_hi,
// N entries per tree at a stride of perm_ld >= N.
// level0_given: the root's per-block partial centroid sums are already in
// the workspace (split_level0_partials), stored by the whitening pass.
int split_launch(int count, int N, int D, int BK, int dtype, const void* xh, int32_t* perm_lo,
                 int32_t* perm_hi, int split_at, long perm_ld, void* ws, hipStream_t st,
                 bool level0_given) {
  if (dtype == SPARK_BF16)
    return D == 128 ? split_t<uint16_t, 128>(count, N, BK, xh, perm_lo, perm_hi, split_at, perm_ld, ws, st, level0_given)
                    : split_t<uint16_t, 64>(count, N, BK, xh, perm_lo, perm_hi, split_at, perm_ld, ws, st, level0_given);
  return D == 128 ? split_t<float, 128>(count, N, BK, xh, perm_lo, perm_hi, split_at, perm_ld, ws, st, level0_given)
                  : split_t<float, 64>(count, N, BK, xh, perm_lo, perm_hi, split_at, perm_ld, ws, st, level0_given);
}

// ---- test hooks: the split's argmin and capacity partition on caller values ----
// Argmin of caller values per row with the splitter's 64-bit (key, id)
// ordering and wave reduction: -0 equals +0, NaN ranks last, ties to the
// lower id.  One workgroup per row.
__global__ __launch_bounds__(SPL_T) void debug_argmin_kernel(const float* __restrict__ vals,
                                                             const int32_t* __restrict__ ids, int n,
                                                             int32_t* __restrict__ out) {
  __shared__ uint64_t s_min[SPL_T / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  uint64_t best = ~0ull;
  for (int i = tid; i < n; i += SPL_T) {
    const uint64_t k = argmin_key(vals[(long)t * n + i], ids[(long)t * n + i]);
    best = k < best ? k : best;
  }
  best = group_min_u64<64>(best);
  if ((tid & 63) == 0) s_min[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = s_min[0];
    for (int w = 1; w < SPL_T / 64; ++w) b = s_min[w] < b ? s_min[w] : b;
    out[t] = (int32_t)(uint32_t)(b & 0xffffffffu);
  }
}

int debug_argmin_launch(int count, int n, const float* vals, const int32_t* ids, int32_t* out,
                        hipStream_t st) {
  hipLaunchKernelGGL(debug_argmin_kernel, dim3(count), dim3(SPL_T), 0, st, vals, ids, n, out);
  return spark_check_launch("debug argmin");
}

// One capacity partition per row of n scores: the split's level-0 kernels
// (above 64 blocks the many-workgroup radix rounds and the segmented
// partition, the one-workgroup select below), with the capacity of a group
// of ceil(n / BK) blocks.
size_t debug_partition_ws_bytes(int count, int n, int BK) {
  const int nb = cdiv(n, BK);
  const long nseg = wide_select(nb, 0) ? ((long)nb * BK + RG_SEG - 1) / RG_SEG : 0;
  return up256((size_t)count * RG_REC * 4) + up256((size_t)count * nseg * 256 * 4) + up256((size_t)count * nseg * 4);
}

int debug_partition_launch(int count, int n, int BK, const float* s, const int32_t* ids_in,
                           int32_t* ids_out, void* ws, hipStream_t st) {
  const int nb = cdiv(n, BK);
  int* rec = (int*)ws;
  int* hpart = (int*)((char*)ws + up256((size_t)count * RG_REC * 4));
  const dim3 gs(1, count);
  if (wide_select(nb, 0)) {
    const int nseg_max = (int)(((long)nb * BK + RG_SEG - 1) / RG_SEG);
    int* segcnt = (int*)((char*)hpart + up256((size_t)count * nseg_max * 256 * 4));
    for (int shift = 24; shift >= 0; shift -= 8) {
      hipLaunchKernelGGL(radix_hist, dim3(nseg_max, count), dim3(RG_T), 0, st, s, rec, hpart, n, BK, nb, 0, 1,
                         nseg_max, shift);
      hipLaunchKernelGGL(radix_pick_groups, gs, dim3(RG_T), 0, st, rec, hpart, n, BK, nb, 0, 1, nseg_max, shift);
    }
    hipLaunchKernelGGL(seg_count, dim3(nseg_max, count), dim3(RG_T), 0, st, s, rec, segcnt, n, BK, nb, 0, 1,
                       nseg_max);
    hipLaunchKernelGGL(seg_partition, dim3(nseg_max, count), dim3(SEG_T), 0, st, s, ids_in, ids_out, n, BK, nb, 0,
                       (const int*)rec, (const int*)segcnt, 1, nseg_max);
  } else {
    hipLaunchKernelGGL(select_partition<SPL_T>, gs, dim3(SPL_T), 0, st, s, ids_in, ids_out, n, BK, nb, 0);
  }
  return spark_check_launch("debug partition");
}

// Where split_launch keeps its per-block partial centroid sums
// ([count][n_b][D] fp32) inside ws; NULL when the tree has a single block
// (no global level runs).
float* split_level0_partials(void* ws, int count, int N, int D, int BK, int dtype) {
  const int esz = dtype == SPARK_BF16 ? 2 : 4;
  const SplitPlan p = split_plan(N, D, BK, esz);
  if (p.nb <= 1 || p.Lf == 0) return nullptr;
  return (float*)((char*)ws + 3 * up256((size_t)count * N * 4));   // after ids_a, ids_b, s
}

}  // namespace spark
