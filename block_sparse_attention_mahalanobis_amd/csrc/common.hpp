// Shared device/host helpers of libspark (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdlib>
#include <utility>

#include "../../include/spark.h"

namespace spark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- bf16 <-> fp32 (storage is uint16_t; round to nearest even) ----------
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Element access for the two storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float zero_bits() { return 0.f; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f2bf(v); }
};

// Load 8 consecutive elements as floats (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 u;
  u.x = pack_bf2(v[0], v[1]);
  u.y = pack_bf2(v[2], v[3]);
  u.z = pack_bf2(v[4], v[5]);
  u.w = pack_bf2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Monotone map of a float to uint32 so that unsigned order == float order;
// -0 is folded onto +0 and every NaN maps above +inf.
__device__ __forceinline__ uint32_t float_key_asc(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// k-th smallest (1-based) of n uint32 keys, found by ONE wave with a private
// LDS histogram of NC x 256 ints: 4 radix rounds of 8 bits (count the keys
// that match the prefix so far, then pick the digit holding rank k).
// Returns the key; *ties_needed = k - count(key < result).
// count(prefix, hmask, shift, h) adds, for every key with (key & hmask) ==
// prefix, one to h[(key >> shift) & 255], where h is the lane's copy of the
// histogram (lane % NC picks it: keys that share a digit then contend NC
// times less on the same LDS word); the keys may sit in LDS or in registers.
//
// The hardware runs one wave's LDS instructions in issue order, but to the
// compiler the other lanes' atomics race with the plain reads: without an
// ordering point it may forward a lane's own zero store to its read of the
// same bin (seen: lanes past n read empty bins).  wave_lds_sync() waits for
// the wave's LDS operations and is a compiler memory barrier.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int NC = 1, typename CountFn>
__device__ __forceinline__ uint32_t wave_radix_select(int k, int* hist, int* ties_needed,
                                                      CountFn&& count) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4 * NC; ++j) hist[64 * j + lane] = 0;
    wave_lds_sync();
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    count(prefix, hmask, shift, hist + 256 * (lane % NC));
    wave_lds_sync();
    int c[4], run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int v = 0;
#pragma unroll
      for (int r = 0; r < NC; ++r) v += hist[256 * r + 4 * lane + j];
      run += v;
      c[j] = run;
    }
    wave_lds_sync();  // every lane has read its bins before the next round clears them
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int base = incl - run;
    int found = -1, fb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int before = base + (j ? c[j - 1] : 0);
      if (before < need && base + c[j] >= need) {
        found = 4 * lane + j;
        fb = before;
      }
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(found >= 0);
    const int src = __builtin_ctzll(m);
    const int digit = __builtin_amdgcn_readlane(found, src);
    need -= __builtin_amdgcn_readlane(fb, src);
    prefix |= (uint32_t)digit << shift;
  }
  *ties_needed = need;
  return prefix;
}

// The n keys in LDS, lane i counting keys i, i + 64, ...
__device__ __forceinline__ uint32_t wave_radix_kth(const uint32_t* keys, int n, int k, int* hist,
                                                   int* ties_needed) {
  const int lane = threadIdx.x & 63;
  return wave_radix_select(k, hist, ties_needed, [&](uint32_t prefix, uint32_t hmask, int shift, int* h) {
    for (int i = lane; i < n; i += 64) {
      const uint32_t key = keys[i];
      if ((key & hmask) == prefix) atomicAdd(&h[(key >> shift) & 255], 1);
    }
  });
}

// Butterfly reductions over aligned groups of G lanes (G a power of two,
// 2..64); every lane of a group ends with the group's result, bit-identical
// across the group.  Step S combines each lane with its xor-S partner.  Within
// a 16-lane row the partner comes from DPP moves; across rows,
// v_permlane16_swap / v_permlane32_swap exchange whole rows in one VALU op.
// No LDS crossbar (ds_bpermute) traffic.
//
// A reduction that starts at step 1 may use a half-row / row mirror for steps
// 4 and 8 (after the earlier steps every S-subgroup is uniform, so lane 7-i
// holds what lane i^4 holds); one that starts at S0 > 1 (folding lanes that
// own the same column chunk of different rows) needs the exact xor, built
// from two bank-masked row shifts.
template <int CTRL, int BANKS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xf, BANKS, false);
}
template <int S, bool UNIFORM>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8, "DPP step");
  if constexpr (S == 1) return dpp_u32<0xB1>(0, v);       // quad_perm [1,0,3,2]
  else if constexpr (S == 2) return dpp_u32<0x4E>(0, v);  // quad_perm [2,3,0,1]
  else if constexpr (UNIFORM && S == 4) return dpp_u32<0x141>(0, v);  // row_half_mirror
  else if constexpr (UNIFORM && S == 8) return dpp_u32<0x140>(0, v);  // row_mirror
  else if constexpr (S == 4)
    // banks (4-lane groups of a row) 0 and 2 read lane+4, banks 1 and 3 lane-4
    return dpp_u32<0x104, 0x5>(dpp_u32<0x114, 0xA>(0, v), v);
  else
    // banks 0-1 read lane+8, banks 2-3 lane-8
    return dpp_u32<0x108, 0x3>(dpp_u32<0x118, 0xC>(0, v), v);
}
// (a, b) = this lane's value and its xor-S partner's (in either order).
template <int S, bool UNIFORM>
__device__ __forceinline__ void bfly_pair(uint32_t v, uint32_t& a, uint32_t& b) {
  if constexpr (S <= 8) {
    a = v;
    b = dpp_partner<S, UNIFORM>(v);
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else {
    static_assert(S == 32, "step");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
}

// Sum over aligned groups of G lanes; with S0 > 1, lanes S0 apart hold
// partial sums of the same quantity and lanes within an S0-group are unrelated.
template <int G, int S0 = 1, int S = S0>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (S < G) {
    uint32_t a, b;
    bfly_pair<S, S0 == 1>(__float_as_uint(v), a, b);
    return group_sum<G, S0, 2 * S>(__uint_as_float(a) + __uint_as_float(b));
  } else {
    return v;
  }
}
template <int G, int S = 1>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (S < G) {
    uint32_t a, b;
    bfly_pair<S, true>(__float_as_uint(v), a, b);
    return group_max<G, 2 * S>(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  } else {
    return v;
  }
}
template <int G, int S = 1>
__device__ __forceinline__ uint64_t group_min_u64(uint64_t v) {
  if constexpr (S < G) {
    uint32_t ah, bh, al, bl;
    bfly_pair<S, true>((uint32_t)(v >> 32), ah, bh);
    bfly_pair<S, true>((uint32_t)v, al, bl);
    const uint64_t a = ((uint64_t)ah << 32) | al, b = ((uint64_t)bh << 32) | bl;
    return group_min_u64<G, 2 * S>(a < b ? a : b);
  } else {
    return v;
  }
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// 16-byte chunk of a row as floats
template <typename T> struct Chunk;
template <> struct Chunk<uint16_t> {
  static constexpr int VE = 8;
  __device__ __forceinline__ static void load(const uint16_t* p, float* v) { load8(p, v); }
};
template <> struct Chunk<float> {
  static constexpr int VE = 4;
  __device__ __forceinline__ static void load(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
};

inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

}  // namespace spark

// Host-side status plumbing (spark_api.cpp).
int spark_set_error(int status, const char* fmt, ...);
int spark_check_launch(const char* what);
