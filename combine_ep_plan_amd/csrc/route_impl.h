// route_impl.h -- top-k routing of one token by a group of G lanes, shared by
// the routing kernel and the fused routing + layout kernel ("Ultra-Large MoE
// Models" article, sections 2.1 and 3.1-3.2: top-k over the gate's scores
// and a fused top-k + routing operator).  See route.hip for the method.
#pragma once

#include <math.h>

#include "device.h"

namespace epk {

constexpr int32_t kTakenKey = INT32_MIN;

// Lane exchanges inside a 16-lane DPP row: after the four steps xor-1,
// xor-2 (quad permutes), half-row mirror (lane i <-> 7-i of each 8) and row
// mirror (lane i <-> 15-i) every lane has combined all 16 lanes' values.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int32_t)v, CTRL, 0xF, 0xF, false);
}

// The value of lane l ^ 16 (permlane16 swap of a register with itself: the
// first result holds lane l & ~16, the second lane l | 16).
__device__ __forceinline__ uint32_t xor16(uint32_t v, bool upper16) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return upper16 ? r[0] : r[1];
}

// The value of lane l ^ 32 (first result: lane l & 31, second: (l & 31) + 32).
__device__ __forceinline__ uint32_t xor32(uint32_t v, bool upper32) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return upper32 ? r[0] : r[1];
}

// Integer key with the order of the float: non-negative floats keep their
// bits, negative ones flip the magnitude bits (still negative as int32).
__device__ __forceinline__ int32_t order_key(float f) {
  int32_t b = __float_as_int(f);
  b = b == INT32_MIN ? 0 : b;   // -0 -> +0
  return b >= 0 ? b : (b ^ 0x7FFFFFFF);
}

__device__ __forceinline__ float key_value(int32_t key) {
  return __int_as_float(key >= 0 ? key : (key ^ 0x7FFFFFFF));
}

// (key, expert) as one unsigned 64-bit word whose maximum is the larger key,
// then the lower expert; 0 means "none" (key INT_MIN and no expert).
__device__ __forceinline__ uint64_t pack_choice(int32_t key, int32_t e) {
  const uint32_t hi = (uint32_t)key ^ 0x80000000u;
  return e < 0 ? 0ull : (((uint64_t)hi << 32) | (uint32_t)~(uint32_t)e);
}

__device__ __forceinline__ uint64_t join(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp(uint64_t p) {
  const uint64_t o = join(dpp<CTRL>((uint32_t)p), dpp<CTRL>((uint32_t)(p >> 32)));
  return o > p ? o : p;
}

// maximum over the token's G lanes (a 16-lane row, or the whole wave)
template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t p, bool up16, bool up32) {
  p = max_dpp<kDppXor1>(p);
  p = max_dpp<kDppXor2>(p);
  p = max_dpp<kDppHalfMirror>(p);
  p = max_dpp<kDppMirror>(p);
  if constexpr (G == 64) {
    uint64_t o = join(xor16((uint32_t)p, up16), xor16((uint32_t)(p >> 32), up16));
    p = o > p ? o : p;
    o = join(xor32((uint32_t)p, up32), xor32((uint32_t)(p >> 32), up32));
    p = o > p ? o : p;
  }
  return p;
}

template <int G>
__device__ __forceinline__ float group_sum(float s, bool up16, bool up32) {
  s += __uint_as_float(dpp<kDppXor1>(__float_as_uint(s)));
  s += __uint_as_float(dpp<kDppXor2>(__float_as_uint(s)));
  s += __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(s)));
  s += __uint_as_float(dpp<kDppMirror>(__float_as_uint(s)));
  if constexpr (G == 64) {
    s += __uint_as_float(xor16(__float_as_uint(s), up16));
    s += __uint_as_float(xor32(__float_as_uint(s), up32));
  }
  return s;
}

// Route token t with the G lanes of the calling group (sub = lane % G).  All
// G lanes call it, live or not (dead groups still take part in the lane
// exchanges).  On return lane sub < k holds choice sub: the expert (or -1)
// and its softmax weight over the chosen logits.
template <int G, int PER>
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int64_t t, bool live,
                                            int32_t E, int32_t k, int lane, int32_t &out_i,
                                            float &out_w) {
  static_assert(G == 16 || G == 64, "a token takes one DPP row or the whole wave");
  const int sub = lane & (G - 1);
  const bool up16 = (lane & 16) != 0, up32 = (lane & 32) != 0;
  const float *l = logits + (live ? t : 0) * E;
  // All loads first (clamped index, so every one is in bounds and none
  // waits behind a branch), then the keys; columns past E are taken.
  float x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = l[min(sub + G * i, E - 1)];
  int32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int32_t kv = order_key(x[i]);
    key[i] = sub + G * i < E ? kv : kTakenKey;
  }
  uint64_t mine = 0, top = 0;
  for (int32_t j = 0; j < k; ++j) {
    int32_t bk = kTakenKey, bp = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool g = key[i] > bk;
      bk = g ? key[i] : bk;
      bp = g ? i : bp;
    }
    const uint64_t p = group_max<G>(pack_choice(bk, bp < 0 ? -1 : sub + G * bp), up16, up32);
    if (j == 0) top = p;  // the largest logit
    const int32_t we = (int32_t)~(uint32_t)p;
    const int32_t tpos = (p != 0 && (we & (G - 1)) == sub) ? we / G : -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = i == tpos ? kTakenKey : key[i];
    mine = sub == j ? p : mine;
  }
  const bool chosen = sub < k && mine != 0;
  const int32_t my_i = chosen ? (int32_t)~(uint32_t)mine : -1;
  const float my_v = key_value((int32_t)((uint32_t)(mine >> 32) ^ 0x80000000u));
  const float vmax = key_value((int32_t)((uint32_t)(top >> 32) ^ 0x80000000u));
  const float z = chosen ? expf(my_v - vmax) : 0.0f;
  const float s = group_sum<G>(z, up16, up32);
  out_i = my_i;
  out_w = chosen ? z / s : 0.0f;
}

}  // namespace epk
