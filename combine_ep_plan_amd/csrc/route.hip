// route.hip -- top-k routing on gfx950: router logits [T, E] -> the k
// experts of each token (descending logit, equal logits to the lower expert
// id, choice 0 the largest) and the softmax over the chosen logits.  This is
// the gate step before dispatch ("Ultra-Large MoE Models" article, sections
// 2.1 and 3.1-3.2: top-k selection over the gate's scores, a fused top-k +
// routing operator); its outputs are the top-k index and weight tensors of
// the NCCL EP listing's Table IV.
//
// G lanes per token: a whole wave (G = 64) when there are few tokens, so one
// token's rounds are short; 16 lanes (four tokens per wave) when there are
// many, where fewer instructions per token matter more than latency.  Each
// lane holds E/G logits (coalesced loads), turned
// once into order keys: signed integers that compare like the floats (-0
// made +0 first, so it ties with +0 as the float compare does).  Each of the
// k rounds takes the largest key not yet taken: a branch-free scan of the
// lane's own keys (strict '>', so the lowest of equal keys in the lane
// stays), then a maximum over the token's G lanes of (key, ~expert) packed
// into 64 bits, which breaks ties toward the lower expert id.  The exchange
// is all VALU: four DPP lane moves inside each 16-lane row, then (G = 64) the
// gfx950 permlane16 / permlane32 swaps across rows and halves (no LDS round
// trips).
// The owning lane sets the taken key to INT_MIN, below every float's key, so
// it is never chosen again.  Lane j keeps round j's winner, so the softmax
// (fp32 exp, wave sum) and the stores are one instruction per output.  With
// fewer than k experts the extra choices are -1 with weight 0.
#include <math.h>

#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kRouteWaves = 4;          // waves per workgroup
constexpr int32_t kRouteWideTokens = 1024;  // up to this many tokens: one wave per token
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

template <int G, int PER>  // lanes per token (16 or 64); logits per lane: ceil(E / G) <= PER
__global__ __launch_bounds__(64 * kRouteWaves) void k_route(const float *__restrict__ logits,
                                                            int32_t T, int32_t E, int32_t k,
                                                            int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out) {
  static_assert(G == 16 || G == 64, "a token takes one DPP row or the whole wave");
  const int lane = threadIdx.x & 63;
  const int sub = lane & (G - 1);
  const bool up16 = (lane & 16) != 0, up32 = (lane & 32) != 0;
  const int64_t t = ((int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  if (G == 64 && t >= T) return;  // the whole wave leaves together
  const bool live = t < T;        // (G = 16) dead rows still take part in the exchanges
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
  if (live && sub < k) {
    idx_out[t * k + sub] = my_i;
    w_out[t * k + sub] = chosen ? z / s : 0.0f;
  }
}

hipError_t launch_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx,
                        float *w, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define L(G, P)                                                                             \
  hipLaunchKernelGGL((k_route<G, P>), dim3(blocks), dim3(64 * kRouteWaves), 0, s, logits, T, \
                     E, k, idx, w)
  if (T <= kRouteWideTokens) {
    const unsigned blocks = (unsigned)((T + kRouteWaves - 1) / kRouteWaves);
    const int per = (E + 63) / 64;
    if (per <= 1) L(64, 1);
    else if (per <= 2) L(64, 2);
    else if (per <= 4) L(64, 4);
    else if (per <= 8) L(64, 8);
    else L(64, 16);
  } else {
    const int64_t tokens_per_block = (int64_t)kRouteWaves * 4;
    const unsigned blocks = (unsigned)((T + tokens_per_block - 1) / tokens_per_block);
    const int per = (E + 15) / 16;
    if (per <= 1) L(16, 1);
    else if (per <= 2) L(16, 2);
    else if (per <= 4) L(16, 4);
    else if (per <= 8) L(16, 8);
    else if (per <= 16) L(16, 16);
    else if (per <= 32) L(16, 32);
    else L(16, 64);
  }
#undef L
  return hipGetLastError();
}

}  // namespace epk
