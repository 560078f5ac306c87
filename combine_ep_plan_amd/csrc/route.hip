// route.hip -- top-k routing on gfx950: router logits [T, E] -> the k
// experts of each token (descending logit, equal logits to the lower expert
// id, choice 0 the largest) and the softmax over the chosen logits.  This is
// the gate step before dispatch ("Ultra-Large MoE Models" article, sections
// 2.1 and 3.1-3.2: top-k selection over the gate's scores, a fused top-k +
// routing operator); its outputs are the top-k index and weight tensors of
// the NCCL EP listing's Table IV.
//
// Sixteen lanes per token (four tokens per wave).  Each lane holds E/16
// logits (coalesced loads), turned once into order keys: signed integers
// that compare like the floats (-0 made +0 first, so it ties with +0 as the
// float compare does).  Each of the k rounds takes the largest key not yet
// taken: a branch-free scan of the lane's own keys (strict '>', so the
// lowest of equal keys in the lane stays), then a maximum over the token's
// 16 lanes of (key, ~expert) packed into 64 bits, which breaks ties toward
// the lower expert id, moved between lanes by DPP (no LDS round trips).  The
// owning lane sets the taken key to INT_MIN, below every float's key, so it
// is never chosen again.  Lane j of the group keeps round j's winner, so the
// softmax (fp32 exp, group sum) and the stores are one instruction per
// output.  With fewer than k experts the extra choices are -1 with weight 0.
#include <math.h>

#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kRouteWaves = 4;
constexpr int kLanesPerToken = 16;   // one DPP row; >= the largest k
constexpr int kTokensPerWave = 64 / kLanesPerToken;
constexpr int32_t kTakenKey = INT32_MIN;

// Lane exchanges inside a 16-lane DPP row: after the four steps xor-1,
// xor-2 (quad permutes), half-row mirror (lane i <-> 7-i of each 8) and row
// mirror (lane i <-> 15-i) every lane has combined all 16 lanes' values.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int32_t dpp(int32_t v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
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

template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t p) {
  const uint32_t lo = (uint32_t)dpp<CTRL>((int32_t)(uint32_t)p);
  const uint32_t hi = (uint32_t)dpp<CTRL>((int32_t)(uint32_t)(p >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > p ? o : p;
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float s) {
  return s + __int_as_float(dpp<CTRL>(__float_as_int(s)));
}

template <int PER>  // logits per lane: ceil(E / 16) <= PER
__global__ __launch_bounds__(64 * kRouteWaves) void k_route(const float *__restrict__ logits,
                                                            int32_t T, int32_t E, int32_t k,
                                                            int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out) {
  constexpr int L = kLanesPerToken;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (L - 1);
  const int64_t t = ((int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * kTokensPerWave +
                    (lane / L);
  const bool live = t < T;   // dead groups read token 0 and still take part in the exchanges
  const float *l = logits + (live ? t : 0) * E;
  // All loads first (clamped index, so every one is in bounds and none
  // waits behind a branch), then the keys; columns past E are taken.
  float x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = l[min(sub + L * i, E - 1)];
  int32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int32_t kv = order_key(x[i]);
    key[i] = sub + L * i < E ? kv : kTakenKey;
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
    uint64_t p = pack_choice(bk, bp < 0 ? -1 : sub + L * bp);
    p = max_step<kDppXor1>(p);       // stays inside the token's 16 lanes
    p = max_step<kDppXor2>(p);
    p = max_step<kDppHalfMirror>(p);
    p = max_step<kDppMirror>(p);
    if (j == 0) top = p;             // every lane of the token sees the largest logit
    const int32_t we = (int32_t)~(uint32_t)p;
    const int32_t tpos = (p != 0 && (we & (L - 1)) == sub) ? we / L : -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = i == tpos ? kTakenKey : key[i];
    mine = sub == j ? p : mine;
  }
  const bool chosen = sub < k && mine != 0;
  const int32_t my_i = chosen ? (int32_t)~(uint32_t)mine : -1;
  const float my_v = key_value((int32_t)((uint32_t)(mine >> 32) ^ 0x80000000u));
  const float vmax = key_value((int32_t)((uint32_t)(top >> 32) ^ 0x80000000u));
  const float z = chosen ? expf(my_v - vmax) : 0.0f;
  float s = sum_step<kDppXor1>(z);
  s = sum_step<kDppXor2>(s);
  s = sum_step<kDppHalfMirror>(s);
  s = sum_step<kDppMirror>(s);
  if (live && sub < k) {
    idx_out[t * k + sub] = my_i;
    w_out[t * k + sub] = chosen ? z / s : 0.0f;
  }
}

hipError_t launch_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx,
                        float *w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kRouteWaves * kTokensPerWave;
  const unsigned blocks = (unsigned)((T + per_block - 1) / per_block);
  const int per = (E + kLanesPerToken - 1) / kLanesPerToken;
#define L(P) hipLaunchKernelGGL(k_route<P>, dim3(blocks), dim3(64 * kRouteWaves), 0, s, logits, T, E, k, idx, w)
  if (per <= 1) L(1);
  else if (per <= 2) L(2);
  else if (per <= 4) L(4);
  else if (per <= 8) L(8);
  else if (per <= 16) L(16);
  else if (per <= 32) L(32);
  else L(64);
#undef L
  return hipGetLastError();
}

}  // namespace epk
