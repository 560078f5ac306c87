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
#include "ep_internal.h"
#include "route_impl.h"

namespace epk {

constexpr int kRouteWaves = 4;          // waves per workgroup
constexpr int32_t kRouteWideTokens = 1024;  // up to this many tokens: one wave per token

template <int G, int PER>  // lanes per token (16 or 64); logits per lane: ceil(E / G) <= PER
__global__ __launch_bounds__(64 * kRouteWaves) void k_route(const float *__restrict__ logits,
                                                            int32_t T, int32_t E, int32_t k,
                                                            int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (G - 1);
  const int64_t t = ((int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  if (G == 64 && t >= T) return;  // the whole wave leaves together
  const bool live = t < T;        // (G = 16) dead rows still take part in the exchanges
  int32_t my_i;
  float my_w;
  route_token<G, PER>(logits, t, live, E, k, lane, my_i, my_w);
  if (live && sub < k) {
    idx_out[t * k + sub] = my_i;
    w_out[t * k + sub] = my_w;
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
