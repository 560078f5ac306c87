// combine.hip -- combine (NCCL EP paper listing, Table II: gather each
// token's expert outputs back to the token's place), its unit-weight form
// (the backward of dispatch) and the backward of combine (NCCL EP listing,
// Figure 5: the forward pass's routing state is reused), on gfx950.
//
// One workgroup per token (per piece of the row for small batches, as in
// dispatch; combine backward keeps whole rows for its grad_w reduction).
// Each lane owns 8 channels (one 16-byte vector)
// and keeps all k gathers of its vector in flight before reducing them in
// fp32 in ascending j, so the k rows of a token cost one HBM read each and
// the output one HBM write.  The output rows are written cached (the next
// layer finds them in the Infinity Cache) or, as the group asks,
// non-temporally.  Combine backward reads each token's gradient row once, so
// it reads it non-temporally, like the expert rows (a training step
// measured faster so).
#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kRowThreads = 512;

template <int K, bool WEIGHTED, bool OUT_F32, bool NT>
__global__ __launch_bounds__(kRowThreads) void k_combine(const u32x4 *__restrict__ rows,
                                                         const int32_t *__restrict__ dst,
                                                         const float *__restrict__ w,
                                                         void *__restrict__ out, int64_t nrows,
                                                         int32_t V, int32_t kr, int32_t chunk) {
  constexpr int KN = K > 0 ? K : kMaxTopK;
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  int32_t d[KN];
  float wj[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    const bool on = K > 0 || j < k;
    d[j] = on ? dst[t * k + j] : -1;
    if (d[j] >= nrows) d[j] = -1;
    wj[j] = (WEIGHTED && on) ? w[t * k + j] : 1.0f;
  }
  const int32_t lo = blockIdx.y * chunk;
  const int32_t hi = lo + chunk < V ? lo + chunk : V;
  for (int32_t v = lo + threadIdx.x; v < hi; v += kRowThreads) {
    u32x4 r[KN];
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      r[j] = u32x4{0u, 0u, 0u, 0u};
      if (d[j] >= 0) r[j] = load_stream(rows + (int64_t)d[j] * V + v);
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (d[j] < 0) continue;
      float f[8];
      unpack8(r[j], f);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = WEIGHTED ? __builtin_fmaf(wj[j], f[c], acc[c]) : acc[c] + f[c];
    }
    if constexpr (OUT_F32) {
      f32x4 *o = reinterpret_cast<f32x4 *>(out) + (t * V + v) * 2;
      const f32x4 lo4{acc[0], acc[1], acc[2], acc[3]}, hi4{acc[4], acc[5], acc[6], acc[7]};
      if constexpr (NT) {
        store_stream(o, lo4);
        store_stream(o + 1, hi4);
      } else {
        o[0] = lo4;
        o[1] = hi4;
      }
    } else {
      u32x4 *o = reinterpret_cast<u32x4 *>(out) + t * V + v;
      if constexpr (NT) store_stream(o, pack8(acc));
      else *o = pack8(acc);
    }
  }
}

// grad_expert_out[d] = bf16(w * gy) exactly rounded; grad_w[t, j] = <gy, out[d]>
// reduced over the workgroup in a fixed order (deterministic).
template <int K>
__global__ __launch_bounds__(kRowThreads) void k_combine_bwd(const u32x4 *__restrict__ gy,
                                                             const u32x4 *__restrict__ out,
                                                             const int32_t *__restrict__ dst,
                                                             const float *__restrict__ w,
                                                             u32x4 *__restrict__ gout,
                                                             float *__restrict__ gw, int64_t nrows,
                                                             int32_t V, int32_t kr) {
  constexpr int KN = K > 0 ? K : kMaxTopK;
  __shared__ float red[kRowThreads / 64][KN];
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  int32_t d[KN];
  float wj[KN], dot[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    const bool on = K > 0 || j < k;
    d[j] = on ? dst[t * k + j] : -1;
    if (d[j] >= nrows) d[j] = -1;
    wj[j] = on ? w[t * k + j] : 0.0f;
    dot[j] = 0.0f;
  }
  for (int32_t v = threadIdx.x; v < V; v += kRowThreads) {
    float g[8];
    unpack8(load_stream(gy + t * V + v), g);
    u32x4 r[KN];
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      r[j] = u32x4{0u, 0u, 0u, 0u};
      if (d[j] >= 0) r[j] = load_stream(out + (int64_t)d[j] * V + v);
    }
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (d[j] < 0) continue;
      float o[8];
      unpack8(r[j], o);
#pragma unroll
      for (int c = 0; c < 8; ++c) dot[j] = __builtin_fmaf(g[c], o[c], dot[j]);
      u32x4 p;
      p.x = bf16_of_product(wj[j], g[0]) | (bf16_of_product(wj[j], g[1]) << 16);
      p.y = bf16_of_product(wj[j], g[2]) | (bf16_of_product(wj[j], g[3]) << 16);
      p.z = bf16_of_product(wj[j], g[4]) | (bf16_of_product(wj[j], g[5]) << 16);
      p.w = bf16_of_product(wj[j], g[6]) | (bf16_of_product(wj[j], g[7]) << 16);
      store_stream(gout + (int64_t)d[j] * V + v, p);
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    float s = dot[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) red[wv][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowThreads / 64; ++i) s += red[i][j];
    gw[t * k + j] = dst[t * k + j] >= 0 ? s : 0.0f;
  }
}

hipError_t launch_combine(const Geometry &g, const Workspace &ws, const uint16_t *rows,
                          int32_t H, const float *topk_w, void *out, bool out_fp32,
                          hipStream_t s) {
  if (g.T == 0) return hipSuccess;
  const int32_t V = H / 8;
  const u32x4 *r = reinterpret_cast<const u32x4 *>(rows);
  int32_t chunk = V;
  const int32_t pieces = row_pieces(g.T, V, &chunk);
  const bool nt = g.cstores == 2;
#define L5(KK, WT, OF, NT)                                                                        \
  hipLaunchKernelGGL((k_combine<KK, WT, OF, NT>), dim3(g.T, pieces), dim3(kRowThreads), 0, s, r, \
                     ws.dst, topk_w, out, g.rows, V, g.k, chunk)
#define L4(KK, WT, OF)         \
  do {                         \
    if (nt) L5(KK, WT, OF, true); \
    else L5(KK, WT, OF, false);   \
  } while (0)
#define L(KK)                           \
  do {                                  \
    if (topk_w) {                       \
      if (out_fp32) L4(KK, true, true); \
      else L4(KK, true, false);         \
    } else {                            \
      if (out_fp32) L4(KK, false, true);\
      else L4(KK, false, false);        \
    }                                   \
  } while (0)
  EP_K_SWITCH(g.k, L)
#undef L
#undef L4
#undef L5
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const Geometry &g, const Workspace &ws, const uint16_t *gy,
                              const uint16_t *expert_out, int32_t H, const float *topk_w,
                              uint16_t *grad_out, float *grad_w, hipStream_t s) {
  if (g.T == 0) return hipSuccess;
  const int32_t V = H / 8;
#define L(KK)                                                                            \
  hipLaunchKernelGGL(k_combine_bwd<KK>, dim3(g.T), dim3(kRowThreads), 0, s,             \
                     reinterpret_cast<const u32x4 *>(gy),                               \
                     reinterpret_cast<const u32x4 *>(expert_out), ws.dst, topk_w,       \
                     reinterpret_cast<u32x4 *>(grad_out), grad_w, g.rows, V, g.k)
  EP_K_SWITCH(g.k, L)
#undef L
  return hipGetLastError();
}

}  // namespace epk
