// dispatch.hip -- token rows to their expert-grouped receive rows on gfx950
// (MoonEP article, paragraph 4: straight into the final position, no
// staging buffer; NCCL EP paper listing, Table III layouts), optionally
// quantised to FP8 e4m3 with one fp32 scale per 128 channels (NCCL EP
// listing, Table IV: FP8 scales travel with the tokens).
//
// One workgroup per token (per piece of a token's row when there are too
// few tokens to fill the GPU): the row is read once with 16-byte loads and
// written to each of its k destinations with 16-byte stores, so x costs one
// HBM read and every receive row one HBM write.  By default the stores are
// cached while the rows written fit in twice the 256 MB Infinity Cache (the
// next kernel then finds much of them there) and non-temporal beyond that,
// where cached stores only leave write-backs for the next kernel to pay;
// below 64 MiB the dispatch is latency-bound and writing its dirty lines
// back at the kernel's end costs more than the cache saves, so small batches
// stream too.  The group's configuration can fix either kind.
#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kRowThreads = 512;
constexpr int kUnroll = 2;
constexpr int64_t kCachedStoreBytes = (int64_t)512 << 20;  // twice the Infinity Cache
constexpr int64_t kCachedStoreMin = (int64_t)64 << 20;     // below: latency-bound

// The size rule of the default store choice: cached between 64 MiB and
// 512 MiB of rows written.
static bool streaming_stores(int32_t stores, int64_t bytes) {
  if (stores != 0) return stores == 2;
  return bytes <= kCachedStoreMin || bytes > kCachedStoreBytes;
}

// Pieces per row: small batches (decode) split each row over several
// workgroups, so the grid reaches about kSplitTarget workgroups; pieces are
// whole 128-channel blocks (16 vectors), as FP8 scales need.
constexpr int64_t kSplitTarget = 1024;

int32_t row_pieces(int32_t T, int32_t V, int32_t *chunk) {
  int64_t want = T > 0 ? (kSplitTarget + T - 1) / T : 1;
  const int64_t most = (V + 15) / 16;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int32_t c = (int32_t)((V + want - 1) / want);
  c = (c + 15) / 16 * 16;
  *chunk = c;
  return (V + c - 1) / c;
}

template <int K, bool NT>
__global__ __launch_bounds__(kRowThreads) void k_dispatch_bf16(const u32x4 *__restrict__ x,
                                                               const int32_t *__restrict__ dst,
                                                               u32x4 *__restrict__ recv,
                                                               int64_t rows, int32_t V,
                                                               int32_t kr, int32_t chunk) {
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  const int32_t *dt = dst + t * k;
  const u32x4 *xr = x + t * V;
  const int32_t lo = blockIdx.y * chunk;
  const int32_t hi = lo + chunk < V ? lo + chunk : V;
  for (int32_t v0 = lo + threadIdx.x; v0 < hi; v0 += kRowThreads * kUnroll) {
    u32x4 val[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t v = v0 + u * kRowThreads;
      if (v < hi) val[u] = xr[v];
    }
#pragma unroll
    for (int j = 0; j < (K > 0 ? K : kMaxTopK); ++j) {
      if (K == 0 && j >= k) break;
      const int32_t d = dt[j];
      if (d < 0 || d >= rows) continue;
      u32x4 *o = recv + (int64_t)d * V;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t v = v0 + u * kRowThreads;
        if (v < hi) {
          if constexpr (NT) store_stream(o + v, val[u]);
          else o[v] = val[u];
        }
      }
    }
  }
}

// FP8: a 128-channel block is 16 lanes x 8 channels; amax is reduced over
// those 16 lanes.  scale = amax / 448 and x / scale are IEEE fp32 divisions,
// the quotient is clamped to +-448 and rounded to nearest even by
// v_cvt_pk_fp8_f32 (OCP e4m3fn on gfx950).
template <int K, bool NT>
__global__ __launch_bounds__(kRowThreads) void k_dispatch_fp8(const u32x4 *__restrict__ x,
                                                              const int32_t *__restrict__ dst,
                                                              u32x2 *__restrict__ recv_q,
                                                              float *__restrict__ recv_s,
                                                              int64_t rows, int32_t V,
                                                              int32_t kr, int32_t chunk) {
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  const int32_t *dt = dst + t * k;
  const int32_t nb = V >> 4;
  // pieces are whole 16-vector blocks, so a block's 16 lanes are all in or all out
  const int32_t lo = blockIdx.y * chunk;
  const int32_t hi = lo + chunk < V ? lo + chunk : V;
  for (int32_t v = lo + threadIdx.x; v < hi; v += kRowThreads) {
    float f[8];
    unpack8(x[t * V + v], f);
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(f[c]));
    amax = fmaxf(amax, __shfl_xor(amax, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    float q[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) q[c] = fminf(fmaxf(f[c] / s, -448.0f), 448.0f);
    uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
    uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
    const u32x2 packed = {w0, w1};
    for (int j = 0; j < (K > 0 ? K : kMaxTopK); ++j) {
      if (K == 0 && j >= k) break;
      const int32_t d = dt[j];
      if (d < 0 || d >= rows) continue;
      if constexpr (NT) store_stream(recv_q + (int64_t)d * V + v, packed);
      else recv_q[(int64_t)d * V + v] = packed;
      if ((v & 15) == 0) recv_s[(int64_t)d * nb + (v >> 4)] = s;
    }
  }
}

// Per receive row: expert id and router weight of the entry it holds (-1 / 0
// for rows no entry maps to: past offsets[E] in HT, past min(count, cap) in
// an LL expert block, past load[r] in a STATIC rank block).
__global__ __launch_bounds__(256) void k_recv_meta(Geometry g, Workspace ws,
                                                   const float *__restrict__ w,
                                                   int32_t *__restrict__ recv_idx,
                                                   float *__restrict__ recv_w) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= g.rows) return;
  bool used;
  if (g.layout == kHT) {
    used = r < ws.offsets[g.E];
  } else {
    const int32_t len = g.layout == kLL ? g.cap : g.C;
    const int32_t b = (int32_t)r / len, slot = (int32_t)r - b * len;
    const int32_t n = g.layout == kLL ? ws.counts[b] : ws.load[b];
    used = slot < n;
  }
  const int32_t src = used ? ws.recv_src[r] : -1;
  if (recv_idx) recv_idx[r] = src >= 0 ? ws.eidx[src] : -1;
  if (recv_w) recv_w[r] = src >= 0 ? w[src] : 0.0f;
}

hipError_t launch_dispatch_bf16(const Geometry &g, const Workspace &ws, const uint16_t *x,
                                int32_t H, uint16_t *recv, hipStream_t s) {
  if (g.T == 0) return hipSuccess;
  const int32_t V = H / 8;
  int32_t chunk = V;
  const int32_t pieces = row_pieces(g.T, V, &chunk);
  const bool nt = streaming_stores(g.stores, g.n * H * 2);
#define L2(KK, NT)                                                                     \
  hipLaunchKernelGGL((k_dispatch_bf16<KK, NT>), dim3(g.T, pieces), dim3(kRowThreads), 0, s, \
                     reinterpret_cast<const u32x4 *>(x), ws.dst,                      \
                     reinterpret_cast<u32x4 *>(recv), g.rows, V, g.k, chunk)
#define L(KK)               \
  do {                      \
    if (nt) L2(KK, true);   \
    else L2(KK, false);     \
  } while (0)
  EP_K_SWITCH(g.k, L)
#undef L
#undef L2
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const Geometry &g, const Workspace &ws, const uint16_t *x,
                               int32_t H, uint8_t *recv_q, float *recv_scale, hipStream_t s) {
  if (g.T == 0) return hipSuccess;
  const int32_t V = H / 8;
  int32_t chunk = V;
  const int32_t pieces = row_pieces(g.T, V, &chunk);
  const bool nt = streaming_stores(g.stores, g.n * (H + H / 128 * 4));
#define L2(KK, NT)                                                                     \
  hipLaunchKernelGGL((k_dispatch_fp8<KK, NT>), dim3(g.T, pieces), dim3(kRowThreads), 0, s, \
                     reinterpret_cast<const u32x4 *>(x), ws.dst,                      \
                     reinterpret_cast<u32x2 *>(recv_q), recv_scale, g.rows, V,        \
                     g.k, chunk)
#define L(KK)               \
  do {                      \
    if (nt) L2(KK, true);   \
    else L2(KK, false);     \
  } while (0)
  EP_K_SWITCH(g.k, L)
#undef L
#undef L2
  return hipGetLastError();
}

hipError_t launch_recv_meta(const Geometry &g, const Workspace &ws, const float *topk_w,
                            int32_t *recv_idx, float *recv_w, hipStream_t s) {
  if (g.rows == 0) return hipSuccess;
  const int64_t blocks = (g.rows + 255) / 256;
  hipLaunchKernelGGL(k_recv_meta, dim3((unsigned)blocks), dim3(256), 0, s, g, ws, topk_w,
                     recv_idx, recv_w);
  return hipGetLastError();
}

}  // namespace epk
