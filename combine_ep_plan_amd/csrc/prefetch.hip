// prefetch.hip -- replica-weight prefetch (MoonEP article, paragraphs 3 and
// 5): after the static-shape plan picks redundant experts, each receiving
// rank's prefetch slots are filled with a copy of those experts' weights,
// one contiguous row of bytes per expert projection.
//
// The slots to fill are known only on the device (the plan's segment table
// and seg_slot), so the grid has a fixed size.  Every workgroup first
// compacts the filled slots into LDS (segment i with seg_slot[i] = s >= 0
// gives source expert segments[i][0] and destination slot
// segments[i][1] * S + s; at most E + R of them), then walks the
// (slot, chunk) pairs with a grid stride.  Each chunk is 512 lanes x 4
// vectors: all loads issue before any store, a wave covers 64 contiguous
// vectors.  Rows that are a multiple of 16 bytes move in 16-byte vectors
// (32 KB chunks); other rows (a multiple of 4 bytes, such as the fp32 scale
// rows of FP8 weights) in 4-byte words.  Distinct segments name distinct
// slots, so no two workgroups write the same bytes.
#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kPrefetchThreads = 512;
constexpr int kPrefetchUnroll = 4;
constexpr int kPrefetchMaxBlocks = 2048;

template <typename V>
constexpr int64_t prefetch_chunk() { return (int64_t)kPrefetchThreads * kPrefetchUnroll * sizeof(V); }

template <typename V>
__global__ __launch_bounds__(kPrefetchThreads) void k_prefetch(
    const uint8_t *__restrict__ weights, uint8_t *__restrict__ slots,
    const int32_t *__restrict__ segments, const int32_t *__restrict__ seg_slot,
    const int32_t *__restrict__ n_segments, int32_t max_segments, int32_t E, int32_t R,
    int32_t S, int64_t row_bytes) {
  __shared__ int32_t s_src[kMaxExperts * 2];   // E + R <= 2 * kMaxExperts
  __shared__ int32_t s_dst[kMaxExperts * 2];
  __shared__ int32_t s_wave[kPrefetchThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t ns = *n_segments;
  ns = ns < 0 ? 0 : (ns > max_segments ? max_segments : ns);

  // Compact the filled slots, in segment order.
  int32_t nfill = 0;
  for (int32_t c0 = 0; c0 < ns; c0 += kPrefetchThreads) {
    const int32_t i = c0 + tid;
    int32_t e = -1, r = -1, sl = -1;
    if (i < ns) {
      sl = seg_slot[i];
      e = segments[(int64_t)i * 5 + 0];
      r = segments[(int64_t)i * 5 + 1];
    }
    const bool f = sl >= 0 && sl < S && e >= 0 && e < E && r >= 0 && r < R;
    const uint64_t b = __ballot(f);
    if (lane == 0) s_wave[w] = __popcll(b);
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kPrefetchThreads / 64; ++v) {
      before += v < w ? s_wave[v] : 0;
      total += s_wave[v];
    }
    if (f) {
      const int32_t at = nfill + before + __popcll(b & ((1ull << lane) - 1ull));
      s_src[at] = e;
      s_dst[at] = r * S + sl;
    }
    nfill += total;
    __syncthreads();
  }

  constexpr int64_t kChunk = prefetch_chunk<V>();
  const int64_t cpr = (row_bytes + kChunk - 1) / kChunk;  // chunks per row
  const int64_t work = (int64_t)nfill * cpr;
  for (int64_t q = blockIdx.x; q < work; q += gridDim.x) {
    const int32_t j = (int32_t)(q / cpr);
    const int64_t off = (q - (int64_t)j * cpr) * kChunk;
    const int64_t bytes = row_bytes - off < kChunk ? row_bytes - off : kChunk;
    const V *src = reinterpret_cast<const V *>(weights + (int64_t)s_src[j] * row_bytes + off);
    V *dst = reinterpret_cast<V *>(slots + (int64_t)s_dst[j] * row_bytes + off);
    const int32_t nv = (int32_t)(bytes / (int64_t)sizeof(V));
    V v[kPrefetchUnroll];
#pragma unroll
    for (int u = 0; u < kPrefetchUnroll; ++u) {
      const int32_t x = u * kPrefetchThreads + tid;
      if (x < nv) v[u] = load_stream(src + x);
    }
#pragma unroll
    for (int u = 0; u < kPrefetchUnroll; ++u) {
      const int32_t x = u * kPrefetchThreads + tid;
      if (x < nv) store_stream(dst + x, v[u]);
    }
  }
}

hipError_t launch_prefetch(const Geometry &g, const Workspace &ws, const uint8_t *weights,
                           int64_t row_bytes, uint8_t *slots, hipStream_t s) {
  if ((int64_t)g.R * g.S == 0 || row_bytes == 0) return hipSuccess;
  const int32_t max_segments = g.E + g.R;
  const bool wide = row_bytes % 16 == 0;
  const int64_t chunk = wide ? prefetch_chunk<u32x4>() : prefetch_chunk<uint32_t>();
  const int64_t cpr = (row_bytes + chunk - 1) / chunk;
  // no more slots can be filled than segments, nor than slots
  const int64_t most = (int64_t)(max_segments < g.R * g.S ? max_segments : g.R * g.S) * cpr;
  const unsigned blocks = (unsigned)(most < kPrefetchMaxBlocks ? most : kPrefetchMaxBlocks);
  if (wide)
    hipLaunchKernelGGL(k_prefetch<u32x4>, dim3(blocks), dim3(kPrefetchThreads), 0, s, weights,
                       slots, ws.segments, ws.seg_slot, ws.n_segments, max_segments, g.E, g.R,
                       g.S, row_bytes);
  else
    hipLaunchKernelGGL(k_prefetch<uint32_t>, dim3(blocks), dim3(kPrefetchThreads), 0, s, weights,
                       slots, ws.segments, ws.seg_slot, ws.n_segments, max_segments, g.E, g.R,
                       g.S, row_bytes);
  return hipGetLastError();
}

}  // namespace epk
