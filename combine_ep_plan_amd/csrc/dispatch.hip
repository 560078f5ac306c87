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
//
// Fused layout (ep_plan_dispatch, LL and HT, at most one layout tile of
// entries): the layout and the dispatch in one launch.  Every token's
// workgroup places its own k entries: over all n <= 2048 ids (a few KB, read
// from L2 by every workgroup), one ballot per entry and chunk of 64 ids counts
// the earlier entries of the same expert (its position) and, for HT, the
// entries of lower experts (its expert's offset); the first piece of each
// token writes dst, eidx and recv_src.  One extra workgroup writes the counts
// (LDS histogram), offsets (workgroup scan), flags and status word.  Same
// tables, bit for bit, as ep_plan's layout kernel, one launch fewer.
#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kRowThreads = 512;
constexpr int kUnroll = 2;
constexpr int64_t kCachedStoreBytes = (int64_t)512 << 20;  // twice the Infinity Cache
constexpr int64_t kCachedStoreMin = (int64_t)64 << 20;     // below: latency-bound

// The size rule of the default store choice: cached between 64 MiB and
// 512 MiB of rows written by one dispatch, the rows of every pass in flight
// counted against the upper bound (they share the cache).
static bool streaming_stores(int32_t stores, int64_t bytes, int32_t in_flight) {
  if (stores != 0) return stores == 2;
  return bytes <= kCachedStoreMin || bytes * (in_flight > 1 ? in_flight : 1) > kCachedStoreBytes;
}

// Pieces per row: small batches (decode) split each row over several
// workgroups, so the grid reaches about kSplitTarget workgroups; pieces are
// whole 128-channel blocks (16 vectors), as FP8 scales need.
constexpr int64_t kSplitTarget = 1024;

// The fused layout places a token's entries once per piece, so it splits rows
// only below this many tokens (a decode batch of 128 tokens keeps whole rows:
// 129 workgroups measured faster than 257, 513 or 1025).
constexpr int64_t kFusedSplitTarget = 128;

static int32_t row_pieces_to(int32_t T, int32_t V, int32_t *chunk, int64_t target) {
  int64_t want = T > 0 ? (target + T - 1) / T : 1;
  const int64_t most = (V + 15) / 16;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int32_t c = (int32_t)((V + want - 1) / want);
  c = (c + 15) / 16 * 16;
  *chunk = c;
  return (V + c - 1) / c;
}

int32_t row_pieces(int32_t T, int32_t V, int32_t *chunk) {
  return row_pieces_to(T, V, chunk, kSplitTarget);
}

constexpr int kRowWaves = kRowThreads / 64;

// Tables the fused layout reads and writes.
struct FusedLayout {
  const int32_t *idx;  // top-k ids [T, k]
  Geometry g;
  Workspace ws;
};

// Destinations of token t's k entries into s_dst (every thread of the
// workgroup takes part; ends with a barrier).  The first piece of the row
// also writes dst, eidx and recv_src for them.
template <int K>
__device__ void fused_place(const FusedLayout &fl, int64_t t, int32_t *s_dst,
                            uint32_t (*s_cnt)[2][kMaxTopK]) {
  const Geometry &g = fl.g;
  constexpr int KN = K > 0 ? K : kMaxTopK;
  const int32_t k = K > 0 ? K : g.k;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t n = (int32_t)g.n;
  const bool ht = g.layout == kHT;
  int32_t ej[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    const int32_t raw = (K > 0 || j < k) ? fl.idx[t * k + j] : -1;
    ej[j] = raw >= 0 && raw < g.E ? raw : -1;
  }
  uint32_t pos[KN], less[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) pos[j] = less[j] = 0;
  // chunks of 64 ids, wave w takes chunks w, w + waves, ...; all loads
  // first.  LL positions depend only on earlier entries, so the ids past the
  // token's own are not read; HT offsets count every entry.
  const int32_t n_read = ht ? n : (int32_t)((t + 1) * k);
  constexpr int kChunksPerWave = kTileEntries / 64 / kRowWaves;
  int32_t id[kChunksPerWave];
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int32_t f = (w + c * kRowWaves) * 64 + lane;
    id[c] = f < n_read ? fl.idx[f] : -1;
  }
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    if ((w + c * kRowWaves) * 64 >= n_read) break;   // wave-uniform
    const int32_t f = (w + c * kRowWaves) * 64 + lane;
    const bool valid = id[c] >= 0 && id[c] < g.E;
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (K > 0 || j < k) {   // a guard, not a break: the loop unrolls fully
        const int64_t fj = t * k + j;
        pos[j] += __popcll(__ballot(valid && id[c] == ej[j] && f < fj));
        if (ht) less[j] += __popcll(__ballot(valid && id[c] < ej[j]));
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (K > 0 || j < k) {
        s_cnt[w][0][j] = pos[j];
        s_cnt[w][1][j] = less[j];
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < k) {
    const int j = threadIdx.x;
    const int32_t e = fl.idx[t * k + j];
    const bool valid = e >= 0 && e < g.E;
    int32_t p = 0, lt = 0;
#pragma unroll
    for (int i = 0; i < kRowWaves; ++i) {
      p += (int32_t)s_cnt[i][0][j];
      lt += (int32_t)s_cnt[i][1][j];
    }
    int32_t d = -1;
    if (valid) d = ht ? lt + p : (p < g.cap ? e * g.cap + p : -1);
    if (d >= g.rows) d = -1;
    s_dst[j] = d;
    if (blockIdx.y == 0) {
      const int64_t f = t * k + j;
      fl.ws.eidx[f] = valid ? e : -1;
      fl.ws.dst[f] = d;
      if (d >= 0) fl.ws.recv_src[d] = (int32_t)f;
    }
  }
  __syncthreads();
}

// The fused layout's table workgroup: counts (LDS histogram), offsets
// (workgroup scan, E <= 2 * kRowThreads), the index-range and capacity flags
// and the status word.
__device__ void fused_tables(const FusedLayout &fl, int32_t *s_hist, int32_t *s_wsum,
                             uint32_t *s_flags) {
  const Geometry &g = fl.g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t E = g.E, n = (int32_t)g.n;
  for (int e = tid; e < E; e += kRowThreads) s_hist[e] = 0;
  if (tid == 0) *s_flags = 0;
  __syncthreads();
  uint32_t flags = 0;
  for (int32_t f = tid; f < n; f += kRowThreads) {
    const int32_t id = fl.idx[f];
    if (id >= 0 && id < E) atomicAdd(&s_hist[id], 1);
    else if (id != -1) flags |= kFlagIndexRange;
  }
  if (flags) atomicOr(s_flags, flags);
  __syncthreads();
  // two experts per thread, a DPP scan per wave, then the wave totals
  const int32_t e0 = 2 * tid;
  const int32_t v0 = e0 < E ? s_hist[e0] : 0, v1 = e0 + 1 < E ? s_hist[e0 + 1] : 0;
  const int32_t sum = v0 + v1;
  int32_t incl = sum;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int32_t pre = 0;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) pre += i < w ? s_wsum[i] : 0;
  const int32_t ex = pre + incl - sum;
  uint32_t cap = 0;
  if (e0 < E) {
    fl.ws.counts[e0] = v0;
    fl.ws.offsets[e0] = ex;
    if (g.layout == kLL && v0 > g.cap) cap = kFlagCapacity;
  }
  if (e0 + 1 < E) {
    fl.ws.counts[e0 + 1] = v1;
    fl.ws.offsets[e0 + 1] = ex + v0;
    if (g.layout == kLL && v1 > g.cap) cap = kFlagCapacity;
  }
  if (e0 < E && e0 + 2 >= E) fl.ws.offsets[E] = ex + sum;   // the thread holding the last expert
  if (cap) atomicOr(s_flags, cap);
  __syncthreads();
  if (tid == 0) *fl.ws.status = *s_flags;
}

// The fused launch's table workgroup (the last block column): counts,
// offsets, flags and the status word.
__device__ void fused_table_block(const FusedLayout &fl) {
  __shared__ int32_t s_hist[kMaxExperts];
  __shared__ int32_t s_wsum[kRowWaves];
  __shared__ uint32_t s_flags;
  if (blockIdx.y == 0) fused_tables(fl, s_hist, s_wsum, &s_flags);
}

// The k destinations of the workgroup's token: from the plan's dst table, or
// (FUSED) placed here.
template <int K, bool FUSED>
__device__ __forceinline__ void token_dst(const int32_t *__restrict__ dst, int64_t t, int32_t k,
                                          const FusedLayout &fl,
                                          int32_t (&d)[K > 0 ? K : kMaxTopK]) {
  constexpr int KN = K > 0 ? K : kMaxTopK;
  if constexpr (FUSED) {
    __shared__ int32_t s_dst[kMaxTopK];
    __shared__ uint32_t s_cnt[kRowWaves][2][kMaxTopK];
    fused_place<K>(fl, t, s_dst, s_cnt);
#pragma unroll
    for (int j = 0; j < KN; ++j) d[j] = (K > 0 || j < k) ? s_dst[j] : -1;
  } else {
#pragma unroll
    for (int j = 0; j < KN; ++j) d[j] = (K > 0 || j < k) ? dst[t * k + j] : -1;
  }
}

template <int K, bool NT, bool FUSED>
__global__ __launch_bounds__(kRowThreads) void k_dispatch_bf16(const u32x4 *__restrict__ x,
                                                               const int32_t *__restrict__ dst,
                                                               u32x4 *__restrict__ recv,
                                                               int64_t rows, int32_t V,
                                                               int32_t kr, int32_t chunk,
                                                               FusedLayout fl) {
  constexpr int KN = K > 0 ? K : kMaxTopK;
  if constexpr (FUSED) {
    if (blockIdx.x == gridDim.x - 1) {
      fused_table_block(fl);
      return;
    }
  }
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  const u32x4 *xr = x + t * V;
  const int32_t lo = blockIdx.y * chunk;
  const int32_t hi = lo + chunk < V ? lo + chunk : V;
  // the row's first vectors are in flight while the destinations are found
  int32_t v0 = lo + threadIdx.x;
  u32x4 val[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int32_t v = v0 + u * kRowThreads;
    if (v < hi) val[u] = xr[v];
  }
  int32_t d[KN];
  token_dst<K, FUSED>(dst, t, k, fl, d);
  while (v0 < hi) {
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (K == 0 && j >= k) break;
      if (d[j] < 0 || d[j] >= rows) continue;
      u32x4 *o = recv + (int64_t)d[j] * V;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t v = v0 + u * kRowThreads;
        if (v < hi) {
          if constexpr (NT) store_stream(o + v, val[u]);
          else o[v] = val[u];
        }
      }
    }
    v0 += kRowThreads * kUnroll;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t v = v0 + u * kRowThreads;
      if (v < hi) val[u] = xr[v];
    }
  }
}

// FP8 quantisation of one 16-byte vector (8 bf16 channels) whose 128-channel
// block spans 16 consecutive lanes: amax reduced over those lanes, scale =
// amax / 448 and x / scale IEEE fp32 divisions, the quotient clamped to +-448
// and rounded to nearest even by v_cvt_pk_fp8_f32 (OCP e4m3fn on gfx950).
// pow2: the scale is rounded up to a power of two (at least 2^-126), so that
// it is an 8-bit exponent the grouped GEMM's matrix cores can apply.
// Returns the 8 codes; *scale gets the block's scale.
__device__ __forceinline__ u32x2 quantize_fp8_vec(u32x4 xv, float *scale, bool pow2) {
  float f[8];
  unpack8(xv, f);
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(f[c]));
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  float s = amax == 0.0f ? 1.0f : amax / 448.0f;
  if (pow2 && amax != 0.0f) {
    uint32_t b = __float_as_uint(s);
    if (b < 0x00800000u) b = 0x00800000u;                                  // 2^-126
    else if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;         // next power of two
    s = __uint_as_float(b);
  }
  float q[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) q[c] = fminf(fmaxf(f[c] / s, -448.0f), 448.0f);
  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
  *scale = s;
  return u32x2{w0, w1};
}

// FP8 dispatch: each token's row quantised once (quantize_fp8_vec) and the
// codes and scales written to its k destinations.
template <int K, bool NT, bool FUSED>
__global__ __launch_bounds__(kRowThreads) void k_dispatch_fp8(const u32x4 *__restrict__ x,
                                                              const int32_t *__restrict__ dst,
                                                              u32x2 *__restrict__ recv_q,
                                                              float *__restrict__ recv_s,
                                                              int64_t rows, int32_t V,
                                                              int32_t kr, int32_t chunk,
                                                              FusedLayout fl) {
  constexpr int KN = K > 0 ? K : kMaxTopK;
  if constexpr (FUSED) {
    if (blockIdx.x == gridDim.x - 1) {
      fused_table_block(fl);
      return;
    }
  }
  const int64_t t = blockIdx.x;
  const int32_t k = K > 0 ? K : kr;
  const int32_t nb = V >> 4;
  // pieces are whole 16-vector blocks, so a block's 16 lanes are all in or all out
  const int32_t lo = blockIdx.y * chunk;
  const int32_t hi = lo + chunk < V ? lo + chunk : V;
  // the row's first vector is in flight while the destinations are found
  u32x4 xv = u32x4{0u, 0u, 0u, 0u};
  if (lo + (int32_t)threadIdx.x < hi) xv = x[t * V + lo + threadIdx.x];
  int32_t d[KN];
  token_dst<K, FUSED>(dst, t, k, fl, d);
  for (int32_t v = lo + threadIdx.x; v < hi; v += kRowThreads) {
    const u32x4 cur = xv;
    if (v + kRowThreads < hi) xv = x[t * V + v + kRowThreads];
    float s;
    const u32x2 packed = quantize_fp8_vec(cur, &s, fl.g.fp8_pow2 == 1);
#pragma unroll
    for (int j = 0; j < KN; ++j) {
      if (K == 0 && j >= k) break;
      if (d[j] < 0 || d[j] >= rows) continue;
      if constexpr (NT) store_stream(recv_q + (int64_t)d[j] * V + v, packed);
      else recv_q[(int64_t)d[j] * V + v] = packed;
      if ((v & 15) == 0) recv_s[(int64_t)d[j] * nb + (v >> 4)] = s;
    }
  }
}

// Rows of bf16 (K % 128 == 0) to e4m3 codes and one fp32 scale per 128, the
// FP8 dispatch's recipe (quantize_fp8_vec), for rows that do not come from
// a dispatch -- the activation between the expert FFN's two GEMMs.  A grid
// stride over the 16-byte vectors; 16 consecutive vectors are one block, so
// a block's lanes are all in or all out of a pass (the stride is a multiple
// of 16 and the vector count is too).
__global__ __launch_bounds__(256) void k_quantize_fp8(const u32x4 *__restrict__ x,
                                                      u32x2 *__restrict__ q,
                                                      float *__restrict__ scales, int64_t nvec,
                                                      bool pow2) {
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * 256) {
    float s;
    const u32x2 codes = quantize_fp8_vec(x[v], &s, pow2);
    q[v] = codes;
    if ((v & 15) == 0) scales[v >> 4] = s;
  }
}

hipError_t launch_quantize_fp8(const uint16_t *x, int64_t rows, int32_t K, uint8_t *q,
                               float *scales, bool pow2, hipStream_t s) {
  const int64_t nvec = rows * (K / 8);
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_quantize_fp8, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(x), reinterpret_cast<u32x2 *>(q), scales,
                     nvec, pow2);
  return hipGetLastError();
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

// The fused layout serves LL and HT batches of at most one layout tile.
bool fused_layout_fits(const Geometry &g) {
  return (g.layout == kLL || g.layout == kHT) && g.n <= kTileEntries;
}

// fused == false: dst from the plan.  fused == true: the layout too (one
// extra block column writes the tables; T == 0 launches only that).
hipError_t launch_dispatch_bf16(const Geometry &g, const Workspace &ws, const uint16_t *x,
                                int32_t H, uint16_t *recv, hipStream_t s, const int32_t *idx,
                                bool fused) {
  if (g.T == 0 && !fused) return hipSuccess;
  const int32_t V = H / 8;
  int32_t chunk = V;
  const int32_t pieces = row_pieces_to(g.T, V, &chunk, fused ? kFusedSplitTarget : kSplitTarget);
  const bool nt = streaming_stores(g.stores, g.n * H * 2, g.in_flight);
  const FusedLayout fl{idx, g, ws};
  const unsigned gx = (unsigned)g.T + (fused ? 1u : 0u);
#define L3(KK, NT, FU)                                                                 \
  hipLaunchKernelGGL((k_dispatch_bf16<KK, NT, FU>), dim3(gx, pieces), dim3(kRowThreads), 0, s, \
                     reinterpret_cast<const u32x4 *>(x), ws.dst,                      \
                     reinterpret_cast<u32x4 *>(recv), g.rows, V, g.k, chunk, fl)
#define L2(KK, NT)                    \
  do {                                \
    if (fused) L3(KK, NT, true);      \
    else L3(KK, NT, false);           \
  } while (0)
#define L(KK)               \
  do {                      \
    if (nt) L2(KK, true);   \
    else L2(KK, false);     \
  } while (0)
  EP_K_SWITCH(g.k, L)
#undef L
#undef L2
#undef L3
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const Geometry &g, const Workspace &ws, const uint16_t *x,
                               int32_t H, uint8_t *recv_q, float *recv_scale, hipStream_t s,
                               const int32_t *idx, bool fused) {
  if (g.T == 0 && !fused) return hipSuccess;
  const int32_t V = H / 8;
  int32_t chunk = V;
  const int32_t pieces = row_pieces_to(g.T, V, &chunk, fused ? kFusedSplitTarget : kSplitTarget);
  const bool nt = streaming_stores(g.stores, g.n * (H + H / 128 * 4), g.in_flight);
  const FusedLayout fl{idx, g, ws};
  const unsigned gx = (unsigned)g.T + (fused ? 1u : 0u);
#define L3(KK, NT, FU)                                                                 \
  hipLaunchKernelGGL((k_dispatch_fp8<KK, NT, FU>), dim3(gx, pieces), dim3(kRowThreads), 0, s, \
                     reinterpret_cast<const u32x4 *>(x), ws.dst,                      \
                     reinterpret_cast<u32x2 *>(recv_q), recv_scale, g.rows, V,        \
                     g.k, chunk, fl)
#define L2(KK, NT)                    \
  do {                                \
    if (fused) L3(KK, NT, true);      \
    else L3(KK, NT, false);           \
  } while (0)
#define L(KK)               \
  do {                      \
    if (nt) L2(KK, true);   \
    else L2(KK, false);     \
  } while (0)
  EP_K_SWITCH(g.k, L)
#undef L
#undef L2
#undef L3
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
