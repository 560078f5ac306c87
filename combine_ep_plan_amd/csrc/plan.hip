// plan.hip -- layout of one pass on gfx950: per-expert counts, offsets,
// stable destination rows for the LL / HT layouts (NCCL EP paper listing,
// Table III; Figures 3-4) and the static-shape plan (MoonEP article,
// paragraphs 3-5), all on the device with no host round trip (MoonEP
// article, paragraph 4: no per-layer host synchronisation).
//
// k_plan_tiles: one 1024-thread workgroup per tile of 2048 flat entries.
//   Each wave ranks its 128 entries chunk by chunk (64 lanes): lanes with
//   the same expert are found with one ballot per bit of the expert id
//   (multisplit), the rank inside the chunk is the popcount of lower peers,
//   and a per-wave LDS counter per expert carries ranks across chunks.  A
//   per-expert scan over the 16 waves gives ranks inside the tile and the
//   tile histogram.  No atomics touch the ranks, so every output is
//   deterministic.  A single tile keeps its histogram in LDS, needs no
//   handshake and also writes the destinations.
//   Several tiles, all resident at once (no more tiles than compute units):
//   every tile publishes its histogram, waits until all tiles have, and
//   then computes its own per-expert base and the totals from all the
//   histograms, so it writes its destinations in the same launch.  For the
//   static layout every tile also runs the planner on those totals and
//   places its entries from its own copy of the tables in LDS; counts,
//   offsets, flags and the planner's tables are written out by tile 0.  The
//   wait for the histograms is bounded: a tile that runs out of it raises
//   EP_FLAG_PLAN_STALL (the layout is then incomplete) instead of hanging.
//   More tiles than that: the last workgroup to finish (ticket counter)
//   scans the tile histograms into per-tile bases, counts and offsets,
//   raises the flags and runs the planner; then k_plan_dst, one thread per
//   entry, adds the tile base to the tile rank.
// recv_src is written for the rows that hold an entry; which rows those are
// follows from counts (LL), load (STATIC) or offsets[E] (HT).
#include "device.h"
#include "ep_internal.h"
#include "route_impl.h"

namespace epk {

struct PlanArgs {
  Geometry g;
  Workspace ws;
  const int32_t *idx;     // top-k ids [T, k] (read when the layout kernel does not route)
  const float *logits;    // fused routing: router logits [T, E]
  int32_t *idx_out;       // fused routing: top-k ids and weights written here
  float *w_out;
};

// In-place exclusive scan of a[0, n) in LDS by the 64 lanes of the calling
// wave; returns the total to every lane.  Each lane scans a contiguous run
// of ceil(n/64) elements and the lane totals are scanned with shuffles, so
// the scan needs no workgroup barrier (the caller synchronises around it).
__device__ int32_t wave_exclusive_scan(int32_t *a, int32_t n) {
  const int lane = threadIdx.x & 63;
  const int32_t per = (n + 63) >> 6;
  const int32_t beg = lane * per;
  const int32_t end = beg + per < n ? beg + per : n;
  int32_t sum = 0;
  for (int32_t j = beg; j < end; ++j) sum += a[j];
  int32_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int32_t run = incl - sum;
  for (int32_t j = beg; j < end; ++j) {
    const int32_t v = a[j];
    a[j] = run;
    run += v;
  }
  return __shfl(incl, 63);
}

// Largest i in [0, n) with a[i] <= x, for non-decreasing a with a[0] <= x.
__device__ __forceinline__ int32_t last_le(const int32_t *a, int32_t n, int32_t x) {
  int32_t lo = 0, hi = n - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Wait until this wave's global stores have reached L2 (s_waitcnt vmcnt(0);
// lgkmcnt and expcnt fields left at their no-wait maxima).  A workgroup
// barrier on gfx950 does not wait for them, so every wave does this before
// the barrier that precedes a release by one wave of the workgroup.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Receive row of an entry of expert e at position pos among e's entries,
// from the plan tables in global memory (the two-launch layout).
__device__ __forceinline__ int32_t entry_dst(const Geometry &g, const Workspace &ws,
                                             const int32_t *offs, int32_t e, int32_t pos) {
  if (g.layout == kHT) return offs[e] + pos;
  if (g.layout == kLL) return pos < g.cap ? e * g.cap + pos : -1;
  const int32_t m = g.E / g.R;
  const int32_t kp = ws.keep[e];
  if (pos < kp) return (e / m) * g.C + ws.native_row[e] + pos;
  if (ws.seg_count[e] <= 0) return -1;
  int32_t lo = ws.seg_first[e], hi = lo + ws.seg_count[e] - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if (ws.segments[mid * 5 + 2] <= pos) lo = mid;
    else hi = mid - 1;
  }
  const int32_t *s = ws.segments + lo * 5;
  return s[1] * g.C + s[4] + (pos - s[2]);
}

// Static-shape planner, run by one workgroup on the final counts.
//  targets: rank r gets floor(N/R) + (r < N mod R) rows;
//  donors (own rows > target) shed the tail rows of their hottest experts
//  (count descending, id ascending) until they are at target;
//  the shed pieces (donor rank, then walk order) and the receivers' deficits
//  (rank order) are laid end to end; each overlap is one segment, placed in
//  the receiver behind its own rows; a receiver's replica slot of a segment
//  is the segment's rank among the pieces that reach that receiver.  Past
//  the S-th slot a segment has none: an error in training, the direct-read
//  overflow in inference (MoonEP article, par. 5).
// Every phase is parallel over ranks, experts, pieces or segments; the five
// prefix sums are single-wave scans (four of them on four waves at once).
// The planner's tables in LDS (region A of the layout kernel).
struct StaticLds {
  int32_t *tgt, *home, *D;
  int32_t *recv_rank;    // [R] rank of the i-th receiver
  int32_t *rbase;        // [R+1] receiver interval starts
  int32_t *rord;         // [R+1] receivers before r
  int32_t *rshed;        // [R+1] spill base of rank r
  int32_t *rnp;          // [R+1] first piece of rank r
  int32_t *ord;          // [E] hotness order inside the rank; at the end: native row
  int32_t *shed;         // [E]
  int32_t *piece_e;      // [E]
  int32_t *piece_start;  // [E+1]
  int32_t *nseg;         // [E+1] segments of piece p, then first segment; at the end:
                         // start of expert e's piece in the shed sequence
};
__device__ __forceinline__ StaticLds static_lds(int32_t *pl, int32_t E, int32_t R) {
  StaticLds t;
  t.tgt = pl;
  t.home = t.tgt + R;
  t.D = t.home + R;
  t.recv_rank = t.D + R;
  t.rbase = t.recv_rank + R;
  t.rord = t.rbase + R + 1;
  t.rshed = t.rord + R + 1;
  t.rnp = t.rshed + R + 1;
  t.ord = t.rnp + R + 1;
  t.shed = t.ord + E;
  t.piece_e = t.shed + E;
  t.piece_start = t.piece_e + E;
  t.nseg = t.piece_start + E + 1;
  return t;
}

// publish: write the tables to the workspace (one workgroup of a launch);
// every caller ends with the tables entry_dst_static reads in LDS.
__device__ void plan_static(const Geometry &g, const Workspace &ws, const int32_t *cnt,
                            int32_t N, int32_t *pl, int32_t *s_small, uint32_t *s_flags,
                            bool publish) {
  const int tid = threadIdx.x, nt = blockDim.x, w = tid >> 6;
  const int32_t E = g.E, R = g.R, S = g.S, m = E / R;
  const StaticLds L = static_lds(pl, E, R);
  int32_t *tgt = L.tgt, *home = L.home, *D = L.D, *recv_rank = L.recv_rank, *rbase = L.rbase;
  int32_t *rord = L.rord, *rshed = L.rshed, *rnp = L.rnp, *ord = L.ord, *shed = L.shed;
  int32_t *piece_e = L.piece_e, *piece_start = L.piece_start, *nseg = L.nseg;

  for (int r = tid; r < R; r += nt) {
    const int32_t t = N / R + (r < N % R ? 1 : 0);
    int32_t h = 0;
    for (int i = 0; i < m; ++i) h += cnt[r * m + i];
    tgt[r] = t;
    home[r] = h;
    D[r] = h < t ? t - h : 0;
    rbase[r] = D[r];
    rord[r] = D[r] > 0 ? 1 : 0;
    if (publish) ws.load[r] = t;
  }
  if (publish)
    for (int i = tid; i < R * S; i += nt) ws.replica[i] = -1;
  __syncthreads();

  for (int e = tid; e < E; e += nt) {
    const int32_t r = e / m, c = cnt[e];
    int32_t o = 0, before = 0;
    for (int i = 0; i < m; ++i) {
      const int32_t e2 = r * m + i, c2 = cnt[e2];
      const bool hotter = c2 > c || (c2 == c && e2 < e);
      o += hotter ? 1 : 0;
      before += hotter ? c2 : 0;
    }
    const int32_t X = home[r] - tgt[r];
    int32_t s = 0;
    if (X > 0) {
      s = X - before;
      s = s < 0 ? 0 : (s > c ? c : s);
    }
    ord[e] = o;
    shed[e] = s;
    if (publish) ws.keep[e] = c - s;
  }
  __syncthreads();

  if (publish) {
    for (int e = tid; e < E; e += nt) {
      const int32_t r = e / m;
      int32_t row = 0;
      for (int32_t e2 = r * m; e2 < e; ++e2) row += cnt[e2] - shed[e2];
      ws.native_row[e] = row;
      if (shed[e] == 0) {
        ws.seg_first[e] = 0;
        ws.seg_count[e] = 0;
      }
    }
  }
  for (int r = tid; r < R; r += nt) {
    int32_t s = 0, np = 0;
    for (int i = 0; i < m; ++i) {
      const int32_t v = shed[r * m + i];
      s += v;
      np += v > 0 ? 1 : 0;
    }
    rshed[r] = s;
    rnp[r] = np;
  }
  __syncthreads();
  if (w == 0) wave_exclusive_scan(rbase, R);
  else if (w == 1) wave_exclusive_scan(rord, R);
  else if (w == 2) wave_exclusive_scan(rshed, R);
  else if (w == 3) {
    const int32_t np = wave_exclusive_scan(rnp, R);
    if ((tid & 63) == 0) s_small[0] = np;
  }
  __syncthreads();
  const int32_t npieces = s_small[0];

  for (int r = tid; r < R; r += nt)
    if (D[r] > 0) recv_rank[rord[r]] = r;
  for (int e = tid; e < E; e += nt) {
    if (shed[e] == 0) continue;
    const int32_t r = e / m;
    int32_t within = 0, cb = 0;
    for (int i = 0; i < m; ++i) {
      const int32_t e2 = r * m + i;
      if (shed[e2] > 0 && ord[e2] < ord[e]) {
        within += shed[e2];
        ++cb;
      }
    }
    const int32_t p = rnp[r] + cb;
    piece_e[p] = e;
    piece_start[p] = rshed[r] + within;
  }
  __syncthreads();

  for (int p = tid; p < npieces; p += nt) {
    const int32_t e = piece_e[p], a0 = piece_start[p], b0 = a0 + shed[e];
    const int32_t rlo = last_le(rbase, R, a0), rhi = last_le(rbase, R, b0 - 1);
    nseg[p] = rord[rhi] - rord[rlo] + 1;
  }
  __syncthreads();
  if (w == 0) {
    const int32_t ns = wave_exclusive_scan(nseg, npieces);
    if ((tid & 63) == 0) {
      s_small[1] = ns;
      if (publish) *ws.n_segments = ns;
    }
  }
  __syncthreads();
  const int32_t nsegs = s_small[1];

  if (publish) {
    for (int p = tid; p < npieces; p += nt) {
      const int32_t e = piece_e[p];
      ws.seg_first[e] = nseg[p];
      ws.seg_count[e] = (p + 1 < npieces ? nseg[p + 1] : nsegs) - nseg[p];
    }
  }
  // one thread per segment: its piece, its receiver, its rows and its slot
  for (int sid = tid; sid < nsegs; sid += nt) {
    const int32_t p = last_le(nseg, npieces, sid);
    const int32_t e = piece_e[p], a0 = piece_start[p], b0 = a0 + shed[e];
    const int32_t r = recv_rank[rord[last_le(rbase, R, a0)] + (sid - nseg[p])];
    const int32_t lo = a0 > rbase[r] ? a0 : rbase[r];
    const int32_t hi = b0 < rbase[r] + D[r] ? b0 : rbase[r] + D[r];
    const int32_t slot = p - last_le(piece_start, npieces, rbase[r]);
    if (publish) {
      int32_t *sg = ws.segments + (int64_t)sid * 5;
      sg[0] = e;
      sg[1] = r;
      sg[2] = (cnt[e] - shed[e]) + (lo - a0);
      sg[3] = hi - lo;
      sg[4] = home[r] + (lo - rbase[r]);
      ws.seg_slot[sid] = slot < S ? slot : -1;
      if (slot < S) ws.replica[r * S + slot] = e;
    }
    if (slot >= S && g.slot_mode == 0) atomicOr(s_flags, kFlagSlotBudget);  // inference: direct read
  }
  // The tables the destinations need, in arrays no phase reads any more:
  // ord[e] = expert e's first row among its rank's own rows, nseg[e] = where
  // e's shed rows start in the sequence of all shed rows.
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    const int32_t r = e / m;
    int32_t row = 0;
    for (int32_t e2 = r * m; e2 < e; ++e2) row += cnt[e2] - shed[e2];
    ord[e] = row;
  }
  for (int p = tid; p < npieces; p += nt) nseg[piece_e[p]] = piece_start[p];
}

// Receive row of an entry of expert e at position pos among e's entries,
// static layout, from the planner's tables in LDS (after plan_static and a
// barrier).  The first keep = cnt - shed entries stay on e's rank, after
// the rows the rank keeps for its lower-numbered experts; entry keep + i is
// entry i of e's piece of the shed sequence, which lands on the receiver
// whose deficit interval holds it, after that receiver's own rows.
__device__ __forceinline__ int32_t entry_dst_static(const Geometry &g, const StaticLds &L,
                                                    const int32_t *cnt, int32_t e, int32_t pos) {
  const int32_t m = g.E / g.R;
  const int32_t kp = cnt[e] - L.shed[e];
  if (pos < kp) return (e / m) * g.C + L.ord[e] + pos;
  const int32_t a = L.nseg[e] + (pos - kp);
  const int32_t r = last_le(L.rbase, g.R, a);
  return r * g.C + L.home[r] + (a - L.rbase[r]);
}

// LDS of the layout kernel, in int32 words: region A holds the per-wave
// counters while ranking and the planner's tables afterwards; then the
// counts [E] and offsets [E+1].
__host__ __device__ inline int32_t plan_region_a(int32_t E, int32_t R) {
  const int32_t waves = (kTileWaves * E + 1) / 2;            // uint16 counters
  const int32_t planner = R > 0 ? 5 * E + 8 * R + 8 : 0;
  return waves > planner ? waves : planner;
}

// Inclusive scan over the 64 lanes of a wave in six DPP steps: shifts by 1,
// 2, 4 and 8 lanes inside each 16-lane row (lanes without a source add 0),
// then lane 15 of each row added to the next row and lane 31 to the upper
// half.
template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_add(int32_t v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, true);
}
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  v = dpp_add<0x111, 0xF>(v);   // row_shr:1
  v = dpp_add<0x112, 0xF>(v);   // row_shr:2
  v = dpp_add<0x114, 0xF>(v);   // row_shr:4
  v = dpp_add<0x118, 0xF>(v);   // row_shr:8
  v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive scan of cnt[0, E) into offs[0, E] (offs[E] = total) by the whole
// workgroup, E <= its size: a DPP scan per wave, then the wave totals.
// Callers make cnt complete (barrier) before; the scan ends with a barrier.
__device__ void block_exclusive_scan(const int32_t *cnt, int32_t *offs, int32_t E,
                                     int32_t *s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t v = tid < E ? cnt[tid] : 0;
  const int32_t incl = wave_inclusive_scan(v);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int32_t pre = 0;
#pragma unroll
  for (int i = 0; i < kTileWaves; ++i) pre += i < w ? s_wsum[i] : 0;   // loads issued together
  if (tid < E) offs[tid] = pre + incl - v;
  if (tid == E - 1) offs[E] = pre + incl;
  __syncthreads();
}

// Resident-tiles handshake words are 64-bit: (epoch mark << 32) | value.  A
// reader polls each word until it carries this call's mark, so publishing and
// waiting are one round trip and no cache write-back or invalidate is needed
// (the words are written and read at agent scope, through to the point every
// XCD sees).
__device__ __forceinline__ uint64_t tagged(uint32_t mark, uint32_t v) {
  return ((uint64_t)mark << 32) | v;
}

// Polling rounds a handshake wait may take before it gives up: each round
// is a memory round trip and a short sleep, so one to two seconds.
constexpr uint32_t kSpinLimit = 1u << 21;

// Loads the words p[i * stride], i < n <= 16, into v, polling until every one
// carries `mark`; each round re-issues all stale loads together, so a round
// costs one memory latency however many are stale.  Bounded: returns false
// once `spins` exceeds the limit (v then holds what was last read).
template <int N>
__device__ __forceinline__ bool load_tagged(const uint64_t *p, int64_t stride, int n,
                                            uint32_t mark, uint64_t (&v)[N], uint32_t &spins) {
#pragma unroll
  for (int u = 0; u < N; ++u)
    v[u] = u < n ? __hip_atomic_load(p + u * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : tagged(mark, 0u);
  for (;;) {
    bool stale = false;
#pragma unroll
    for (int u = 0; u < N; ++u) stale |= (uint32_t)(v[u] >> 32) != mark;
    if (!stale) return true;
    if (++spins > kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int u = 0; u < N; ++u)
      if ((uint32_t)(v[u] >> 32) != mark)
        v[u] = __hip_atomic_load(p + u * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// RG > 0: the tile first routes the tokens its entries belong to (RG lanes
// per token, RPER logits per lane; route_impl.h), writes their ids and
// weights and ranks them from LDS: routing and the tile histogram in one
// launch.  RG = 0: the ids come from a.idx.
// RES: several tiles, all resident at once; every tile finishes its own
// entries after reading every tile's histogram (no second launch).
// ST: the static layout (the planner runs in the kernel).
template <int RG, int RPER, bool RES, bool ST>
__global__ __launch_bounds__(kTileThreads) void k_plan_tiles(PlanArgs a) {
  extern __shared__ int32_t lds[];
  __shared__ uint32_t s_flags;
  __shared__ int32_t s_last;     // two-launch form: this workgroup finishes; RES: a wait ran out
  __shared__ uint32_t s_mark;    // RES: this call's epoch mark
  __shared__ int32_t s_tmp[kTileWaves + 2];
  const Geometry &g = a.g;
  const Workspace &ws = a.ws;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t E = g.E;
  const bool single = gridDim.x == 1;
  uint16_t *wcnt = reinterpret_cast<uint16_t *>(lds);   // [waves][E], <= 256 each
  int32_t *pl = lds;                                     // planner tables (after ranking)
  int32_t *cnt = lds + plan_region_a(E, ST ? g.R : 0);   // [E]
  int32_t *offs = cnt + E;                               // [E+1]
  int32_t *s_idx = offs + E + 1;                         // RG > 0: the tile's routed ids

  const int64_t f0 = (int64_t)blockIdx.x * kTileEntries;   // the tile's first entry
  const int64_t wbase = f0 + (int64_t)w * (64 * kTileChunks);
  int32_t ev[kTileChunks], rr[kTileChunks];
  if constexpr (RG == 0) {   // the id loads are in flight while LDS is set up
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c) {
      const int64_t f = wbase + c * 64 + lane;
      ev[c] = f < g.n ? a.idx[f] : -1;
    }
  }
  // Each wave zeroes and uses only its own counters, so ranking needs no
  // workgroup barrier first (the waves of a 1024-thread workgroup start up
  // to a microsecond apart); routing shares its ids through LDS and does.
  for (int i = lane; i < E; i += 64) wcnt[w * E + i] = 0;
  __builtin_amdgcn_wave_barrier();
  if (tid == 0) {
    s_flags = 0;
    s_last = 0;
    // This call's epoch: calls so far, from the arrival count (this tile has
    // not arrived, so at most ntiles - 1 arrivals of this call are in it).
    if constexpr (RES)
      s_mark = (uint32_t)(__hip_atomic_load(ws.arrive, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) / gridDim.x) + 1u;
  }
  if constexpr (RG > 0) {
    // The tokens whose entries fall in [f0, f1); a token split between two
    // tiles is routed by both (same result), each keeping its own entries.
    const int64_t f1 = f0 + kTileEntries < g.n ? f0 + kTileEntries : g.n;
    const int64_t t0 = f0 / g.k, t1 = (f1 + g.k - 1) / g.k;
    constexpr int kPass = kTileThreads / RG;   // tokens per pass
    const int sub = lane & (RG - 1);
    for (int64_t tb = t0; tb < t1; tb += kPass) {
      const int64_t t = tb + tid / RG;
      const bool live = t < t1;
      int32_t ri;
      float rw;
      route_token<RG, RPER>(a.logits, live ? t : t0, live, E, g.k, lane, ri, rw);
      const int64_t f = t * g.k + sub;
      if (live && sub < g.k && f >= f0 && f < f1) {
        a.idx_out[f] = ri;
        a.w_out[f] = rw;
        s_idx[f - f0] = ri;
      }
    }
    __syncthreads();
  }
  if constexpr (RG > 0) {
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c) {
      const int64_t f = wbase + c * 64 + lane;
      ev[c] = f < g.n ? s_idx[f - f0] : -1;
    }
  }

  uint32_t flags = 0;
#pragma unroll
  for (int c = 0; c < kTileChunks; ++c) {
    const int64_t f = wbase + c * 64 + lane;
    int32_t e = -1;
    if (f < g.n) {
      const int32_t raw = ev[c];
      if (raw >= 0 && raw < E) e = raw;
      else if (raw != -1) flags |= kFlagIndexRange;
      if (!single && !RES) ws.eidx[f] = e;
    }
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < g.nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    int32_t r = 0;
    if (valid) {
      const int32_t before = wcnt[w * E + e];
      r = before + __popcll(peers & ((1ull << lane) - 1ull));
      if ((peers >> lane) == 1ull) wcnt[w * E + e] = (uint16_t)(before + __popcll(peers));
    }
    ev[c] = e;
    rr[c] = r;
  }
  __syncthreads();

  uint32_t mark = 0;
  if constexpr (RES) mark = s_mark;
  for (int e = tid; e < E; e += kTileThreads) {
    int32_t v[kTileWaves];
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) v[ww] = wcnt[ww * E + e];
    int32_t run = 0;
#pragma unroll
    for (int ww = 0; ww < kTileWaves; ++ww) {
      wcnt[ww * E + e] = (uint16_t)run;
      run += v[ww];
    }
    if (single) cnt[e] = run;                              // the tile is the whole layout
    else if (RES)   // published with this call's mark
      __hip_atomic_store(ws.tagged + (int64_t)blockIdx.x * E + e, tagged(mark, (uint32_t)run),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else ws.tile_hist[(int64_t)blockIdx.x * E + e] = run;
  }
  if (flags) atomicOr(&s_flags, flags);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kTileChunks; ++c) {
    if (ev[c] >= 0) {
      rr[c] += wcnt[w * E + ev[c]];
      if (!single && !RES) ws.lrank[wbase + c * 64 + lane] = rr[c];
    }
  }

  if constexpr (RES) {
    const int32_t ntiles = gridDim.x;
    uint64_t *tflags = ws.tagged + (int64_t)ntiles * E;   // [ntiles] flags words
    if (tid == 0) {
      __hip_atomic_store(tflags + blockIdx.x, tagged(mark, s_flags), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(ws.arrive, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();   // the per-wave counters are read; region A takes the bases
    // This tile's base and every expert's total from all the histograms.
    int32_t *sbase = lds;
    uint32_t spins = 0;
    bool ok = true;
    for (int e = tid; e < E; e += kTileThreads) {
      int32_t run = 0, base = 0;
      for (int32_t t0 = 0; t0 < ntiles; t0 += 16) {
        uint64_t v[16];
        const int n = ntiles - t0 < 16 ? ntiles - t0 : 16;
        ok = load_tagged(ws.tagged + (int64_t)t0 * E + e, E, n, mark, v, spins) && ok;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (u < n) {
            if (t0 + u == (int32_t)blockIdx.x) base = run;
            run += (int32_t)(uint32_t)v[u];
          }
        }
      }
      cnt[e] = run;
      sbase[e] = base;
    }
    if (blockIdx.x == 0) {   // every tile's flags, for the status word
      for (int32_t t = tid; t < ntiles; t += kTileThreads) {
        uint64_t v[1];
        ok = load_tagged(tflags + t, 0, 1, mark, v, spins) && ok;
        const uint32_t fl = (uint32_t)v[0];
        if (fl) atomicOr(&s_flags, fl);
      }
    }
    if (!ok) s_last = 1;
    __syncthreads();
    // positions inside the expert, kept in registers so region A can hold
    // the planner's tables next
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c)
      if (ev[c] >= 0) rr[c] += sbase[ev[c]];
  }

  if (!single && !RES) {
    // Publish this tile; the last one to arrive finishes the layout.  Every
    // wave waits for its own stores to reach L2, the barrier joins them, then
    // a single wave makes them visible to the other XCDs (agent-scope release:
    // one L2 write-back per workgroup, not one per wave) and takes a ticket.
    // The last workgroup's agent-scope acquire (one invalidate) lets all its
    // waves see every tile.
    if (tid == 0) ws.tile_flags[blockIdx.x] = s_flags;
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const uint32_t t = atomicAdd(ws.ticket, 1u);
      s_last = (t == gridDim.x - 1) ? 1 : 0;
      if (s_last) __threadfence();
    }
    __syncthreads();
    if (!s_last) return;

    const int32_t ntiles = gridDim.x;
    // Per-expert exclusive scan over the tiles.  The loads of 16 tiles are
    // issued together so the scan costs ntiles/16 memory latencies, not ntiles.
    for (int e = tid; e < E; e += kTileThreads) {
      int32_t run = 0;
      for (int32_t t0 = 0; t0 < ntiles; t0 += 16) {
        int32_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          v[u] = t0 + u < ntiles ? ws.tile_hist[(int64_t)(t0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (t0 + u < ntiles) ws.tile_hist[(int64_t)(t0 + u) * E + e] = run;
          run += v[u];
        }
      }
      cnt[e] = run;
    }
    for (int32_t t = tid; t < ntiles; t += kTileThreads) {
      const uint32_t fl = ws.tile_flags[t];
      if (fl) atomicOr(&s_flags, fl);
    }
    if (tid == 0) *ws.ticket = 0;
  }
  // From here on the layout lives in LDS; global results are written at the
  // end, because every barrier waits for the wave's outstanding global
  // stores as well as its loads.
  __syncthreads();
  block_exclusive_scan(cnt, offs, E, s_tmp);
  const int32_t total = offs[E];
  const bool writer = !RES || blockIdx.x == 0;   // the tile that writes the shared tables
  if (g.layout == kLL && writer) {
    for (int e = tid; e < E; e += kTileThreads)
      if (cnt[e] > g.cap) atomicOr(&s_flags, kFlagCapacity);
    __syncthreads();
  } else if constexpr (ST) {
    // Every resident tile has every count, so each runs the planner on its
    // own (the same tables, in its LDS) and places its entries from there;
    // tile 0 also writes the tables out.  No tile waits for another's.
    plan_static(g, ws, cnt, total, pl, s_tmp, &s_flags, writer);
    __syncthreads();
  }
  if (writer) {
    for (int e = tid; e <= E; e += kTileThreads) {
      ws.offsets[e] = offs[e];
      if (e < E) ws.counts[e] = cnt[e];
    }
    if (tid == 0) *ws.status = s_flags;
  }
  // A tile whose wait for the histograms ran out leaves this call's mark in
  // the stall word, which ep_handle_status reports as EP_FLAG_PLAN_STALL.
  if constexpr (RES)
    if (tid == 0 && s_last)
      __hip_atomic_store(ws.stall, mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  if (single || RES) {
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c) {
      const int64_t f = wbase + c * 64 + lane;
      if (f < g.n) {
        int32_t d = -1;
        if (ev[c] >= 0) {
          if constexpr (ST) d = entry_dst_static(g, static_lds(pl, E, g.R), cnt, ev[c], rr[c]);
          else d = entry_dst(g, ws, offs, ev[c], rr[c]);
        }
        if (d >= g.rows) d = -1;
        ws.eidx[f] = ev[c];
        ws.dst[f] = d;
        if (d >= 0) ws.recv_src[d] = (int32_t)f;
      }
    }
  }
}

// Several tiles: one thread per entry (destination from its tile base and
// tile rank).
__global__ __launch_bounds__(256) void k_plan_dst(PlanArgs a) {
  const Geometry &g = a.g;
  const Workspace &ws = a.ws;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < g.n) {
    const int32_t e = ws.eidx[i];
    int32_t d = -1;
    if (e >= 0) {
      const int64_t tile = i / kTileEntries;
      const int32_t pos = ws.tile_hist[tile * g.E + e] + ws.lrank[i];
      d = entry_dst(g, ws, ws.offsets, e, pos);
      if (d >= g.rows) d = -1;
    }
    ws.dst[i] = d;
    if (d >= 0) ws.recv_src[d] = (int32_t)i;
  }
}

size_t plan_lds_bytes(int32_t E, int32_t R) {
  return (size_t)(plan_region_a(E, R) + 2 * E + 1) * sizeof(int32_t);
}

// All tiles in one launch when they can all be resident at once: one
// 1024-thread workgroup per compute unit at most.
static bool resident_tiles(const Geometry &g) { return g.ntiles > 1 && g.ntiles <= g.cus; }

static hipError_t launch_plan_dst(const Geometry &g, const PlanArgs &a, hipStream_t s) {
  if (g.ntiles > 1 && !resident_tiles(g)) {
    const int64_t blocks = (g.n + 255) / 256;
    hipLaunchKernelGGL(k_plan_dst, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// Fused routing + layout: 16 lanes per token, up to 32 logits per lane
// (E <= 512); larger E routes in its own launch first.
constexpr int kFusedRouteLanes = 16;
constexpr int kFusedRouteMaxPer = 32;

hipError_t launch_route_plan(const Geometry &g, const Workspace &ws, const float *logits,
                             int32_t *idx, float *w, hipStream_t s) {
  const int per = (g.E + kFusedRouteLanes - 1) / kFusedRouteLanes;
  if (per > kFusedRouteMaxPer) {
    hipError_t err = launch_route(logits, g.T, g.E, g.k, idx, w, s);
    return err != hipSuccess ? err : launch_plan(g, ws, idx, s);
  }
  PlanArgs a{g, ws, idx, logits, idx, w};
  const size_t lds =
      plan_lds_bytes(g.E, g.layout == kStatic ? g.R : 0) + (size_t)kTileEntries * sizeof(int32_t);
#define L3(P, RES, ST)                                                                          \
  hipLaunchKernelGGL((k_plan_tiles<kFusedRouteLanes, P, RES, ST>), dim3(g.ntiles),            \
                     dim3(kTileThreads), lds, s, a)
#define L2(P, RES)                                   \
  do {                                               \
    if (g.layout == kStatic) L3(P, RES, true);       \
    else L3(P, RES, false);                          \
  } while (0)
#define L(P)                            \
  do {                                  \
    if (resident_tiles(g)) L2(P, true); \
    else L2(P, false);                  \
  } while (0)
  if (per <= 1) L(1);
  else if (per <= 2) L(2);
  else if (per <= 4) L(4);
  else if (per <= 8) L(8);
  else if (per <= 16) L(16);
  else L(32);
#undef L
#undef L2
#undef L3
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_plan_dst(g, a, s);
}

hipError_t launch_plan(const Geometry &g, const Workspace &ws, const int32_t *topk_idx,
                       hipStream_t s) {
  PlanArgs a{g, ws, topk_idx, nullptr, nullptr, nullptr};
  const size_t lds = plan_lds_bytes(g.E, g.layout == kStatic ? g.R : 0);
#define L(RES, ST) \
  hipLaunchKernelGGL((k_plan_tiles<0, 0, RES, ST>), dim3(g.ntiles), dim3(kTileThreads), lds, s, a)
  const bool st = g.layout == kStatic;
  if (resident_tiles(g)) {
    if (st) L(true, true);
    else L(true, false);
  } else {
    if (st) L(false, true);
    else L(false, false);
  }
#undef L
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_plan_dst(g, a, s);
}

}  // namespace epk
