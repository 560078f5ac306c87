// gemm.hip -- grouped GEMM of the experts on gfx950 MFMA ("Ultra-Large MoE
// Models" article, section 3.1: the core of the expert computation, one
// irregularly sized matrix product per expert over the tokens grouped by
// expert; NCCL EP listing, Figure 2: the expert FFN sits between dispatch
// and combine).
//
// For every group of consecutive receive rows that share one weight matrix
// (an expert's rows, or a STATIC segment through its prefetch slot):
//   Y[row][n] = bf16( sum_c X[row][c] * W[n][c] ),  fp32 accumulation.
//
// Kernels:
//  * k_gemm_tiles (one workgroup) cuts the groups of the current plan into
//    row tiles -- (row0, rows, weight index) -- with a prefix sum over the
//    groups, so the GEMM grid can have a fixed size;
//  * k_grouped_gemm_256 for large groups (at least 128 rows per expert on
//    average) and N >= 256: one 256-thread workgroup per CU and per
//    (256-row tile, 256 columns); each wave owns a 128 x 128 block as 4 x 4
//    MFMA accumulators (256 accumulation registers), which halves the LDS
//    bytes read per flop against the 128 x 128 tile -- LDS bandwidth, not
//    the matrix cores, is what bounds these kernels.  Loads are buffer loads
//    (a scalar resource and one 32-bit offset per lane); the next slab is
//    staged in registers, and its LDS writes and the global loads of the one
//    after go under the first two 16-deep steps' MFMAs, the LDS reads of the
//    next step under the first half of each step, and the one barrier per
//    slab sits before the last step, so the first reads of the next slab run
//    under that step's MFMAs;
//  * k_grouped_gemm: one 256-thread workgroup per (128-row tile, 128 columns),
//    two per CU; four waves in a 2 x 2 arrangement, each owning a 64 x 64
//    block of the output as 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators.
//    Slabs 64 deep of X and W go through LDS, double-buffered.  Pipelining:
//    the global loads of slab kt+2 are in flight during slab kt+1; within a
//    slab, the fragments of the next 16-deep step are read from LDS while
//    the MFMAs of the current one run, and the first step of the next slab
//    is read right after the barrier that publishes it.  In the steady state
//    (no branches) all 16 MFMAs of a slab come before the barrier and
//    sched_group_barrier spreads the LDS reads over the first 8 and the next
//    slab's LDS writes and the global loads of the one after over the last 8,
//    so the matrix cores stay busy while the wave issues its memory traffic.
//    Epilogue (N a multiple of 8): the tile goes through LDS as bf16 rows and
//    leaves with 16-byte row stores instead of 2-byte column stores.
//    LDS: rows of a slab are 128 bytes (eight 16-byte chunks); with 64
//    4-byte banks two rows share a 256-byte bank row, so chunk c of row r is
//    stored at c ^ ((r / 2) % 8): the 16 rows one 16-lane phase of an MFMA
//    operand read touches then cover all 64 banks once (no conflicts).
//    Rows past a tile's end load a valid row instead of branching (their
//    products land in outputs that are never stored), and a wave whose
//    32-row blocks hold no rows of the tile skips their fragment reads and
//    MFMAs: the main loop is compiled once per count of live blocks and each
//    wave runs its own copy (all copies have the same barriers).  The wide
//    and FP8 kernels do the same.
//    Workgroup order (balanced_tile): workgroup b runs on XCD b % 8; every
//    XCD takes the same share of the full row tiles (MFMA-bound) and of the
//    short ones (bound by streaming their weight slice), merged, column tile
//    fastest, so no XCD holds only one kind: with skewed routing the hot
//    experts' full tiles would otherwise sit on the first XCDs and the cold
//    experts' short tiles on the last ones, which then idle.  Each XCD takes
//    every eighth tile of a kind, so the XCDs walk the groups together and
//    a hot expert's row tiles, spread over all of them at once, share its
//    weight slices through the Infinity Cache.
#include "device.h"
#include "ep_internal.h"

namespace epk {

constexpr int kTileM = kGemmBM;
constexpr int kBN = 128;
constexpr int kWavesM = 2, kWavesN = 2;
constexpr int kGemmThreads = 64 * kWavesM * kWavesN;
constexpr int kWTM = kTileM / kWavesM, kWTN = kBN / kWavesN;  // one wave's output block
constexpr int kFM = kWTM / 32, kFN = kWTN / 32;                // 32 x 32 MFMA blocks per wave
constexpr int kBK = 64;
constexpr int kChunks = kBK / 8;  // 16-byte chunks in one row of a slab
constexpr int kXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int row, int c) { return row * kChunks + (c ^ ((row >> 1) & 7)); }
static_assert(kChunks == 8, "the swizzle assumes 128-byte slab rows");

// ---------------------------------------------------------------------------
// tile table

struct TileArgs {
  Geometry g;
  Workspace ws;
  int32_t use_slots;  // STATIC segments with a slot read weights from the slot
};

// Group q of the current plan: first receive row, rows, weight index
// (< E: owner expert; E + r*S + s: slot s of rank r).
__device__ __forceinline__ void group_of(const TileArgs &a, int32_t q, int32_t &row0,
                                         int32_t &rows, int32_t &widx) {
  const Geometry &g = a.g;
  const Workspace &ws = a.ws;
  if (g.layout == kHT) {
    row0 = ws.offsets[q];
    rows = ws.offsets[q + 1] - row0;
    widx = q;
  } else if (g.layout == kLL) {
    const int32_t c = ws.counts[q];
    row0 = q * g.cap;
    rows = c < g.cap ? c : g.cap;
    widx = q;
  } else if (q < g.E) {  // kept rows of expert q on its home rank
    const int32_t m = g.E / g.R;
    row0 = (q / m) * g.C + ws.native_row[q];
    rows = ws.keep[q];
    widx = q;
  } else {  // segment q - E on its receiving rank
    const int32_t *s = ws.segments + (int64_t)(q - g.E) * 5;
    const int32_t slot = ws.seg_slot[q - g.E];
    row0 = s[1] * g.C + s[4];
    rows = s[3];
    widx = (a.use_slots && slot >= 0) ? g.E + s[1] * g.S + slot : s[0];
  }
}

// PART: row tiles come in two kinds, full ones (more than TM/2 rows), whose
// time is MFMA work, and short ones (a group's tail or a small group), whose
// time is streaming their weight slice.  The table then holds the full tiles
// in group order from the front and the short ones in group order from the
// back (entry max_tiles - 1 - j is short tile j), so the GEMM kernel can give
// every XCD the same share of each kind (balanced_tile).  Without PART every
// tile counts as full: the table is in group order, and XCD x takes tiles
// x, x + 8, x + 16, ... of it.
// ntiles[0] = all tiles, ntiles[1] = full tiles.
template <int TM, bool PART>
__global__ __launch_bounds__(1024) void k_gemm_tiles(TileArgs a, int32_t max_tiles) {
  __shared__ int32_t s_wave[2][16];
  __shared__ int32_t s_base[2];
  const Geometry &g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t ngroups = g.layout == kStatic ? g.E + *a.ws.n_segments : g.E;
  if (tid < 2) s_base[tid] = 0;
  __syncthreads();
  for (int32_t q0 = 0; q0 < ngroups; q0 += 1024) {
    const int32_t q = q0 + tid;
    int32_t row0 = 0, rows = 0, widx = 0;
    if (q < ngroups) group_of(a, q, row0, rows, widx);
    const int32_t nt = rows > 0 ? (rows + TM - 1) / TM : 0;
    const int32_t tail = rows - (nt - 1) * TM;                 // rows of the last tile
    const int32_t nshort = PART && nt > 0 && 2 * tail <= TM ? 1 : 0;   // the last may be short
    const int32_t nfull = nt - nshort;
    // inclusive scans of nfull and nshort over the workgroup: lanes, then waves
    int32_t xf = nfull, xs = nshort;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t yf = __shfl_up(xf, d), ys = __shfl_up(xs, d);
      if (lane >= d) {
        xf += yf;
        xs += ys;
      }
    }
    if (lane == 63) {
      s_wave[0][w] = xf;
      s_wave[1][w] = xs;
    }
    __syncthreads();
    int32_t bf = s_base[0], bs = s_base[1], tf = 0, ts = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      bf += v < w ? s_wave[0][v] : 0;
      bs += v < w ? s_wave[1][v] : 0;
      tf += s_wave[0][v];
      ts += s_wave[1][v];
    }
    bf += xf - nfull;   // full tiles before this group's
    bs += xs - nshort;  // short tiles before this group's
    for (int32_t i = 0; i < nt; ++i) {
      const int32_t t = i < nfull ? bf + i : max_tiles - 1 - bs;
      if (t < 0 || t >= max_tiles) continue;   // not reached: the table holds every tile
      int32_t *e = a.ws.gemm_tiles + (int64_t)t * 4;
      e[0] = row0 + i * TM;
      e[1] = rows - i * TM < TM ? rows - i * TM : TM;
      e[2] = widx;
      e[3] = 0;
    }
    __syncthreads();
    if (tid == 0) {
      s_base[0] += tf;
      s_base[1] += ts;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int32_t nf = s_base[0], all = s_base[0] + s_base[1];
    a.ws.gemm_ntiles[0] = all < max_tiles ? all : max_tiles;
    a.ws.gemm_ntiles[1] = nf < max_tiles ? nf : max_tiles;
  }
}

// Work of workgroup blockIdx.x: its row tile (an index into the table) and
// column tile.  Workgroup b runs on XCD b % 8; XCD x takes full tiles x,
// x + 8, x + 16, ... and short tiles x, x + 8, ..., each in group order,
// merged in proportion (Bresenham), every row tile with its column tiles one
// after another.  So every XCD gets the same MFMA-bound and streaming-bound
// work and runs both kinds side by side; the column tiles of a row tile stay
// on one XCD (they share X rows in its L2); and the eight XCDs walk the
// groups together, so the row tiles of one expert run on all of them at about
// the same time and its weight slices, after the first read, come from the
// Infinity Cache that the XCDs share (with each XCD taking a contiguous
// eighth, the row tiles of a hot expert ran one after another on one XCD and
// read its weights from HBM again each time).  The grid holds at least
// (max_tiles / 8 + 2) * n_col_tiles workgroups per XCD (gemm_grid).
__device__ __forceinline__ bool balanced_tile(const int32_t *__restrict__ ntiles,
                                              int32_t max_tiles, int32_t n_col_tiles,
                                              int32_t &tile, int32_t &col) {
  const int32_t nf = ntiles[1], ns = ntiles[0] - nf;
  const int32_t x = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  // this XCD's full and short tiles: those whose index is x modulo 8
  const int32_t b = x < nf ? (nf - x + kXcds - 1) / kXcds : 0;
  const int32_t n = b + (x < ns ? (ns - x + kXcds - 1) / kXcds : 0);
  const int32_t p = slot / n_col_tiles;
  if (p >= n) return false;
  col = slot - p * n_col_tiles;
  const int32_t before = (int32_t)((int64_t)p * b / n), upto = (int32_t)((int64_t)(p + 1) * b / n);
  tile = upto > before ? x + kXcds * before : max_tiles - 1 - (x + kXcds * (p - before));
  return true;
}

// ---------------------------------------------------------------------------
// grouped GEMM

// SwiGLU epilogue of the expert FFN's first GEMM.  Its weight rows come
// interleaved (row 2j the gate projection of output j, row 2j + 1 the up
// projection), so a 16-byte vector of the staged bf16 output tile holds four
// (gate, up) pairs, gate in the low half of each 32-bit word.  Each pair
// becomes bf16(silu(gate) * up), silu(g) = g / (1 + e^-g) in fp32 with the
// hardware reciprocal (about 1 ulp of fp32, far below the bf16 rounding).
// That reciprocal is a normal fp32 while 1 + e^-g < 2^126; from g < -64 on
// (1 + e^-g > 2^92, and 1 + e^g == 1 in fp32) the value is taken as
// g * up * e^g in double instead, so tiny and subnormal results match the
// exact value to one rounding over the whole range.
__device__ __forceinline__ uint2 swiglu4(u32x4 v) {
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g = __uint_as_float(in[i] << 16), u = __uint_as_float(in[i] & 0xFFFF0000u);
    if (g < -64.0f) o[i] = (float)((double)g * (double)u * exp((double)g));
    else o[i] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
  }
  return uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 2) void k_grouped_gemm(
    const u32x4 *__restrict__ X, const u32x4 *__restrict__ W, const u32x4 *__restrict__ Wslot,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ ntiles, int32_t max_tiles,
    int32_t K, int32_t N,
    int32_t E, int32_t n_col_tiles, uint16_t *__restrict__ Y) {
  __shared__ u32x4 sa[2][kTileM * kChunks];
  static_assert(kTileM * kChunks % kGemmThreads == 0 && kBN * kChunks % kGemmThreads == 0, "loader");
  __shared__ u32x4 sb[2][kBN * kChunks];
  // XCD-aware order over the valid work only (the grid is sized for the
  // largest possible tile count)
  int32_t tile, ctile;
  if (!balanced_tile(ntiles, max_tiles, n_col_tiles, tile, ctile)) return;
  const int32_t n0 = ctile * kBN;
  const int32_t row0 = tiles[tile * 4 + 0], rows = tiles[tile * 4 + 1], widx = tiles[tile * 4 + 2];
  const int64_t KV = K / 8;  // 16-byte vectors per row
  const u32x4 *Wm = widx < E ? W + (int64_t)widx * N * KV : Wslot + (int64_t)(widx - E) * N * KV;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wv / kWavesN, wn = wv % kWavesN;

  // loader: chunk q = tid + i * 256 of a slab is row q / 8, chunk q % 8.
  // Rows past the tile's end read a valid row instead (their products land
  // in outputs that are never stored), so every load is unconditional.
  constexpr int kLoads = kTileM * kChunks / kGemmThreads;
  constexpr int kLoadsB = kBN * kChunks / kGemmThreads;
  const int c_ld = tid & (kChunks - 1);
  const u32x4 *pa[kLoads];
  const u32x4 *pb[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    pa[i] = X + (int64_t)(row0 + (r < rows ? r : rows - 1)) * KV + c_ld;
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    pb[i] = Wm + (int64_t)(n0 + r < N ? n0 + r : N - 1) * KV + c_ld;
  }
  u32x4 ra0[kLoads], rb0[kLoadsB];

#define GLOAD(RA, RB, kt)                                                              \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i) RA[i] = pa[i][(kt) * kChunks];    \
  _Pragma("unroll") for (int i = 0; i < kLoadsB; ++i) RB[i] = pb[i][(kt) * kChunks];
#define SWRITE(RA, RB, buf)                                                                 \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i)                                        \
      sa[buf][swz((tid + i * kGemmThreads) / kChunks, c_ld)] = RA[i];                       \
  _Pragma("unroll") for (int i = 0; i < kLoadsB; ++i)                                       \
      sb[buf][swz((tid + i * kGemmThreads) / kChunks, c_ld)] = RB[i];

  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One 16-deep step of fragments is read from LDS while the MFMAs of the
  // previous step run (two small register sets); the first step of slab
  // kt+1 is read right after the barrier that publishes it, under the last
  // MFMAs of slab kt.  The global loads of slab kt+2 are in flight during
  // all of slab kt+1.
#define READK(FA, FB, buf, kk, LB)                                                                  \
  {                                                                                                 \
    const int c_ = (kk) * 2 + (lane >> 5);                                                          \
    _Pragma("unroll") for (int i = 0; i < (LB); ++i)                                                \
        FA[i] = __builtin_bit_cast(bf16x8, sa[buf][swz(wm * kWTM + i * 32 + (lane & 31), c_)]);     \
    _Pragma("unroll") for (int j = 0; j < kFN; ++j)                                                 \
        FB[j] = __builtin_bit_cast(bf16x8, sb[buf][swz(wn * kWTN + j * 32 + (lane & 31), c_)]);     \
  }
#define MFMAK(FA, FB, LB)                                                                           \
  _Pragma("unroll") for (int i = 0; i < (LB); ++i)                                                  \
  _Pragma("unroll") for (int j = 0; j < kFN; ++j)                                                   \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0);

  static_assert(kBK == 64, "four 16-deep steps per slab");
  const int KT = K / kBK;
  bf16x8 fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  GLOAD(ra0, rb0, 0);
  SWRITE(ra0, rb0, 0);
  if (KT > 1) { GLOAD(ra0, rb0, 1); }
  __syncthreads();
  // sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read, 0x200 LDS write,
  // 0x020 global load; each call asks for the next n instructions of that kind
#define SGB(m, n) __builtin_amdgcn_sched_group_barrier(m, n, 0)
  // LB: the wave's 32-row blocks that hold rows of the tile (2, 1 or 0); the
  // loop is compiled for each with the same barriers, and empty blocks are
  // neither read nor multiplied.  The interleaving pattern is for full waves.
#define MAIN_LOOP(LB)                                                                               \
  {                                                                                                 \
    READK(fa0, fb0, 0, 0, LB);                                                                      \
    int kt = 0;                                                                                     \
    for (; kt + 2 < KT; ++kt) { /* steady state */                                                  \
      const int buf = kt & 1;                                                                       \
      READK(fa1, fb1, buf, 1, LB);                                                                  \
      MFMAK(fa0, fb0, LB);                                                                          \
      READK(fa0, fb0, buf, 2, LB);                                                                  \
      MFMAK(fa1, fb1, LB);                                                                          \
      READK(fa1, fb1, buf, 3, LB);                                                                  \
      MFMAK(fa0, fb0, LB);                                                                          \
      SWRITE(ra0, rb0, buf ^ 1);                                                                    \
      GLOAD(ra0, rb0, kt + 2);                                                                      \
      MFMAK(fa1, fb1, LB);                                                                          \
      if constexpr ((LB) == kFM) {                                                                  \
        _Pragma("unroll") for (int q = 0; q < 8; ++q) { SGB(0x008, 1); SGB(0x100, 1); }             \
        _Pragma("unroll") for (int q = 0; q < 8; ++q) { SGB(0x008, 1); SGB(0x200, 1); SGB(0x020, 1); } \
      }                                                                                             \
      __syncthreads();                                                                              \
      READK(fa0, fb0, buf ^ 1, 0, LB);                                                              \
    }                                                                                               \
    for (; kt < KT; ++kt) { /* the last two slabs (no more global loads) */                         \
      const int buf = kt & 1;                                                                       \
      READK(fa1, fb1, buf, 1, LB);                                                                  \
      MFMAK(fa0, fb0, LB);                                                                          \
      READK(fa0, fb0, buf, 2, LB);                                                                  \
      MFMAK(fa1, fb1, LB);                                                                          \
      READK(fa1, fb1, buf, 3, LB);                                                                  \
      MFMAK(fa0, fb0, LB);                                                                          \
      if (kt + 1 < KT) {                                                                            \
        SWRITE(ra0, rb0, buf ^ 1);                                                                  \
        __syncthreads();                                                                            \
        READK(fa0, fb0, buf ^ 1, 0, LB);                                                            \
      }                                                                                             \
      MFMAK(fa1, fb1, LB);                                                                          \
    }                                                                                               \
  }
  const int live = (rows - wm * kWTM + 31) / 32;  // wave-uniform
  if (live >= kFM) MAIN_LOOP(kFM)
  else if (live == 1) MAIN_LOOP(1)
  else MAIN_LOOP(0)
#undef MAIN_LOOP
#undef SGB
#undef READK
#undef MFMAK
#undef GLOAD
#undef SWRITE

  if (GLU || (N & 7) == 0) {   // a SwiGLU launch has N % 16 == 0
    // Through LDS: the tile as bf16 rows of 128, the 16-byte chunk of column c
    // of row r stored at chunk (c / 8) ^ (((r / 4) % 4) * 4), so the two
    // half-waves of a store (rows r and r + 4) land on different banks; then
    // 16-byte row stores.
    __syncthreads();   // every wave is done with the slab buffers
    uint16_t *so = reinterpret_cast<uint16_t *>(&sa[0][0]);
    static_assert(kTileM * kBN * 2 <= (int)sizeof(sa), "output tile fits the slab buffers");
#define OSW(r_, cv_) ((r_) * kBN + (((cv_) ^ ((((r_) >> 2) & 3) << 2)) << 3))
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int c = wn * kWTN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int rr = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
          so[OSW(rr, c >> 3) + (c & 7)] = (uint16_t)(p & 0xFFFFu);
          so[OSW(rr + 1, c >> 3) + (c & 7)] = (uint16_t)(p >> 16);
        }
      }
    __syncthreads();
    constexpr int kVecs = kTileM * kBN / 8;   // 16-byte vectors in the tile
#pragma unroll
    for (int q = 0; q < kVecs / kGemmThreads; ++q) {
      const int idx = tid + q * kGemmThreads;
      const int rr = idx / (kBN / 8), cv = idx % (kBN / 8);
      const int col = n0 + cv * 8;
      if (rr < rows && col < N) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(so + OSW(rr, cv));
        if constexpr (GLU)   // columns col .. col + 7 give outputs col / 2 .. col / 2 + 3
          *reinterpret_cast<uint2 *>(Y + (int64_t)(row0 + rr) * (N / 2) + col / 2) = swiglu4(v);
        else
          *reinterpret_cast<u32x4 *>(Y + (int64_t)(row0 + rr) * N + col) = v;
      }
    }
#undef OSW
    return;
  }
  // accumulator r of a lane: row (r / 4) * 8 + (lane / 32) * 4 + r % 4, column lane % 32
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);  // rows row, row + 1
        if (row < rows) Y[(int64_t)(row0 + row) * N + col] = (uint16_t)(p & 0xFFFFu);
        if (row + 1 < rows) Y[(int64_t)(row0 + row + 1) * N + col] = (uint16_t)(p >> 16);
      }
    }
}

// ---------------------------------------------------------------------------
// grouped GEMM, 256 x 256 tiles (large groups)

constexpr int kBM2 = 256, kBN2 = 256;                     // tile
constexpr int kWTM2 = kBM2 / 2, kWTN2 = kBN2 / 2;         // one wave's block (2 x 2 waves)
constexpr int kFM2 = kWTM2 / 32, kFN2 = kWTN2 / 32;       // 4 x 4 MFMA accumulators per wave
constexpr int kLoads2 = kBM2 * kChunks / kGemmThreads;    // 16-byte loads per thread per slab of X
constexpr int kLoadsB2 = kBN2 * kChunks / kGemmThreads;   // ... and of W
constexpr int kSlabA2 = kBM2 * kChunks, kSlabB2 = kBN2 * kChunks;
constexpr int kBufDword3 = 0x00020000;                    // buffer resource word 3 (raw, 32-bit data)

// Epilogue of the 256 x 256 kernels: the fp32 tile (a wave's 4 x 4 blocks of
// 32 x 32) to bf16 rows of Y (plain, or SwiGLU pairs).  N % 8 == 0: through
// LDS (the slab buffers, free by now) as bf16 rows of 256 with the 128 x 128
// kernel's chunk swizzle, then 16-byte row stores; otherwise 2-byte stores.
template <bool GLU>
__device__ __forceinline__ void wide_epilogue(f32x16 (&acc)[kFM2][kFN2], u32x4 *lds, int32_t rows,
                                              int32_t row0, int32_t n0, int32_t N,
                                              uint16_t *__restrict__ Y, int wm, int wn, int lane,
                                              int tid) {
  if (GLU || (N & 7) == 0) {   // a SwiGLU launch has N % 16 == 0
    __syncthreads();
    uint16_t *so = reinterpret_cast<uint16_t *>(lds);
#define OSW(r_, cv_) ((r_) * kBN2 + (((cv_) ^ ((((r_) >> 2) & 3) << 2)) << 3))
#pragma unroll
    for (int i = 0; i < kFM2; ++i)
#pragma unroll
      for (int j = 0; j < kFN2; ++j) {
        const int c = wn * kWTN2 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int rr = wm * kWTM2 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
          so[OSW(rr, c >> 3) + (c & 7)] = (uint16_t)(p & 0xFFFFu);
          so[OSW(rr + 1, c >> 3) + (c & 7)] = (uint16_t)(p >> 16);
        }
      }
    __syncthreads();
    constexpr int kVecs = kBM2 * kBN2 / 8;
#pragma unroll 4
    for (int q = 0; q < kVecs / kGemmThreads; ++q) {
      const int idx = tid + q * kGemmThreads;
      const int rr = idx / (kBN2 / 8), cv = idx % (kBN2 / 8);
      const int col = n0 + cv * 8;
      if (rr < rows && col < N) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(so + OSW(rr, cv));
        if constexpr (GLU)   // columns col .. col + 7 give outputs col / 2 .. col / 2 + 3
          *reinterpret_cast<uint2 *>(Y + (int64_t)(row0 + rr) * (N / 2) + col / 2) = swiglu4(v);
        else
          *reinterpret_cast<u32x4 *>(Y + (int64_t)(row0 + rr) * N + col) = v;
      }
    }
#undef OSW
    return;
  }
#pragma unroll
  for (int i = 0; i < kFM2; ++i)
#pragma unroll
    for (int j = 0; j < kFN2; ++j) {
      const int col = n0 + wn * kWTN2 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = wm * kWTM2 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
        if (row < rows) Y[(int64_t)(row0 + row) * N + col] = (uint16_t)(p & 0xFFFFu);
        if (row + 1 < rows) Y[(int64_t)(row0 + row + 1) * N + col] = (uint16_t)(p >> 16);
      }
    }
}

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_256(
    const u32x4 *__restrict__ X, const u32x4 *__restrict__ W, const u32x4 *__restrict__ Wslot,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ ntiles, int32_t max_tiles,
    int32_t K, int32_t N,
    int32_t E, int32_t n_col_tiles, uint16_t *__restrict__ Y) {
  // two 64-deep slabs of X and W (128 KB), then the bf16 output tile
  __shared__ u32x4 lds[2 * kSlabA2 + 2 * kSlabB2];
  static_assert(kBM2 * kBN2 * 2 <= (int)sizeof(lds), "output tile fits the slab buffers");
  u32x4 *const sa = lds, *const sb = lds + 2 * kSlabA2;
  int32_t tile, ctile;
  if (!balanced_tile(ntiles, max_tiles, n_col_tiles, tile, ctile)) return;
  const int32_t n0 = ctile * kBN2;
  const int32_t row0 = tiles[tile * 4 + 0], rows = tiles[tile * 4 + 1], widx = tiles[tile * 4 + 2];
  const int64_t KV = K / 8;  // 16-byte vectors per row
  const u32x4 *Xt = X + (int64_t)row0 * KV;
  const u32x4 *Wt = (widx < E ? W + (int64_t)widx * N * KV : Wslot + (int64_t)(widx - E) * N * KV) +
                    (int64_t)n0 * KV;
  const int32_t wrows = N - n0 < kBN2 ? N - n0 : kBN2;
  // Buffer resources over the tile's rows of X and W.  Every offset below is
  // in range by construction (rows past the end are clamped to the last
  // row); the hardware range check is a second guard.
  const __amdgpu_buffer_rsrc_t rX =
      __builtin_amdgcn_make_buffer_rsrc((void *)Xt, (short)0, rows * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc((void *)Wt, (short)0, wrows * K * 2, kBufDword3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wv >> 1, wn = wv & 1;
  const int c_ld = tid & (kChunks - 1);
  // byte offsets of this thread's chunks: chunk q = tid + i * 256 of a slab
  // is row q / 8, 16-byte chunk q % 8; rows past the tile's end read the last
  // row (their products land in outputs that are never stored)
  int32_t oa[kLoads2], ob[kLoadsB2];
#pragma unroll
  for (int i = 0; i < kLoads2; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    oa[i] = ((r < rows ? r : rows - 1) * (int32_t)KV + c_ld) * 16;
  }
#pragma unroll
  for (int i = 0; i < kLoadsB2; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    ob[i] = ((r < wrows ? r : wrows - 1) * (int32_t)KV + c_ld) * 16;
  }
  u32x4 ra[kLoads2], rb[kLoadsB2];
#define GLOAD_A(kt)                                                                            \
  _Pragma("unroll") for (int i = 0; i < kLoads2; ++i) ra[i] =                                  \
      __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, oa[i], (kt) * 128, 0));
#define GLOAD_B(kt)                                                                            \
  _Pragma("unroll") for (int i = 0; i < kLoadsB2; ++i) rb[i] =                                 \
      __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, ob[i], (kt) * 128, 0));
#define SWRITE_A(buf)                                                                          \
  _Pragma("unroll") for (int i = 0; i < kLoads2; ++i)                                          \
      sa[(buf) * kSlabA2 + swz((tid + i * kGemmThreads) / kChunks, c_ld)] = ra[i];
#define SWRITE_B(buf)                                                                          \
  _Pragma("unroll") for (int i = 0; i < kLoadsB2; ++i)                                         \
      sb[(buf) * kSlabB2 + swz((tid + i * kGemmThreads) / kChunks, c_ld)] = rb[i];
// NB: the wave's 32-row blocks that hold rows of the tile (the others are
// neither read nor multiplied); all four column blocks are always live
#define READK(FA, FB, buf, kk, NB)                                                             \
  {                                                                                            \
    const int c_ = (kk) * 2 + (lane >> 5);                                                     \
    _Pragma("unroll") for (int i = 0; i < (NB); ++i) FA[i] = __builtin_bit_cast(               \
        bf16x8, sa[(buf) * kSlabA2 + swz(wm * kWTM2 + i * 32 + (lane & 31), c_)]);            \
    _Pragma("unroll") for (int j = 0; j < kFN2; ++j) FB[j] = __builtin_bit_cast(               \
        bf16x8, sb[(buf) * kSlabB2 + swz(wn * kWTN2 + j * 32 + (lane & 31), c_)]);            \
  }
#define MFMAK(FA, FB, NB)                                                                      \
  _Pragma("unroll") for (int i = 0; i < (NB); ++i)                                             \
  _Pragma("unroll") for (int j = 0; j < kFN2; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0);
#define SGB(m, n) __builtin_amdgcn_sched_group_barrier(m, n, 0)
// Full blocks (NB = 4): the next step's 8 LDS reads over the first 8 of a
// step's 16 MFMAs ...
#define SCHED_READS(NB)                                                                        \
  if constexpr ((NB) == kFM2) {                                                                \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) { SGB(0x008, 1); SGB(0x100, 1); }            \
    SGB(0x008, 8);                                                                             \
  }
// ... and, in the first two steps, 8 LDS writes and 8 global loads over the
// other 8; waves with fewer live blocks are left to the compiler's schedule
#define SCHED_READS_WRITES_LOADS(NB)                                                           \
  if constexpr ((NB) == kFM2) {                                                                \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) { SGB(0x008, 1); SGB(0x100, 1); }            \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) { SGB(0x008, 1); SGB(0x200, 1); SGB(0x020, 1); } \
  }

  f32x16 acc[kFM2][kFN2];
#pragma unroll
  for (int i = 0; i < kFM2; ++i)
#pragma unroll
    for (int j = 0; j < kFN2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = K / kBK;
  bf16x8 fa0[kFM2], fb0[kFN2], fa1[kFM2], fb1[kFN2];
  GLOAD_A(0);
  GLOAD_B(0);
  SWRITE_A(0);
  SWRITE_B(0);
  if (KT > 1) {
    GLOAD_A(1);
    GLOAD_B(1);
  }
  __syncthreads();
  // The loop is compiled once per count of live 32-row blocks and each wave
  // runs its own (every copy has the same barriers); a tile of 18 rows costs
  // one block of MFMAs in one wave instead of sixteen.
#define WIDE_LOOP(NB)                                                                          \
  {                                                                                            \
    READK(fa0, fb0, 0, 0, NB);                                                                 \
    int kt = 0;                                                                                \
    for (; kt + 2 < KT; ++kt) { /* slab kt in LDS, slab kt + 1 in registers */                 \
      const int buf = kt & 1;                                                                  \
      READK(fa1, fb1, buf, 1, NB);                                                             \
      SWRITE_A(buf ^ 1);                                                                       \
      GLOAD_A(kt + 2);                                                                         \
      MFMAK(fa0, fb0, NB);                                                                     \
      SCHED_READS_WRITES_LOADS(NB);                                                            \
      READK(fa0, fb0, buf, 2, NB);                                                             \
      SWRITE_B(buf ^ 1);                                                                       \
      GLOAD_B(kt + 2);                                                                         \
      MFMAK(fa1, fb1, NB);                                                                     \
      SCHED_READS_WRITES_LOADS(NB);                                                            \
      READK(fa1, fb1, buf, 3, NB);                                                             \
      MFMAK(fa0, fb0, NB);                                                                     \
      SCHED_READS(NB);                                                                         \
      __syncthreads(); /* slab kt + 1 is in LDS; every wave is done reading slab kt */         \
      READK(fa0, fb0, buf ^ 1, 0, NB);                                                         \
      MFMAK(fa1, fb1, NB);                                                                     \
      SCHED_READS(NB);                                                                         \
    }                                                                                          \
    for (; kt < KT; ++kt) { /* the last two slabs (no more global loads) */                    \
      const int buf = kt & 1;                                                                  \
      READK(fa1, fb1, buf, 1, NB);                                                             \
      MFMAK(fa0, fb0, NB);                                                                     \
      READK(fa0, fb0, buf, 2, NB);                                                             \
      MFMAK(fa1, fb1, NB);                                                                     \
      READK(fa1, fb1, buf, 3, NB);                                                             \
      MFMAK(fa0, fb0, NB);                                                                     \
      if (kt + 1 < KT) {                                                                       \
        SWRITE_A(buf ^ 1);                                                                     \
        SWRITE_B(buf ^ 1);                                                                     \
        __syncthreads();                                                                       \
        READK(fa0, fb0, buf ^ 1, 0, NB);                                                       \
      }                                                                                        \
      MFMAK(fa1, fb1, NB);                                                                     \
    }                                                                                          \
  }
  const int live = (rows - wm * kWTM2 + 31) / 32;  // wave-uniform
  if (live >= kFM2) WIDE_LOOP(kFM2)
  else if (live == 3) WIDE_LOOP(3)
  else if (live == 2) WIDE_LOOP(2)
  else if (live == 1) WIDE_LOOP(1)
  else WIDE_LOOP(0)
#undef WIDE_LOOP
#undef SCHED_READS_WRITES_LOADS
#undef SCHED_READS
#undef SGB
#undef MFMAK
#undef READK
#undef SWRITE_B
#undef SWRITE_A
#undef GLOAD_B
#undef GLOAD_A

  wide_epilogue<GLU>(acc, lds, rows, row0, n0, N, Y, wm, wn, lane, tid);
}

// ---------------------------------------------------------------------------
// grouped GEMM on FP8 operands
//
// The rows come as the FP8 dispatch leaves them and the weights in the same
// format: OCP e4m3 codes, one fp32 scale per 128 of K (for a row of X, and
// for a row n of a weight matrix).  A code stands for code * scale, so
//   Y[row][n] = bf16( sum_b SX[row][b] * SW[n][b] * sum_{c in block b} X[row][c] * W[n][c] ).
// Same tiles, waves, XCD order and LDS geometry as k_grouped_gemm: a slab
// is 128 K-bytes, which is one scale block.  Per slab each wave runs two
// 64-deep steps of v_mfma_scale_f32_32x32x64_f8f6f4 (unit hardware scales)
// into a partial accumulator that starts at zero, then folds it into the
// running sum with the block's row and column scales:
//   acc += part * (SX[row][b] * SW[col][b])
// (the hardware block scales are powers of two, the format's are not, so the
// scales are applied on the vector ALU).  The slab's 128 row scales and 128
// column scales go through LDS beside the codes, in four rotating buffers
// so the fold can run after the barrier that publishes the next slab.

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kScaleBufs = 4;
constexpr int kF8Block = 128;  // K per scale; also the slab depth in bytes

// E8M0 exponent of a power-of-two fp32 scale; *bad is set if it is not one.
__device__ __forceinline__ uint32_t scale_exponent(float s, uint32_t *bad) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t e = b >> 23;  // a set sign bit makes it 256 or more
  // no branch: a mantissa bit, a sign, a zero or an all-ones exponent
  *bad |= (b & 0x007FFFFFu) | (uint32_t)(e - 1u > 0xFDu);
  return e & 0xFFu;
}

// WP2 (a group with power-of-two weight scales and amax row scales): each
// block's MFMAs take the weight columns' exponents as their B block scales,
// so the fold multiplies by the row scale alone (one FMA per element); a
// weight scale that is not a power of two raises kFlagScaleFormat.
template <bool GLU, bool WP2>
__global__ __launch_bounds__(kGemmThreads, 2) void k_grouped_gemm_fp8(
    const u32x4 *__restrict__ X, const float *__restrict__ SX, const u32x4 *__restrict__ W,
    const float *__restrict__ SW, const u32x4 *__restrict__ Wslot,
    const float *__restrict__ SWslot, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, int32_t max_tiles, int32_t K, int32_t N, int32_t E,
    int32_t n_col_tiles,
    uint16_t *__restrict__ Y, uint32_t *__restrict__ status) {
  __shared__ u32x4 sa[2][kTileM * kChunks];
  __shared__ u32x4 sb[2][kBN * kChunks];
  __shared__ __attribute__((aligned(16))) float ssc[kScaleBufs][kTileM + kBN];  // row, then column scales
  static_assert(kTileM + kBN == kGemmThreads, "one scale per thread per slab");
  int32_t tile, ctile;
  if (!balanced_tile(ntiles, max_tiles, n_col_tiles, tile, ctile)) return;
  const int32_t n0 = ctile * kBN;
  const int32_t row0 = tiles[tile * 4 + 0], rows = tiles[tile * 4 + 1], widx = tiles[tile * 4 + 2];
  const int64_t KV = K / 16;        // 16-byte vectors per row
  const int32_t NB = K / kF8Block;  // scales per row
  const bool own = widx < E;
  const int64_t wsel = own ? widx : widx - E;
  const u32x4 *Wm = (own ? W : Wslot) + wsel * N * KV;
  const float *SWm = (own ? SW : SWslot) + wsel * N * NB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wv / kWavesN, wn = wv % kWavesN;

  constexpr int kLoads = kTileM * kChunks / kGemmThreads;
  constexpr int kLoadsB = kBN * kChunks / kGemmThreads;
  const int c_ld = tid & (kChunks - 1);
  // Buffer loads: a scalar resource over the tile's rows and one 32-bit byte
  // offset per lane; rows past the end read the last row.  The library takes
  // K <= 2^24, so 128 rows of K bytes are at most 2^31: the record count is
  // formed in unsigned 32-bit arithmetic (the descriptor's field is unsigned)
  // and every offset stays below it.
  const u32x4 *Xt = X + (int64_t)row0 * KV;
  const u32x4 *Wt = Wm + (int64_t)n0 * KV;
  const int32_t wrows = N - n0 < kBN ? N - n0 : kBN;
  const int32_t nrec_x = (int32_t)((uint32_t)rows * (uint32_t)K);
  const int32_t nrec_w = (int32_t)((uint32_t)wrows * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rX =
      __builtin_amdgcn_make_buffer_rsrc((void *)Xt, (short)0, nrec_x, kBufDword3);
  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc((void *)Wt, (short)0, nrec_w, kBufDword3);
  uint32_t oa[kLoads], ob[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    oa[i] = (uint32_t)(((r < rows ? r : rows - 1) * KV + c_ld) * 16);
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int r = (tid + i * kGemmThreads) / kChunks;
    ob[i] = (uint32_t)(((r < wrows ? r : wrows - 1) * KV + c_ld) * 16);
  }
  // thread t < 128 stages the scale of tile row t, thread 128 + c that of column c
  const float *ps = tid < kTileM
                        ? SX + (int64_t)(row0 + (tid < rows ? tid : rows - 1)) * NB
                        : SWm + (int64_t)(n0 + tid - kTileM < N ? n0 + tid - kTileM : N - 1) * NB;
  u32x4 ra0[kLoads], rb0[kLoadsB];
  float rs;

#define GLOAD(kt)                                                                           \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i) ra0[i] = __builtin_bit_cast(             \
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, oa[i], (kt) * 128, 0));                   \
  _Pragma("unroll") for (int i = 0; i < kLoadsB; ++i) rb0[i] = __builtin_bit_cast(            \
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, ob[i], (kt) * 128, 0));                   \
  rs = ps[kt];
#define SWRITE(kt)                                                                            \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i)                                          \
      sa[(kt) & 1][swz((tid + i * kGemmThreads) / kChunks, c_ld)] = ra0[i];                   \
  _Pragma("unroll") for (int i = 0; i < kLoadsB; ++i)                                         \
      sb[(kt) & 1][swz((tid + i * kGemmThreads) / kChunks, c_ld)] = rb0[i];                   \
  ssc[(kt) % kScaleBufs][tid] = rs;

  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Step h (0, 1) of a slab: a lane of the upper half-wave takes chunks
  // 4h + 2, 4h + 3 of its row, the lower half chunks 4h, 4h + 1 (the same
  // K positions for A and B, which is all the product needs).
#define READK(FA, FB, buf, h, LB)                                                              \
  {                                                                                            \
    const int c_ = (h) * 4 + (lane >> 5) * 2;                                                  \
    _Pragma("unroll") for (int i = 0; i < (LB); ++i) {                                         \
      const int r_ = wm * kWTM + i * 32 + (lane & 31);                                         \
      const u32x4 lo = sa[buf][swz(r_, c_)], hi = sa[buf][swz(r_, c_ + 1)];                    \
      FA[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,                                \
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};                               \
    }                                                                                          \
    _Pragma("unroll") for (int j = 0; j < kFN; ++j) {                                          \
      const int r_ = wn * kWTN + j * 32 + (lane & 31);                                         \
      const u32x4 lo = sb[buf][swz(r_, c_)], hi = sb[buf][swz(r_, c_ + 1)];                    \
      FB[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,                                \
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};                               \
    }                                                                                          \
  }
  // One 32 x 32 output block over a whole slab (both 64-deep steps) into the
  // partial sum P.  cbsz = blgp = 0: both operands e4m3; scale exponents
  // 127: 2^0.
#define BLOCK(P, i, j)                                                                         \
  if constexpr (WP2) {                                                                         \
    P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0[i], fb0[j], f32x16{}, 0, 0, 0, 127, \
                                                        j, eb);                                \
    P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1[i], fb1[j], P, 0, 0, 0, 127, j, eb); \
  } else {                                                                                     \
    P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0[i], fb0[j], f32x16{}, 0, 0, 0, 127, \
                                                        0, 127);                               \
    P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1[i], fb1[j], P, 0, 0, 0, 127, 0, 127); \
  }
  // acc += P * (row scale * column scale); accumulator r of a lane is tile
  // row wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4, column wn*64 + j*32 + lane%32
#define FOLD(P, i, j)                                                                          \
  _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4)                                             \
  _Pragma("unroll") for (int q = 0; q < 4; ++q)                                                \
      acc[i][j][g4 * 4 + q] += WP2 ? P[g4 * 4 + q] * srow[g4][q]                               \
                                   : P[g4 * 4 + q] * (srow[g4][q] * scol[j]);
#define ROWSCALES(i)                                                                           \
  _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4) srow[g4] =                                  \
      *reinterpret_cast<const f32x4 *>(sc + wm * kWTM + (i) * 32 + g4 * 8 + (lane >> 5) * 4);

  static_assert(kChunks * 16 == kF8Block, "a slab is one scale block");
  static_assert(kFM == 2 && kFN == 2, "the block order below is written for 2 x 2 blocks");
  const int KT = K / kF8Block;
  // Both steps' fragments of a slab are held at once.  The four 32 x 32
  // blocks of a wave run one after another on two partial sums in turn, so
  // the fold of one block (vector ALU) is issued while the MFMAs of the next
  // are in flight; the last fold of a slab goes behind the barrier that
  // publishes the next one, and the next slab's fragments are read after it
  // (reading them before it needs more registers than two waves per SIMD
  // have).  sched_barrier keeps that order.
  i32x8 fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  f32x16 p0, p1;
  float scol[kFN];
  int eb = 0;          // WP2: the exponent bytes of the lane's two weight columns
  uint32_t bad = 0u;   // WP2: a weight scale that is not a power of two
  f32x4 srow[4];
  GLOAD(0);
  SWRITE(0);
  if (KT > 1) { GLOAD(1); }
  __syncthreads();
  // LB: the wave's 32-row blocks that hold rows of the tile; the loop is
  // compiled for 2, 1 and 0 of them (same barriers in every copy) and the
  // empty blocks are neither read, multiplied nor folded.
#define F8_LOOP(LB)                                                                            \
  {                                                                                            \
    READK(fa0, fb0, 0, 0, LB);                                                                 \
    READK(fa1, fb1, 0, 1, LB);                                                                 \
    for (int kt = 0; kt < KT; ++kt) {                                                          \
      const float *sc = ssc[kt % kScaleBufs];                                                  \
      if constexpr ((LB) > 0) {                                                                \
        _Pragma("unroll") for (int j = 0; j < kFN; ++j)                                        \
            scol[j] = sc[kTileM + wn * kWTN + j * 32 + (lane & 31)];                           \
        if constexpr (WP2)                                                                     \
          eb = (int)(scale_exponent(scol[0], &bad) | (scale_exponent(scol[1], &bad) << 8));    \
        ROWSCALES(0);                                                                          \
        BLOCK(p0, 0, 0);                                                                       \
        BLOCK(p1, 0, 1);                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        FOLD(p0, 0, 0);                                                                        \
      }                                                                                        \
      if constexpr ((LB) == 2) {                                                               \
        BLOCK(p0, 1, 0);                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        FOLD(p1, 0, 1);                                                                        \
        BLOCK(p1, 1, 1);                                                                       \
        ROWSCALES(1);                                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        FOLD(p0, 1, 0);                                                                        \
      } else if constexpr ((LB) == 1) {                                                        \
        FOLD(p1, 0, 1);                                                                        \
      }                                                                                        \
      if (kt + 1 < KT) {                                                                       \
        SWRITE(kt + 1);                                                                        \
        if (kt + 2 < KT) { GLOAD(kt + 2); }                                                    \
        __syncthreads();                                                                       \
      }                                                                                        \
      if constexpr ((LB) == 2) { FOLD(p1, 1, 1); }                                             \
      if (kt + 1 < KT) {                                                                       \
        READK(fa0, fb0, (kt + 1) & 1, 0, LB);                                                  \
        READK(fa1, fb1, (kt + 1) & 1, 1, LB);                                                  \
      }                                                                                        \
    }                                                                                          \
  }
  const int live = (rows - wm * kWTM + 31) / 32;  // wave-uniform
  if (live >= kFM) F8_LOOP(kFM)
  else if (live == 1) F8_LOOP(1)
  else F8_LOOP(0)
  if constexpr (WP2) {
    if (__ballot(bad != 0u) != 0u && lane == 0) atomicOr(status, kFlagScaleFormat);
  }
#undef F8_LOOP
#undef BLOCK
#undef FOLD
#undef ROWSCALES
#undef READK
#undef GLOAD
#undef SWRITE

  if (GLU || (N & 7) == 0) {   // a SwiGLU launch has N % 16 == 0
    // Through LDS: the tile as bf16 rows of 128, the 16-byte chunk of column c
    // of row r stored at chunk (c / 8) ^ (((r / 4) % 4) * 4), so the two
    // half-waves of a store (rows r and r + 4) land on different banks; then
    // 16-byte row stores.
    __syncthreads();   // every wave is done with the slab buffers
    uint16_t *so = reinterpret_cast<uint16_t *>(&sa[0][0]);
    static_assert(kTileM * kBN * 2 <= (int)sizeof(sa), "output tile fits the slab buffers");
#define OSW(r_, cv_) ((r_) * kBN + (((cv_) ^ ((((r_) >> 2) & 3) << 2)) << 3))
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int c = wn * kWTN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int rr = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
          so[OSW(rr, c >> 3) + (c & 7)] = (uint16_t)(p & 0xFFFFu);
          so[OSW(rr + 1, c >> 3) + (c & 7)] = (uint16_t)(p >> 16);
        }
      }
    __syncthreads();
    constexpr int kVecs = kTileM * kBN / 8;   // 16-byte vectors in the tile
#pragma unroll
    for (int q = 0; q < kVecs / kGemmThreads; ++q) {
      const int idx = tid + q * kGemmThreads;
      const int rr = idx / (kBN / 8), cv = idx % (kBN / 8);
      const int col = n0 + cv * 8;
      if (rr < rows && col < N) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(so + OSW(rr, cv));
        if constexpr (GLU)   // columns col .. col + 7 give outputs col / 2 .. col / 2 + 3
          *reinterpret_cast<uint2 *>(Y + (int64_t)(row0 + rr) * (N / 2) + col / 2) = swiglu4(v);
        else
          *reinterpret_cast<u32x4 *>(Y + (int64_t)(row0 + rr) * N + col) = v;
      }
    }
#undef OSW
    return;
  }

#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
        if (row < rows) Y[(int64_t)(row0 + row) * N + col] = (uint16_t)(p & 0xFFFFu);
        if (row + 1 < rows) Y[(int64_t)(row0 + row + 1) * N + col] = (uint16_t)(p >> 16);
      }
    }
}

// ---------------------------------------------------------------------------
// grouped GEMM on FP8 operands with power-of-two scales, 256 x 256 tiles
//
// When every scale is a power of two (the group's fp8_scales = POW2: the FP8
// dispatch and ep_quantize_fp8 then write such scales, and the caller's
// weight scales are such too), the matrix cores apply them:
// v_mfma_scale_f32_32x32x64_f8f6f4 takes one E8M0 exponent per lane for the
// 32 K-values the lane holds (A: the lane's row, B: its column), and both
// 64-deep steps of a 128-deep slab lie in one scale block, so
// SX[row][b] * SW[col][b] is applied exactly inside the MFMA and the
// accumulators run over the whole of K with no vector-ALU fold.  Tiles, waves,
// XCD order and LDS geometry are the bf16 wide kernel's (a 128-deep slab of
// codes is 128 bytes per row, as a 64-deep bf16 slab), with two 64-deep steps
// per slab.  The slabs travel differently: each goes from global memory
// straight into LDS (buffer loads issued from asm, two buffers), the one
// after next issued as soon as its buffer is free, with explicit waits before
// the barrier that publishes a slab.  Each slab's 256 row and 256 column
// scales go into LDS the same way, as fp32; a lane turns the eight it needs
// (its four row blocks' and its four column blocks') into exponent bytes
// packed in two words, and the MFMA's byte select (op_sel) picks them.
// A scale that is not a positive normal power of two raises
// EP_FLAG_SCALE_FORMAT (its block is then computed at 2 to the scale's
// exponent).

constexpr int kF8KV = kF8Block / 16;   // 16-byte chunks per row of a slab (= kChunks)
static_assert(kF8KV == kChunks, "an FP8 slab row is 128 bytes, as a bf16 one");

// One step's 16 (or fewer) MFMAs of a wave: rows blocks I < NB, all column
// blocks; byte I of ea and byte J of eb are the blocks' scale exponents.
template <int I, int NB>
__device__ __forceinline__ void mfma8_rows(f32x16 (&acc)[kFM2][kFN2], const i32x8 (&fa)[kFM2],
                                           const i32x8 (&fb)[kFN2], int ea, int eb) {
  if constexpr (I < NB) {
    acc[I][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[I], fb[0], acc[I][0], 0, 0, I, ea, 0, eb);
    acc[I][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[I], fb[1], acc[I][1], 0, 0, I, ea, 1, eb);
    acc[I][2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[I], fb[2], acc[I][2], 0, 0, I, ea, 2, eb);
    acc[I][3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[I], fb[3], acc[I][3], 0, 0, I, ea, 3, eb);
    mfma8_rows<I + 1, NB>(acc, fa, fb, ea, eb);
  }
}
static_assert(kFN2 == 4, "mfma8_rows writes four column blocks");


#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// A buffer load whose lanes' 16 (or 4) bytes land in LDS at m0 + lane * 16
// (or 4), m0 being the wave's LDS base.  Written in asm on purpose: the
// compiler tracks its own form of this load and, unable to tell which part
// of LDS it writes, makes every later LDS read wait until it has landed --
// which would let no slab load run under the MFMAs of the previous slab.
// Here the caller owns the waits (s_waitcnt vmcnt before the barrier that
// publishes the data).  No result register: nothing the compiler allocates
// is written late.  The s_nop is the wait state the hardware needs between
// the write of m0 and the load that reads it.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base,
                                           uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base,
                                          uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_base) : "memory");
}

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_fp8_256(
    const u32x4 *__restrict__ X, const float *__restrict__ SX, const u32x4 *__restrict__ W,
    const float *__restrict__ SW, const u32x4 *__restrict__ Wslot,
    const float *__restrict__ SWslot, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, int32_t max_tiles, int32_t K, int32_t N, int32_t E,
    int32_t n_col_tiles, uint16_t *__restrict__ Y, uint32_t *__restrict__ status) {
  // two 128-deep slabs of X and W codes (128 KB), later the bf16 output tile;
  // the slabs' fp32 scales: [buffer][256 row scales, 256 column scales]
  __shared__ u32x4 lds[2 * kSlabA2 + 2 * kSlabB2];
  __shared__ float ssc[2][2 * kBM2];
  static_assert(kBM2 * kBN2 * 2 <= (int)sizeof(lds), "output tile fits the slab buffers");
  static_assert(kBM2 == kBN2 && kBM2 == kGemmThreads, "one row and one column scale per thread");
  u32x4 *const sa = lds, *const sb = lds + 2 * kSlabA2;
  int32_t tile, ctile;
  if (!balanced_tile(ntiles, max_tiles, n_col_tiles, tile, ctile)) return;
  const int32_t n0 = ctile * kBN2;
  const int32_t row0 = tiles[tile * 4 + 0], rows = tiles[tile * 4 + 1], widx = tiles[tile * 4 + 2];
  const int32_t KV = K / 16;        // 16-byte vectors per row of codes
  const int32_t NB = K / kF8Block;  // scales per row
  const bool own = widx < E;
  const int64_t wsel = own ? widx : widx - E;
  const int32_t wrows = N - n0 < kBN2 ? N - n0 : kBN2;
  // buffer resources over the tile's rows of codes and of scales (every
  // offset in range by construction: rows past the end read the last row)
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(X + (int64_t)row0 * KV), (short)0, rows * K, kBufDword3);
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((own ? W : Wslot) + wsel * N * KV + (int64_t)n0 * KV), (short)0, wrows * K,
      kBufDword3);
  const __amdgpu_buffer_rsrc_t rSX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(SX + (int64_t)row0 * NB), (short)0, rows * NB * 4, kBufDword3);
  const __amdgpu_buffer_rsrc_t rSW = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((own ? SW : SWslot) + wsel * N * NB + (int64_t)n0 * NB), (short)0, wrows * NB * 4,
      kBufDword3);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wv >> 1, wn = wv & 1;
  // The loads go straight into LDS: load i of wave wv fills the 64 16-byte
  // slots i*256 + wv*64 + lane, slot q holding chunk (q % 8) ^ ((r / 2) % 8)
  // of row r = q / 8 -- the chunk swizzle the fragment reads expect.
  uint32_t oa[kLoads2], ob[kLoadsB2];
#pragma unroll
  for (int i = 0; i < kLoads2; ++i) {
    const int q = i * kGemmThreads + tid, r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    oa[i] = (uint32_t)(((r < rows ? r : rows - 1) * KV + c) * 16);
  }
#pragma unroll
  for (int i = 0; i < kLoadsB2; ++i) {
    const int q = i * kGemmThreads + tid, r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    ob[i] = (uint32_t)(((r < wrows ? r : wrows - 1) * KV + c) * 16);
  }
  const uint32_t osx = (uint32_t)((tid < rows ? tid : rows - 1) * NB * 4);
  const uint32_t osw = (uint32_t)((tid < wrows ? tid : wrows - 1) * NB * 4);
  // The waits before the barriers that publish a slab are explicit
  // (s_waitcnt vmcnt, then s_barrier): the loads are issued from asm (see
  // lds_load16), so the compiler neither counts nor waits for them.
#define LDS_ADDR(p) ((uint32_t)(size_t)LDS_PTR(p))
#define F8W_ISSUE(kt, buf)                                                                     \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < kLoads2; ++i) lds_load16(                            \
        rX, LDS_ADDR(&sa[(buf) * kSlabA2 + i * kGemmThreads + wv * 64]), oa[i], (kt) * 128);   \
    _Pragma("unroll") for (int i = 0; i < kLoadsB2; ++i) lds_load16(                           \
        rW, LDS_ADDR(&sb[(buf) * kSlabB2 + i * kGemmThreads + wv * 64]), ob[i], (kt) * 128);   \
    lds_load4(rSX, LDS_ADDR(&ssc[buf][wv * 64]), osx, (kt) * 4);                               \
    lds_load4(rSW, LDS_ADDR(&ssc[buf][kBM2 + wv * 64]), osw, (kt) * 4);                        \
  }
  static_assert(kLoads2 + kLoadsB2 + 2 == 18, "the waits below count 18 loads per slab");
// step h (0 or 1) of a slab: the lane's 32 K-values of its row (A) or column
// (B) are chunks h*4 + (lane/32)*2 and the next one
#define READK8(FA, FB, buf, h, NBK)                                                            \
  {                                                                                            \
    const int c_ = (h) * 4 + (lane >> 5) * 2;                                                  \
    _Pragma("unroll") for (int i = 0; i < (NBK); ++i) {                                        \
      const int r_ = wm * kWTM2 + i * 32 + (lane & 31);                                        \
      const u32x4 lo = sa[(buf) * kSlabA2 + swz(r_, c_)];                                      \
      const u32x4 hi = sa[(buf) * kSlabA2 + swz(r_, c_ + 1)];                                  \
      FA[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,                                \
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};                               \
    }                                                                                          \
    _Pragma("unroll") for (int j = 0; j < kFN2; ++j) {                                         \
      const int r_ = wn * kWTN2 + j * 32 + (lane & 31);                                        \
      const u32x4 lo = sb[(buf) * kSlabB2 + swz(r_, c_)];                                      \
      const u32x4 hi = sb[(buf) * kSlabB2 + swz(r_, c_ + 1)];                                  \
      FB[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,                                \
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};                               \
    }                                                                                          \
  }
// the exponents of the lane's four row blocks (byte i: row wm*128 + i*32 +
// lane%32) and of its four column blocks
#define READE(EA, EB, buf)                                                                     \
  {                                                                                            \
    uint32_t ea_ = 0u, eb_ = 0u;                                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
      ea_ |= scale_exponent(ssc[buf][wm * kWTM2 + i * 32 + (lane & 31)], &bad) << (8 * i);     \
      eb_ |= scale_exponent(ssc[buf][kBM2 + wn * kWTN2 + i * 32 + (lane & 31)], &bad) << (8 * i); \
    }                                                                                          \
    EA = (int)ea_;                                                                             \
    EB = (int)eb_;                                                                             \
  }

  f32x16 acc[kFM2][kFN2];
#pragma unroll
  for (int i = 0; i < kFM2; ++i)
#pragma unroll
    for (int j = 0; j < kFN2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = K / kF8Block;
  uint32_t bad = 0u;
  i32x8 fa0[kFM2], fb0[kFN2], fa1[kFM2], fb1[kFN2];
  int ea, eb, ea_n = 0, eb_n = 0;
  // Each wave waits for its own loads, then the barrier publishes every
  // wave's share.  The asm reads one element of each accumulator: the MFMAs
  // touch no memory, and without that data dependence the compiler moves
  // most of a step's MFMAs past the wait they are meant to hide.
#define F8W_SYNC(VM)                                                                           \
  asm volatile("s_waitcnt vmcnt(" #VM ") lgkmcnt(0)\n\ts_barrier"                             \
               :: "a"(acc[0][0][0]), "a"(acc[0][1][0]), "a"(acc[0][2][0]), "a"(acc[0][3][0]),  \
                  "a"(acc[1][0][0]), "a"(acc[1][1][0]), "a"(acc[1][2][0]), "a"(acc[1][3][0]),  \
                  "a"(acc[2][0][0]), "a"(acc[2][1][0]), "a"(acc[2][2][0]), "a"(acc[2][3][0]),  \
                  "a"(acc[3][0][0]), "a"(acc[3][1][0]), "a"(acc[3][2][0]), "a"(acc[3][3][0])   \
               : "memory")
  static_assert(kFM2 == 4 && kFN2 == 4, "the barrier names each of the 16 accumulators");
  F8W_ISSUE(0, 0);
  if (KT > 1) {
    F8W_ISSUE(1, 1);
    F8W_SYNC(18);   // slab 0 landed
  } else {
    F8W_SYNC(0);
  }
  // Slab kt is in buffer kt & 1 and slab kt + 1 on its way into the other;
  // step 0's fragments and the slab's exponents were read after the barrier
  // that published slab kt.  Step 1's reads go out, then step 0's MFMAs;
  // then the barrier (slab kt + 1 landed, slab kt read by every wave), the
  // loads of slab kt + 2 into the buffer just freed, the reads of slab
  // kt + 1's step 0 and step 1's MFMAs.  The last two slabs are peeled off,
  // so the body has no branch the compiler could move MFMAs across.
  // (Half-slabs in four buffers, loaded three ahead, measured 1.6 times
  // slower.)  Compiled once per count of the wave's live 32-row blocks (the
  // same barriers in every copy).
#define SGB8(m, n) __builtin_amdgcn_sched_group_barrier(m, n, 0)
// before the barrier: one LDS read after each MFMA
#define F8W_INTERLEAVE_A(NBK)                                                                  \
  if constexpr ((NBK) == kFM2) {                                                               \
    _Pragma("unroll") for (int q_ = 0; q_ < 16; ++q_) { SGB8(0x008, 1); SGB8(0x100, 1); }      \
  }
// after it: three LDS reads after each of the first 8 MFMAs, then the
// exponent arithmetic spread over the last 8
#define F8W_INTERLEAVE_B(NBK)                                                                  \
  if constexpr ((NBK) == kFM2) {                                                               \
    _Pragma("unroll") for (int q_ = 0; q_ < 8; ++q_) { SGB8(0x008, 1); SGB8(0x100, 3); }       \
    _Pragma("unroll") for (int q_ = 0; q_ < 8; ++q_) { SGB8(0x008, 1); SGB8(0x002, 6); }       \
  }
#define F8W_SLAB(NBK, ISSUE)                                                                   \
  {                                                                                            \
    const int buf = kt & 1;                                                                    \
    READK8(fa1, fb1, buf, 1, NBK);                                                             \
    mfma8_rows<0, NBK>(acc, fa0, fb0, ea, eb);                                                 \
    F8W_INTERLEAVE_A(NBK);                                                                     \
    F8W_SYNC(0);                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    if (ISSUE) F8W_ISSUE(kt + 2, buf);                                                         \
    READK8(fa0, fb0, buf ^ 1, 0, NBK);                                                         \
    READE(ea_n, eb_n, buf ^ 1);                                                                \
    mfma8_rows<0, NBK>(acc, fa1, fb1, ea, eb);                                                 \
    F8W_INTERLEAVE_B(NBK);                                                                     \
    ea = ea_n;                                                                                 \
    eb = eb_n;                                                                                 \
  }
#define F8W_LOOP(NBK)                                                                          \
  {                                                                                            \
    READK8(fa0, fb0, 0, 0, NBK);                                                               \
    READE(ea, eb, 0);                                                                          \
    int kt = 0;                                                                                \
    for (; kt + 2 < KT; ++kt) F8W_SLAB(NBK, true)                                              \
    if (kt + 1 < KT) {                                                                         \
      F8W_SLAB(NBK, false)                                                                     \
      ++kt;                                                                                    \
    }                                                                                          \
    READK8(fa1, fb1, kt & 1, 1, NBK);                                                          \
    mfma8_rows<0, NBK>(acc, fa0, fb0, ea, eb);                                                 \
    mfma8_rows<0, NBK>(acc, fa1, fb1, ea, eb);                                                 \
  }
  const int live = (rows - wm * kWTM2 + 31) / 32;  // wave-uniform
  if (live >= kFM2) F8W_LOOP(kFM2)
  else if (live == 3) F8W_LOOP(3)
  else if (live == 2) F8W_LOOP(2)
  else if (live == 1) F8W_LOOP(1)
  else F8W_LOOP(0)
#undef F8W_LOOP
#undef F8W_SLAB
#undef F8W_INTERLEAVE_A
#undef F8W_INTERLEAVE_B
#undef SGB8
#undef F8W_SYNC
#undef READE
#undef READK8
#undef F8W_ISSUE
#undef LDS_ADDR
  const uint64_t any_bad = __ballot(bad != 0u);
  if (any_bad != 0u && lane == 0) atomicOr(status, kFlagScaleFormat);
  wide_epilogue<GLU>(acc, lds, rows, row0, n0, N, Y, wm, wn, lane, tid);
}
#undef LDS_PTR

// Row tiles of kTileM rows the plan can produce; the 256-row tiling needs no more.
int32_t gemm_max_tiles(const Geometry &g) {
  const int64_t groups = g.layout == kStatic ? 2 * (int64_t)g.E + g.R : g.E;
  return (int32_t)((g.n + kTileM - 1) / kTileM + groups);
}

// The 256 x 256 kernel pays off once the groups fill its row tiles: at
// least 128 receive rows per expert on average, and N of a full column tile.
// Its buffer offsets are 32-bit: a tile's rows of X must span under 2 GiB.
// the epilogue is a template parameter: plain bf16 output or SwiGLU pairs
#define GEMM_LAUNCH(KERN, ...)                                \
  do {                                                        \
    if (glu) hipLaunchKernelGGL(KERN<true>, __VA_ARGS__);     \
    else hipLaunchKernelGGL(KERN<false>, __VA_ARGS__);        \
  } while (0)

// Workgroups of a GEMM launch: per XCD, room for an eighth of each kind of
// row tile rounded up (at most max_tiles / 8 + 2 row tiles), times the
// column tiles (balanced_tile).
static unsigned gemm_grid(int32_t max_tiles, int32_t ncol) {
  return (unsigned)((int64_t)kXcds * (max_tiles / kXcds + 2) * ncol);
}

static bool gemm_uses_wide_tiles(const Geometry &g, int32_t K, int32_t N) {
  return N >= kBN2 && g.n >= (int64_t)(kBM2 / 2) * g.E && (int64_t)kBM2 * K * 2 <= INT32_MAX;
}

// The FP8 256 x 256 kernel needs power-of-two scales (the group's format)
// and at least 128 rows per expert on average; its buffer offsets over a
// tile's codes are 32-bit as well.
static bool gemm_fp8_uses_wide_tiles(const Geometry &g, int32_t K, int32_t N) {
  return g.fp8_pow2 == 1 && N >= kBN2 && g.n >= (int64_t)(kBM2 / 2) * g.E &&
         (int64_t)kBM2 * K <= INT32_MAX;
}

// At most as many 256-row tiles as the table holds 128-row ones.
static int32_t wide_max_tiles(const Geometry &g) {
  const int64_t groups = g.layout == kStatic ? 2 * (int64_t)g.E + g.R : g.E;
  return (int32_t)((g.n + kBM2 - 1) / kBM2 + groups);
}

hipError_t launch_grouped_gemm(const Geometry &g, const Workspace &ws, const uint16_t *x,
                               const uint16_t *w, const uint16_t *wslot, int32_t K, int32_t N,
                               uint16_t *y, bool glu, hipStream_t s) {
  const int32_t max_tiles = gemm_max_tiles(g);
  if (max_tiles == 0 || N == 0) return hipSuccess;
  TileArgs ta{g, ws, wslot != nullptr ? 1 : 0};
  if (gemm_uses_wide_tiles(g, K, N)) {
    const int32_t max2 = wide_max_tiles(g);
    hipLaunchKernelGGL((k_gemm_tiles<kBM2, true>), dim3(1), dim3(1024), 0, s, ta, max2);
    const int32_t ncol = (N + kBN2 - 1) / kBN2;
    GEMM_LAUNCH(k_grouped_gemm_256, dim3(gemm_grid(max2, ncol)), dim3(kGemmThreads), 0, s,
                       reinterpret_cast<const u32x4 *>(x), reinterpret_cast<const u32x4 *>(w),
                       reinterpret_cast<const u32x4 *>(wslot), ws.gemm_tiles, ws.gemm_ntiles, max2,
                       K, N, g.E, ncol, y);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_tiles<kTileM, false>), dim3(1), dim3(1024), 0, s, ta, max_tiles);
  const int32_t ncol = (N + kBN - 1) / kBN;
  GEMM_LAUNCH(k_grouped_gemm, dim3(gemm_grid(max_tiles, ncol)), dim3(kGemmThreads), 0, s,
                     reinterpret_cast<const u32x4 *>(x), reinterpret_cast<const u32x4 *>(w),
                     reinterpret_cast<const u32x4 *>(wslot), ws.gemm_tiles, ws.gemm_ntiles,
                     max_tiles, K, N, g.E, ncol, y);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_fp8(const Geometry &g, const Workspace &ws, const uint8_t *x,
                                   const float *sx, const uint8_t *w, const float *sw,
                                   const uint8_t *wslot, const float *swslot, int32_t K, int32_t N,
                                   uint16_t *y, bool glu, hipStream_t s) {
  const int32_t max_tiles = gemm_max_tiles(g);
  if (max_tiles == 0 || N == 0) return hipSuccess;
  TileArgs ta{g, ws, wslot != nullptr ? 1 : 0};
  if (gemm_fp8_uses_wide_tiles(g, K, N)) {
    const int32_t max2 = wide_max_tiles(g);
    hipLaunchKernelGGL((k_gemm_tiles<kBM2, true>), dim3(1), dim3(1024), 0, s, ta, max2);
    const int32_t ncol = (N + kBN2 - 1) / kBN2;
    GEMM_LAUNCH(k_grouped_gemm_fp8_256, dim3(gemm_grid(max2, ncol)), dim3(kGemmThreads), 0, s,
                reinterpret_cast<const u32x4 *>(x), sx, reinterpret_cast<const u32x4 *>(w), sw,
                reinterpret_cast<const u32x4 *>(wslot), swslot, ws.gemm_tiles, ws.gemm_ntiles,
                max2, K, N, g.E, ncol, y, ws.status);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_tiles<kTileM, false>), dim3(1), dim3(1024), 0, s, ta, max_tiles);
  const int32_t ncol = (N + kBN - 1) / kBN;
#define F8_ARGS                                                                                \
  dim3(gemm_grid(max_tiles, ncol)), dim3(kGemmThreads), 0, s, reinterpret_cast<const u32x4 *>(x), sx, \
      reinterpret_cast<const u32x4 *>(w), sw, reinterpret_cast<const u32x4 *>(wslot), swslot,       \
      ws.gemm_tiles, ws.gemm_ntiles, max_tiles, K, N, g.E, ncol, y, ws.status
  if (g.fp8_pow2 == 2) {
    if (glu) hipLaunchKernelGGL((k_grouped_gemm_fp8<true, true>), F8_ARGS);
    else hipLaunchKernelGGL((k_grouped_gemm_fp8<false, true>), F8_ARGS);
  } else {
    if (glu) hipLaunchKernelGGL((k_grouped_gemm_fp8<true, false>), F8_ARGS);
    else hipLaunchKernelGGL((k_grouped_gemm_fp8<false, false>), F8_ARGS);
  }
#undef F8_ARGS
  return hipGetLastError();
}

}  // namespace epk
