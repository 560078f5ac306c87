// ep_internal.h -- internal declarations shared by the C ABI (ep_api.cpp) and
// the gfx950 kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace epk {

// Layout tile: 16 waves x 2 chunks x 64 lanes of flat entries t*k + j.
constexpr int kTileThreads = 1024;
constexpr int kTileWaves = kTileThreads / 64;
constexpr int kTileChunks = 2;
constexpr int kTileEntries = kTileThreads * kTileChunks;  // 2048
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kLdsLimit = 65536;
constexpr int kGemmBM = 128;  // rows of the smaller grouped-GEMM tile (sizes the tile table)
constexpr size_t kScratchBytes = EP_SCRATCH_BYTES;  // the static scratch (scratch.hip)

constexpr uint32_t kFlagIndexRange = 1u;
constexpr uint32_t kFlagCapacity = 2u;
constexpr uint32_t kFlagSlotBudget = 4u;
constexpr uint32_t kFlagPlanStall = 8u;
constexpr uint32_t kFlagScaleFormat = 16u;

enum Layout : int32_t { kLL = 0, kHT = 1, kStatic = 2 };

// Device tables carved out of the caller's workspace (each 256-byte aligned).
struct Workspace {
  uint32_t *status;      // [1]  EP_FLAG_* bits
  uint32_t *ticket;      // [1]  blocks of the layout kernel that finished (two-launch layout)
  // resident-tiles layout handshake (see plan.hip): words only grow or carry
  // the epoch mark of the call that wrote them, so no call resets them
  uint64_t *arrive;      // [1]  tiles that published their histogram, over all calls
  uint32_t *stall;       // [1]  epoch mark of the last call in which a tile's wait ran out
  uint64_t *tagged;      // [ntiles][E] histograms, then [ntiles] flags: (mark << 32) | value
  int32_t *counts;       // [E]
  int32_t *offsets;      // [E+1]
  int32_t *eidx;         // [n]  validated expert id of each entry (-1 = skipped)
  int32_t *lrank;        // [n]  position of the entry among its expert's entries in its tile
  int32_t *dst;          // [n]
  int32_t *tile_hist;    // [ntiles][E] per-tile counts, then per-tile exclusive bases
  uint32_t *tile_flags;  // [ntiles]
  int32_t *recv_src;     // [rows]
  // STATIC plan
  int32_t *keep, *native_row, *seg_first, *seg_count;  // [E] each
  int32_t *segments;     // [(E+R)*5]
  int32_t *n_segments;   // [1]
  int32_t *load;         // [R]
  int32_t *replica;      // [R*S]
  int32_t *seg_slot;     // [E+R] slot of each segment on its rank, -1 if none
  // grouped GEMM
  int32_t *gemm_tiles;   // [gemm_max_tiles][4] row0, rows, weight index, 0 (full tiles
                         // from the front, short ones from the back)
  int32_t *gemm_ntiles;  // [2] all tiles, full tiles
};

struct Geometry {
  int32_t T, k, E, R, S, layout, cap;
  int32_t slot_mode;  // 0 training (overflow flags SLOT_BUDGET), 1 inference
  int32_t stores;     // dispatch stores: 0 by size, 1 cached, 2 non-temporal
  int32_t in_flight;  // passes of the group at once (>= 1): the size rule counts all their rows
  int32_t cstores;    // combine's token rows: 0 or 1 cached, 2 non-temporal
  int32_t fp8_pow2;   // ep_fp8_scales_t: 1 every FP8 scale a power of two, 2 the weights' only
  int32_t C;        // STATIC rows per rank
  int32_t ntiles;   // layout tiles (>= 1)
  int32_t cus;      // compute units of the device (0 if unknown): the most tiles one launch finishes
  int32_t nbits;    // bits of an expert id, >= 1
  int64_t n;        // T*k
  int64_t rows;     // receive rows
};

// Pieces each token row is split into by dispatch and combine (small batches
// spread one row over several workgroups); *chunk = 16-byte vectors per piece.
int32_t row_pieces(int32_t T, int32_t V, int32_t *chunk);

// Byte size of the workspace for `g` (base == nullptr) or carve it (base != nullptr).
size_t carve_workspace(const Geometry &g, char *base, Workspace *ws);
size_t plan_lds_bytes(int32_t E, int32_t R);

// Launchers (return the HIP error of the launch).
hipError_t launch_plan(const Geometry &g, const Workspace &ws, const int32_t *topk_idx,
                       hipStream_t s);
// routing (launch_route's rule) and the layout of its ids in one layout
// launch when E allows, else routing then layout
hipError_t launch_route_plan(const Geometry &g, const Workspace &ws, const float *logits,
                             int32_t *idx, float *w, hipStream_t s);
// dispatch; with fused (fused_layout_fits(g)) the layout of idx is placed in
// the same launch (the tables ep_plan would write)
bool fused_layout_fits(const Geometry &g);
hipError_t launch_dispatch_bf16(const Geometry &g, const Workspace &ws, const uint16_t *x,
                                int32_t H, uint16_t *recv, hipStream_t s,
                                const int32_t *idx = nullptr, bool fused = false);
hipError_t launch_dispatch_fp8(const Geometry &g, const Workspace &ws, const uint16_t *x,
                               int32_t H, uint8_t *recv_q, float *recv_scale, hipStream_t s,
                               const int32_t *idx = nullptr, bool fused = false);
// rows x K bf16 to e4m3 codes + fp32 scales per 128 (the FP8 dispatch's recipe)
hipError_t launch_quantize_fp8(const uint16_t *x, int64_t rows, int32_t K, uint8_t *q,
                               float *scales, bool pow2, hipStream_t s);
hipError_t launch_recv_meta(const Geometry &g, const Workspace &ws, const float *topk_w,
                            int32_t *recv_idx, float *recv_w, hipStream_t s);
hipError_t launch_combine(const Geometry &g, const Workspace &ws, const uint16_t *rows,
                          int32_t H, const float *topk_w, void *out, bool out_fp32,
                          hipStream_t s);
hipError_t launch_combine_bwd(const Geometry &g, const Workspace &ws, const uint16_t *gy,
                              const uint16_t *expert_out, int32_t H, const float *topk_w,
                              uint16_t *grad_out, float *grad_w, hipStream_t s);
hipError_t launch_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx,
                        float *w, hipStream_t s);
hipError_t launch_prefetch(const Geometry &g, const Workspace &ws, const uint8_t *weights,
                           int64_t row_bytes, uint8_t *slots, hipStream_t s);
int32_t gemm_max_tiles(const Geometry &g);
hipError_t launch_grouped_gemm(const Geometry &g, const Workspace &ws, const uint16_t *x,
                               const uint16_t *w, const uint16_t *wslot, int32_t K, int32_t N,
                               uint16_t *y, bool glu, hipStream_t s);
hipError_t launch_grouped_gemm_fp8(const Geometry &g, const Workspace &ws, const uint8_t *x,
                                   const float *sx, const uint8_t *w, const float *sw,
                                   const uint8_t *wslot, const float *swslot, int32_t K, int32_t N,
                                   uint16_t *y, bool glu, hipStream_t s);
// static scratch (scratch.hip): device address on the current device, and a
// zero-filling kernel
hipError_t scratch_base(int *dev, void **base);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_dup_reduce(const uint16_t *rep, const int32_t *rep_e, int32_t n, int64_t P,
                             int32_t E_owner, float *owner, uint32_t *status, hipStream_t s);

}  // namespace epk
