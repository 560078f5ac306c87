// ep_api.cpp -- the C ABI declared in include/ep.h: argument validation,
// group and handle bookkeeping, workspace carving and kernel selection.
// Every check happens on the host before anything is enqueued; the only
// HIP calls are the kernel launches and, in ep_handle_status, one copy and
// one stream synchronisation.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "ep.h"
#include "ep_internal.h"

struct ep_group {
  ep_group_config_t cfg;
  int32_t nbits;
};

struct ep_handle {
  ep_group *g;
  epk::Geometry geo;
  epk::Workspace ws;
  char *base;
  size_t bytes;
  bool planned;
  bool in_scratch;  // made by ep_handle_create_static: static storage, library scratch
};

namespace {
// The handles ep_handle_create_static returns: one per device, in static
// storage, so making one allocates nothing on the host either.
constexpr int kMaxScratchHandles = 64;
ep_handle g_scratch_handles[kMaxScratchHandles];
}  // namespace

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kFp8GemmMaxK = (int64_t)1 << 24;  // bytes per row of an FP8 GEMM operand

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

epk::Geometry make_geometry(const ep_group *g, int32_t T) {
  const ep_group_config_t &c = g->cfg;
  epk::Geometry geo{};
  geo.T = T;
  geo.k = c.top_k;
  geo.E = c.num_experts;
  geo.R = c.num_ranks;
  geo.S = c.slots_per_rank;
  geo.slot_mode = c.slot_mode;
  geo.stores = c.dispatch_stores;
  geo.in_flight = c.passes_in_flight > 1 ? c.passes_in_flight : 1;
  geo.cstores = c.combine_stores;
  geo.fp8_pow2 = c.fp8_scales;   // 0 AMAX, 1 POW2, 2 AMAX rows with POW2 weights
  geo.layout = c.layout;
  geo.cap = c.capacity;
  geo.n = (int64_t)T * c.top_k;
  geo.C = (int32_t)((geo.n + c.num_ranks - 1) / c.num_ranks);
  const int64_t tiles = (geo.n + epk::kTileEntries - 1) / epk::kTileEntries;
  geo.ntiles = (int32_t)(tiles > 0 ? tiles : 1);
  geo.nbits = g->nbits;
  if (c.layout == EP_LAYOUT_HT) geo.rows = geo.n;
  else if (c.layout == EP_LAYOUT_LL) geo.rows = (int64_t)c.num_experts * c.capacity;
  else geo.rows = (int64_t)c.num_ranks * geo.C;
  return geo;
}

int64_t numel(const ep_tensor_t *t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->sizes[i];
  return n;
}

// Generic checks: non-NULL, tag, dtype, ndim in 1..4, sizes >= 0, data set and aligned.
ep_status_t check_tensor(const ep_tensor_t *t, int32_t tag, int32_t dtype) {
  if (!t) return EP_ERR_INVALID_ARG;
  if (t->tag != tag) return EP_ERR_BAD_TAG;
  if (t->dtype != dtype) return EP_ERR_BAD_DTYPE;
  if (t->ndim < 1 || t->ndim > 4 || t->reserved != 0) return EP_ERR_BAD_SHAPE;
  for (int i = 0; i < t->ndim; ++i)
    if (t->sizes[i] < 0) return EP_ERR_BAD_SHAPE;
  if (!t->data && numel(t) > 0) return EP_ERR_INVALID_ARG;
  // rows of tokens, expert weights and gradients move as 16-byte vectors;
  // ids, router weights, logits and scales as 4-byte words
  const uintptr_t need =
      (tag == EP_TAG_TOKENS || tag == EP_TAG_EXPERT_WEIGHTS || tag == EP_TAG_EXPERT_GRADS) ? 16 : 4;
  if (reinterpret_cast<uintptr_t>(t->data) % need != 0) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

// Exactly [d0, d1] as a 2D tensor.
bool is_2d(const ep_tensor_t *t, int64_t d0, int64_t d1) {
  return t->ndim == 2 && t->sizes[0] == d0 && t->sizes[1] == d1;
}

// Leading sizes multiply to `rows`, last size `last` (any ndim >= 2), or a
// 1D tensor of `rows` elements when last == 1 and allow_1d.
bool is_rows(const ep_tensor_t *t, int64_t rows, int64_t last, bool allow_1d = false) {
  if (allow_1d && t->ndim == 1) return last == 1 && t->sizes[0] == rows;
  if (t->ndim < 2) return false;
  int64_t lead = 1;
  for (int i = 0; i + 1 < t->ndim; ++i) lead *= t->sizes[i];
  return lead == rows && t->sizes[t->ndim - 1] == last;
}

ep_status_t hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Compute units of the current device: a layout of at most that many tiles
// runs as one launch with every tile resident.  0 when there is no device (the
// layout then takes its two-launch form); a failed query's error is cleared
// so no later launch reports it.
int32_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace epk {

size_t carve_workspace(const Geometry &g, char *base, Workspace *ws) {
  size_t off = 0;
  Workspace w{};
  auto take = [&](size_t bytes) -> char * {
    char *p = base ? base + off : nullptr;
    off += align_up(bytes > 0 ? bytes : 1);
    return p;
  };
  char *hdr = take(kAlign);
  w.status = reinterpret_cast<uint32_t *>(hdr);
  w.ticket = reinterpret_cast<uint32_t *>(hdr ? hdr + 4 : nullptr);
  w.stall = reinterpret_cast<uint32_t *>(hdr ? hdr + 8 : nullptr);
  w.arrive = reinterpret_cast<uint64_t *>(hdr ? hdr + 16 : nullptr);
  w.counts = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.E));
  w.offsets = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (g.E + 1)));
  w.eidx = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.n));
  w.lrank = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.n));
  w.dst = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.n));
  w.tile_hist = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)g.ntiles * g.E));
  w.tile_flags = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * g.ntiles));
  w.tagged = reinterpret_cast<uint64_t *>(take(sizeof(uint64_t) * (size_t)g.ntiles * (g.E + 1)));
  w.recv_src = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.rows));
  if (g.layout == kStatic) {
    w.keep = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.E));
    w.native_row = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.E));
    w.seg_first = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.E));
    w.seg_count = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.E));
    w.segments = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * 5 * (size_t)(g.E + g.R)));
    w.n_segments = reinterpret_cast<int32_t *>(take(sizeof(int32_t)));
    w.load = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.R));
    w.replica = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)g.R * g.S));
    w.seg_slot = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)(g.E + g.R)));
  }
  w.gemm_tiles = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * 4 * (size_t)gemm_max_tiles(g)));
  w.gemm_ntiles = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * 2));
  if (ws) *ws = w;
  return off;
}

}  // namespace epk

extern "C" {

const char *ep_status_string(ep_status_t st) {
  switch (st) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
    case EP_ERR_BAD_TAG: return "EP_ERR_BAD_TAG";
    case EP_ERR_BAD_DTYPE: return "EP_ERR_BAD_DTYPE";
    case EP_ERR_BAD_SHAPE: return "EP_ERR_BAD_SHAPE";
    case EP_ERR_NOT_PLANNED: return "EP_ERR_NOT_PLANNED";
    case EP_ERR_WORKSPACE_TOO_SMALL: return "EP_ERR_WORKSPACE_TOO_SMALL";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
    case EP_ERR_HIP: return "EP_ERR_HIP";
  }
  return "EP_ERR_UNKNOWN";
}

ep_status_t ep_group_create(const ep_group_config_t *cfg, ep_group_t *out) {
  if (!cfg || !out) return EP_ERR_INVALID_ARG;
  const ep_group_config_t &c = *cfg;
  if (c.num_experts < 1 || c.num_experts > epk::kMaxExperts) return EP_ERR_INVALID_ARG;
  if (c.num_ranks < 1 || c.num_experts % c.num_ranks != 0) return EP_ERR_INVALID_ARG;
  if (c.hidden < 8 || c.hidden % 8 != 0) return EP_ERR_INVALID_ARG;
  if (c.top_k < 1 || c.top_k > epk::kMaxTopK) return EP_ERR_INVALID_ARG;
  if (c.max_tokens < 0) return EP_ERR_INVALID_ARG;
  if ((int64_t)c.max_tokens * c.top_k > INT32_MAX) return EP_ERR_INVALID_ARG;
  if (c.layout != EP_LAYOUT_LL && c.layout != EP_LAYOUT_HT && c.layout != EP_LAYOUT_STATIC)
    return EP_ERR_INVALID_ARG;
  if (c.layout == EP_LAYOUT_LL &&
      (c.capacity < 1 || (int64_t)c.capacity * c.num_experts > INT32_MAX))
    return EP_ERR_INVALID_ARG;
  if (c.layout == EP_LAYOUT_STATIC &&
      (c.slots_per_rank < 0 || (int64_t)c.num_ranks * c.slots_per_rank > INT32_MAX))
    return EP_ERR_INVALID_ARG;
  if (c.dispatch_stores < EP_STORES_AUTO || c.dispatch_stores > EP_STORES_STREAMING)
    return EP_ERR_INVALID_ARG;
  if (c.passes_in_flight < 0 || c.passes_in_flight > 64) return EP_ERR_INVALID_ARG;
  if (c.combine_stores < EP_STORES_AUTO || c.combine_stores > EP_STORES_STREAMING)
    return EP_ERR_INVALID_ARG;
  if (c.fp8_scales != EP_FP8_SCALES_AMAX && c.fp8_scales != EP_FP8_SCALES_POW2 &&
      c.fp8_scales != EP_FP8_SCALES_AMAX_POW2_WEIGHTS)
    return EP_ERR_INVALID_ARG;
  if (c.slot_mode != EP_SLOTS_TRAINING &&
      !(c.slot_mode == EP_SLOTS_INFERENCE && c.layout == EP_LAYOUT_STATIC))
    return EP_ERR_INVALID_ARG;
  const int32_t R = c.layout == EP_LAYOUT_STATIC ? c.num_ranks : 0;
  if (epk::plan_lds_bytes(c.num_experts, R) + 256 > (size_t)epk::kLdsLimit)
    return EP_ERR_UNSUPPORTED;
  ep_group *g = new (std::nothrow) ep_group;
  if (!g) return EP_ERR_INVALID_ARG;
  g->cfg = c;
  g->nbits = 1;
  while ((1 << g->nbits) < c.num_experts) ++g->nbits;
  *out = g;
  return EP_OK;
}

ep_status_t ep_group_destroy(ep_group_t g) {
  if (!g) return EP_ERR_INVALID_ARG;
  delete g;
  return EP_OK;
}

ep_status_t ep_group_recv_rows(ep_group_t g, int32_t num_tokens, int64_t *rows) {
  if (!g || !rows || num_tokens < 0 || num_tokens > g->cfg.max_tokens) return EP_ERR_INVALID_ARG;
  *rows = make_geometry(g, num_tokens).rows;
  return EP_OK;
}

ep_status_t ep_handle_workspace_bytes(ep_group_t g, int32_t num_tokens, size_t *bytes) {
  if (!g || !bytes || num_tokens < 0 || num_tokens > g->cfg.max_tokens) return EP_ERR_INVALID_ARG;
  *bytes = epk::carve_workspace(make_geometry(g, num_tokens), nullptr, nullptr);
  return EP_OK;
}

ep_status_t ep_handle_create(ep_group_t g, int32_t num_tokens, void *workspace,
                             size_t workspace_bytes, ep_handle_t *out) {
  if (!g || !out || !workspace) return EP_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_tokens > g->cfg.max_tokens) return EP_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return EP_ERR_INVALID_ARG;
  epk::Geometry geo = make_geometry(g, num_tokens);
  const size_t need = epk::carve_workspace(geo, nullptr, nullptr);
  if (workspace_bytes < need) return EP_ERR_WORKSPACE_TOO_SMALL;
  geo.cus = device_cus();
  ep_handle *h = new (std::nothrow) ep_handle;
  if (!h) return EP_ERR_INVALID_ARG;
  h->g = g;
  h->geo = geo;
  h->base = static_cast<char *>(workspace);
  h->bytes = workspace_bytes;
  h->planned = false;
  h->in_scratch = false;
  epk::carve_workspace(geo, h->base, &h->ws);
  *out = h;
  return EP_OK;
}

ep_status_t ep_handle_create_static(ep_group_t g, int32_t num_tokens, void *stream,
                                    ep_handle_t *out) {
  if (!g || !out) return EP_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_tokens > g->cfg.max_tokens) return EP_ERR_INVALID_ARG;
  epk::Geometry geo = make_geometry(g, num_tokens);
  const size_t need = epk::carve_workspace(geo, nullptr, nullptr);
  if (need > epk::kScratchBytes) return EP_ERR_WORKSPACE_TOO_SMALL;
  int dev = 0;
  void *base = nullptr;
  if (epk::scratch_base(&dev, &base) != hipSuccess) {
    (void)hipGetLastError();
    return EP_ERR_HIP;
  }
  if (dev >= kMaxScratchHandles) return EP_ERR_UNSUPPORTED;
  // the workspace contract: zero-filled when the handle is made
  if (epk::launch_zero(base, need, as_stream(stream)) != hipSuccess) return EP_ERR_HIP;
  geo.cus = device_cus();
  ep_handle *h = &g_scratch_handles[dev];
  h->g = g;
  h->geo = geo;
  h->base = static_cast<char *>(base);
  h->bytes = epk::kScratchBytes;
  h->planned = false;
  h->in_scratch = true;
  epk::carve_workspace(geo, h->base, &h->ws);
  *out = h;
  return EP_OK;
}

ep_status_t ep_handle_destroy(ep_handle_t h) {
  if (!h) return EP_ERR_INVALID_ARG;
  if (h->in_scratch) return EP_OK;   // static storage: nothing to free
  delete h;
  return EP_OK;
}

ep_status_t ep_handle_query(ep_handle_t h, ep_handle_view_t *v) {
  if (!h || !v) return EP_ERR_INVALID_ARG;
  std::memset(v, 0, sizeof *v);
  const epk::Geometry &g = h->geo;
  v->num_tokens = g.T;
  v->top_k = g.k;
  v->num_experts = g.E;
  v->num_ranks = g.R;
  v->recv_rows = g.rows;
  v->rank_rows = g.layout == EP_LAYOUT_STATIC ? g.C
                 : g.layout == EP_LAYOUT_LL  ? g.cap
                                             : (int32_t)g.n;
  v->max_segments = g.layout == EP_LAYOUT_STATIC ? g.E + g.R : 0;
  v->counts = h->ws.counts;
  v->offsets = h->ws.offsets;
  v->dst = h->ws.dst;
  v->recv_src = h->ws.recv_src;
  v->status = h->ws.status;
  v->keep = h->ws.keep;
  v->native_row = h->ws.native_row;
  v->seg_first = h->ws.seg_first;
  v->seg_count = h->ws.seg_count;
  v->segments = h->ws.segments;
  v->n_segments = h->ws.n_segments;
  v->load = h->ws.load;
  v->replica = h->ws.replica;
  v->seg_slot = h->ws.seg_slot;
  return EP_OK;
}

ep_status_t ep_handle_status(ep_handle_t h, void *stream, uint32_t *flags) {
  if (!h || !flags) return EP_ERR_INVALID_ARG;
  // header: status word, ticket, stall mark, an unused word, arrival count
  uint32_t hdr[6] = {0, 0, 0, 0, 0, 0};
  hipError_t e = hipMemcpyAsync(hdr, h->ws.status, sizeof hdr, hipMemcpyDeviceToHost,
                                as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return EP_ERR_HIP;
  uint32_t v = hdr[0];
  // resident-tiles layout: the last call's epoch mark is its calls so far
  const epk::Geometry &g = h->geo;
  if (g.ntiles > 1 && g.ntiles <= g.cus) {
    uint64_t arrive;
    std::memcpy(&arrive, hdr + 4, sizeof arrive);
    const uint32_t last = (uint32_t)(arrive / (uint64_t)g.ntiles);
    if (last != 0 && hdr[2] == last) v |= EP_FLAG_PLAN_STALL;
  }
  *flags = v;
  return EP_OK;
}

ep_status_t ep_route(ep_handle_t h, const ep_tensor_t *logits, ep_tensor_t *topk_idx,
                     ep_tensor_t *topk_weights, void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(logits, EP_TAG_ROUTER_LOGITS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(logits, g.T, g.E)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(topk_idx, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_idx, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  return hip_status(epk::launch_route(static_cast<const float *>(logits->data), g.T, g.E, g.k,
                                      static_cast<int32_t *>(topk_idx->data),
                                      static_cast<float *>(topk_weights->data),
                                      as_stream(stream)));
}

ep_status_t ep_route_plan(ep_handle_t h, const ep_tensor_t *logits, ep_tensor_t *topk_idx,
                          ep_tensor_t *topk_weights, void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(logits, EP_TAG_ROUTER_LOGITS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(logits, g.T, g.E)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(topk_idx, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_idx, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = hip_status(epk::launch_route_plan(g, h->ws, static_cast<const float *>(logits->data),
                                         static_cast<int32_t *>(topk_idx->data),
                                         static_cast<float *>(topk_weights->data),
                                         as_stream(stream)));
  if (st == EP_OK) h->planned = true;
  return st;
}

ep_status_t ep_plan(ep_handle_t h, const ep_tensor_t *topk_idx, void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(topk_idx, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_idx, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = hip_status(epk::launch_plan(g, h->ws, static_cast<const int32_t *>(topk_idx->data),
                                   as_stream(stream)));
  if (st == EP_OK) h->planned = true;
  return st;
}

// Argument checks of a dispatch (tokens, optional weights, receive rows and
// scales, optional per-row outputs); EP_OK when all hold.
static ep_status_t check_dispatch(const ep_handle *h, const ep_tensor_t *tokens,
                                  const ep_tensor_t *topk_weights, const ep_tensor_t *recv_tokens,
                                  const ep_tensor_t *recv_scales, const ep_tensor_t *recv_topk_idx,
                                  const ep_tensor_t *recv_topk_weights) {
  const epk::Geometry &g = h->geo;
  const int32_t H = h->g->cfg.hidden;
  ep_status_t st = check_tensor(tokens, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_2d(tokens, g.T, H)) return EP_ERR_BAD_SHAPE;
  const bool fp8 = recv_scales != nullptr;
  st = check_tensor(recv_tokens, EP_TAG_TOKENS, fp8 ? EP_DTYPE_FP8_E4M3 : EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_rows(recv_tokens, g.rows, H)) return EP_ERR_BAD_SHAPE;
  if (fp8) {
    if (H % 128 != 0) return EP_ERR_UNSUPPORTED;
    st = check_tensor(recv_scales, EP_TAG_FP8_SCALES, EP_DTYPE_FP32);
    if (st != EP_OK) return st;
    if (!is_rows(recv_scales, g.rows, H / 128)) return EP_ERR_BAD_SHAPE;
  }
  if (topk_weights) {
    st = check_tensor(topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
    if (st != EP_OK) return st;
    if (!is_2d(topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  }
  if (recv_topk_idx) {
    st = check_tensor(recv_topk_idx, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
    if (st != EP_OK) return st;
    if (!(recv_topk_idx->ndim == 1 && recv_topk_idx->sizes[0] == g.rows)) return EP_ERR_BAD_SHAPE;
  }
  if (recv_topk_weights) {
    if (!topk_weights) return EP_ERR_INVALID_ARG;
    st = check_tensor(recv_topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
    if (st != EP_OK) return st;
    if (!(recv_topk_weights->ndim == 1 && recv_topk_weights->sizes[0] == g.rows))
      return EP_ERR_BAD_SHAPE;
  }
  return EP_OK;
}

// Enqueue a checked dispatch; fused: the layout of topk_idx in the same launch.
static ep_status_t run_dispatch(ep_handle *h, const ep_tensor_t *tokens,
                                const ep_tensor_t *topk_weights, ep_tensor_t *recv_tokens,
                                ep_tensor_t *recv_scales, ep_tensor_t *recv_topk_idx,
                                ep_tensor_t *recv_topk_weights, hipStream_t s,
                                const int32_t *topk_idx, bool fused) {
  const epk::Geometry &g = h->geo;
  const int32_t H = h->g->cfg.hidden;
  hipError_t e;
  if (recv_scales)
    e = epk::launch_dispatch_fp8(g, h->ws, static_cast<const uint16_t *>(tokens->data), H,
                                 static_cast<uint8_t *>(recv_tokens->data),
                                 static_cast<float *>(recv_scales->data), s, topk_idx, fused);
  else
    e = epk::launch_dispatch_bf16(g, h->ws, static_cast<const uint16_t *>(tokens->data), H,
                                  static_cast<uint16_t *>(recv_tokens->data), s, topk_idx, fused);
  if (e == hipSuccess && (recv_topk_idx || recv_topk_weights))
    e = epk::launch_recv_meta(
        g, h->ws, topk_weights ? static_cast<const float *>(topk_weights->data) : nullptr,
        recv_topk_idx ? static_cast<int32_t *>(recv_topk_idx->data) : nullptr,
        recv_topk_weights ? static_cast<float *>(recv_topk_weights->data) : nullptr, s);
  return hip_status(e);
}

ep_status_t ep_dispatch(ep_handle_t h, const ep_tensor_t *tokens, const ep_tensor_t *topk_weights,
                        ep_tensor_t *recv_tokens, ep_tensor_t *recv_scales,
                        ep_tensor_t *recv_topk_idx, ep_tensor_t *recv_topk_weights,
                        void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  ep_status_t st = check_dispatch(h, tokens, topk_weights, recv_tokens, recv_scales,
                                  recv_topk_idx, recv_topk_weights);
  if (st != EP_OK) return st;
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return run_dispatch(h, tokens, topk_weights, recv_tokens, recv_scales, recv_topk_idx,
                      recv_topk_weights, as_stream(stream), nullptr, false);
}

ep_status_t ep_plan_dispatch(ep_handle_t h, const ep_tensor_t *topk_idx,
                             const ep_tensor_t *tokens, const ep_tensor_t *topk_weights,
                             ep_tensor_t *recv_tokens, ep_tensor_t *recv_scales,
                             ep_tensor_t *recv_topk_idx, ep_tensor_t *recv_topk_weights,
                             void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(topk_idx, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_idx, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = check_dispatch(h, tokens, topk_weights, recv_tokens, recv_scales, recv_topk_idx,
                      recv_topk_weights);
  if (st != EP_OK) return st;
  hipStream_t s = as_stream(stream);
  const int32_t *idx = static_cast<const int32_t *>(topk_idx->data);
  const bool fused = epk::fused_layout_fits(g);
  if (!fused) {
    st = hip_status(epk::launch_plan(g, h->ws, idx, s));
    if (st != EP_OK) return st;
  }
  h->planned = true;
  return run_dispatch(h, tokens, topk_weights, recv_tokens, recv_scales, recv_topk_idx,
                      recv_topk_weights, s, idx, fused);
}

ep_status_t ep_quantize_fp8(const ep_tensor_t *tokens, ep_tensor_t *codes, ep_tensor_t *scales,
                            int32_t fp8_scales, void *stream) {
  if (fp8_scales != EP_FP8_SCALES_AMAX && fp8_scales != EP_FP8_SCALES_POW2) return EP_ERR_INVALID_ARG;
  ep_status_t st = check_tensor(tokens, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  st = check_tensor(codes, EP_TAG_TOKENS, EP_DTYPE_FP8_E4M3);
  if (st != EP_OK) return st;
  st = check_tensor(scales, EP_TAG_FP8_SCALES, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (tokens->ndim < 2) return EP_ERR_BAD_SHAPE;
  const int64_t K = tokens->sizes[tokens->ndim - 1];
  const int64_t rows = numel(tokens) / (K > 0 ? K : 1);
  if (K <= 0 || K % 128 != 0 || K > INT32_MAX) return EP_ERR_BAD_SHAPE;
  if (!is_rows(codes, rows, K) || !is_rows(scales, rows, K / 128)) return EP_ERR_BAD_SHAPE;
  return hip_status(epk::launch_quantize_fp8(static_cast<const uint16_t *>(tokens->data), rows,
                                             (int32_t)K, static_cast<uint8_t *>(codes->data),
                                             static_cast<float *>(scales->data),
                                             fp8_scales == EP_FP8_SCALES_POW2, as_stream(stream)));
}

ep_status_t ep_combine(ep_handle_t h, const ep_tensor_t *expert_out,
                       const ep_tensor_t *topk_weights, ep_tensor_t *out_tokens, void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  const int32_t H = h->g->cfg.hidden;
  ep_status_t st = check_tensor(expert_out, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_rows(expert_out, g.rows, H)) return EP_ERR_BAD_SHAPE;
  if (topk_weights) {
    st = check_tensor(topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
    if (st != EP_OK) return st;
    if (!is_2d(topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  }
  if (!out_tokens) return EP_ERR_INVALID_ARG;
  const bool out_fp32 = out_tokens->dtype == EP_DTYPE_FP32;
  st = check_tensor(out_tokens, EP_TAG_TOKENS, out_fp32 ? EP_DTYPE_FP32 : EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_2d(out_tokens, g.T, H)) return EP_ERR_BAD_SHAPE;
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return hip_status(epk::launch_combine(
      g, h->ws, static_cast<const uint16_t *>(expert_out->data), H,
      topk_weights ? static_cast<const float *>(topk_weights->data) : nullptr, out_tokens->data,
      out_fp32, as_stream(stream)));
}

ep_status_t ep_combine_bwd(ep_handle_t h, const ep_tensor_t *grad_tokens,
                           const ep_tensor_t *expert_out, const ep_tensor_t *topk_weights,
                           ep_tensor_t *grad_expert_out, ep_tensor_t *grad_topk_weights,
                           void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  const int32_t H = h->g->cfg.hidden;
  ep_status_t st = check_tensor(grad_tokens, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_2d(grad_tokens, g.T, H)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(expert_out, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_rows(expert_out, g.rows, H)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(grad_expert_out, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  if (!is_rows(grad_expert_out, g.rows, H)) return EP_ERR_BAD_SHAPE;
  st = check_tensor(grad_topk_weights, EP_TAG_TOPK_WEIGHTS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (!is_2d(grad_topk_weights, g.T, g.k)) return EP_ERR_BAD_SHAPE;
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return hip_status(epk::launch_combine_bwd(
      g, h->ws, static_cast<const uint16_t *>(grad_tokens->data),
      static_cast<const uint16_t *>(expert_out->data), H,
      static_cast<const float *>(topk_weights->data),
      static_cast<uint16_t *>(grad_expert_out->data),
      static_cast<float *>(grad_topk_weights->data), as_stream(stream)));
}

ep_status_t ep_dup_grad_reduce(ep_handle_t h, const ep_tensor_t *replica_grads,
                               const ep_tensor_t *replica_expert, ep_tensor_t *owner_grads,
                               void *stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  ep_status_t st = check_tensor(replica_grads, EP_TAG_EXPERT_GRADS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  st = check_tensor(owner_grads, EP_TAG_EXPERT_GRADS, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  if (replica_grads->ndim < 2 || owner_grads->ndim < 2) return EP_ERR_BAD_SHAPE;
  const int64_t n = replica_grads->sizes[0];
  const int64_t P = numel(replica_grads) / (n > 0 ? n : 1);
  const int64_t E_owner = owner_grads->sizes[0];
  int64_t Po = 1;
  for (int i = 1; i < owner_grads->ndim; ++i) Po *= owner_grads->sizes[i];
  if (replica_grads->ndim != owner_grads->ndim) return EP_ERR_BAD_SHAPE;
  for (int i = 1; i < owner_grads->ndim; ++i)
    if (replica_grads->sizes[i] != owner_grads->sizes[i]) return EP_ERR_BAD_SHAPE;
  if (n > 65535 || E_owner > INT32_MAX || Po != P) return EP_ERR_BAD_SHAPE;
  const int32_t *rep_e = nullptr;
  if (replica_expert) {
    st = check_tensor(replica_expert, EP_TAG_TOPK_IDX, EP_DTYPE_INT32);
    if (st != EP_OK) return st;
    if (!(replica_expert->ndim == 1 && replica_expert->sizes[0] == n)) return EP_ERR_BAD_SHAPE;
    rep_e = static_cast<const int32_t *>(replica_expert->data);
  } else {
    if (h->geo.layout != EP_LAYOUT_STATIC) return EP_ERR_UNSUPPORTED;
    if (n != (int64_t)h->geo.R * h->geo.S) return EP_ERR_BAD_SHAPE;
    if (!h->planned) return EP_ERR_NOT_PLANNED;
    rep_e = h->ws.replica;
  }
  return hip_status(epk::launch_dup_reduce(
      static_cast<const uint16_t *>(replica_grads->data), rep_e, (int32_t)n, P, (int32_t)E_owner,
      static_cast<float *>(owner_grads->data), h->ws.status, as_stream(stream)));
}

ep_status_t ep_prefetch_replicas(ep_handle_t h, const ep_tensor_t *expert_weights,
                                 ep_tensor_t *slot_weights, void *stream) {
  if (!h || !expert_weights || !slot_weights) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  const int32_t dt = expert_weights->dtype;
  // the weights themselves, or the fp32 scales of FP8 weights
  const int32_t tag = expert_weights->tag == EP_TAG_FP8_SCALES ? EP_TAG_FP8_SCALES
                                                                : EP_TAG_EXPERT_WEIGHTS;
  if (tag == EP_TAG_FP8_SCALES ? dt != EP_DTYPE_FP32
                               : dt != EP_DTYPE_BF16 && dt != EP_DTYPE_FP32 && dt != EP_DTYPE_FP8_E4M3)
    return EP_ERR_BAD_DTYPE;
  ep_status_t st = check_tensor(expert_weights, tag, dt);
  if (st != EP_OK) return st;
  st = check_tensor(slot_weights, tag, dt);
  if (st != EP_OK) return st;
  if (g.layout != EP_LAYOUT_STATIC) return EP_ERR_UNSUPPORTED;
  // expert_weights [E, P...]; slot_weights [R, S, P...] or [R*S, P...]
  const ep_tensor_t *w = expert_weights, *sl = slot_weights;
  if (w->ndim < 2 || w->sizes[0] != g.E) return EP_ERR_BAD_SHAPE;
  int64_t P = 1;
  for (int i = 1; i < w->ndim; ++i) P *= w->sizes[i];
  const int tail = w->ndim - 1;  // dims of one row
  if (sl->ndim == tail + 2) {
    if (sl->sizes[0] != g.R || sl->sizes[1] != g.S) return EP_ERR_BAD_SHAPE;
  } else if (sl->ndim == tail + 1) {
    if (sl->sizes[0] != (int64_t)g.R * g.S) return EP_ERR_BAD_SHAPE;
  } else {
    return EP_ERR_BAD_SHAPE;
  }
  for (int i = 0; i < tail; ++i)
    if (sl->sizes[sl->ndim - tail + i] != w->sizes[1 + i]) return EP_ERR_BAD_SHAPE;
  const int64_t elem = dt == EP_DTYPE_FP32 ? 4 : dt == EP_DTYPE_BF16 ? 2 : 1;
  const int64_t row_bytes = P * elem;
  if (row_bytes % 4 != 0) return EP_ERR_BAD_SHAPE;
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return hip_status(epk::launch_prefetch(g, h->ws, static_cast<const uint8_t *>(w->data),
                                         row_bytes, static_cast<uint8_t *>(sl->data),
                                         as_stream(stream)));
}

// glu: the SwiGLU epilogue (out has N / 2 columns; N % 16 == 0)
static ep_status_t expert_gemm(ep_handle_t h, const ep_tensor_t *recv_tokens,
                               const ep_tensor_t *expert_weights, const ep_tensor_t *slot_weights,
                               ep_tensor_t *out, void *stream, bool glu) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(recv_tokens, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  st = check_tensor(expert_weights, EP_TAG_EXPERT_WEIGHTS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  st = check_tensor(out, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  const ep_tensor_t *w = expert_weights;
  if (w->ndim != 3 || w->sizes[0] != g.E) return EP_ERR_BAD_SHAPE;
  const int64_t N = w->sizes[1], K = w->sizes[2];
  if (K <= 0 || K % 64 != 0 || K > INT32_MAX || N < 1 || N > INT32_MAX) return EP_ERR_BAD_SHAPE;
  if (glu && N % 16 != 0) return EP_ERR_BAD_SHAPE;
  if (!is_rows(recv_tokens, g.rows, K) || !is_rows(out, g.rows, glu ? N / 2 : N))
    return EP_ERR_BAD_SHAPE;
  const uint16_t *wslot = nullptr;
  if (slot_weights) {
    st = check_tensor(slot_weights, EP_TAG_EXPERT_WEIGHTS, EP_DTYPE_BF16);
    if (st != EP_OK) return st;
    if (g.layout != EP_LAYOUT_STATIC) return EP_ERR_UNSUPPORTED;
    const ep_tensor_t *sl = slot_weights;
    const bool four = sl->ndim == 4 && sl->sizes[0] == g.R && sl->sizes[1] == g.S &&
                      sl->sizes[2] == N && sl->sizes[3] == K;
    const bool three = sl->ndim == 3 && sl->sizes[0] == (int64_t)g.R * g.S && sl->sizes[1] == N &&
                       sl->sizes[2] == K;
    if (!four && !three) return EP_ERR_BAD_SHAPE;
    wslot = static_cast<const uint16_t *>(sl->data);
  }
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return hip_status(epk::launch_grouped_gemm(g, h->ws, static_cast<const uint16_t *>(recv_tokens->data),
                                             static_cast<const uint16_t *>(w->data), wslot,
                                             (int32_t)K, (int32_t)N,
                                             static_cast<uint16_t *>(out->data), glu,
                                             as_stream(stream)));
}

ep_status_t ep_expert_gemm(ep_handle_t h, const ep_tensor_t *recv_tokens,
                           const ep_tensor_t *expert_weights, const ep_tensor_t *slot_weights,
                           ep_tensor_t *out, void *stream) {
  return expert_gemm(h, recv_tokens, expert_weights, slot_weights, out, stream, false);
}

ep_status_t ep_expert_gemm_swiglu(ep_handle_t h, const ep_tensor_t *recv_tokens,
                                  const ep_tensor_t *expert_weights,
                                  const ep_tensor_t *slot_weights, ep_tensor_t *out,
                                  void *stream) {
  return expert_gemm(h, recv_tokens, expert_weights, slot_weights, out, stream, true);
}

static ep_status_t expert_gemm_fp8(ep_handle_t h, const ep_tensor_t *recv_tokens,
                                   const ep_tensor_t *recv_scales,
                                   const ep_tensor_t *expert_weights,
                                   const ep_tensor_t *expert_scales,
                                   const ep_tensor_t *slot_weights, const ep_tensor_t *slot_scales,
                                   ep_tensor_t *out, void *stream, bool glu) {
  if (!h) return EP_ERR_INVALID_ARG;
  const epk::Geometry &g = h->geo;
  ep_status_t st = check_tensor(recv_tokens, EP_TAG_TOKENS, EP_DTYPE_FP8_E4M3);
  if (st != EP_OK) return st;
  st = check_tensor(recv_scales, EP_TAG_FP8_SCALES, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  st = check_tensor(expert_weights, EP_TAG_EXPERT_WEIGHTS, EP_DTYPE_FP8_E4M3);
  if (st != EP_OK) return st;
  st = check_tensor(expert_scales, EP_TAG_FP8_SCALES, EP_DTYPE_FP32);
  if (st != EP_OK) return st;
  st = check_tensor(out, EP_TAG_TOKENS, EP_DTYPE_BF16);
  if (st != EP_OK) return st;
  const ep_tensor_t *w = expert_weights, *ws = expert_scales;
  if (w->ndim != 3 || w->sizes[0] != g.E) return EP_ERR_BAD_SHAPE;
  const int64_t N = w->sizes[1], K = w->sizes[2];
  if (K <= 0 || K % 128 != 0 || K > INT32_MAX || N < 1 || N > INT32_MAX) return EP_ERR_BAD_SHAPE;
  if (glu && N % 16 != 0) return EP_ERR_BAD_SHAPE;
  // the kernel addresses a tile's 128 rows of K bytes through 32-bit buffer offsets
  if (K > kFp8GemmMaxK) return EP_ERR_UNSUPPORTED;
  const int64_t NB = K / 128;
  if (!(ws->ndim == 3 && ws->sizes[0] == g.E && ws->sizes[1] == N && ws->sizes[2] == NB))
    return EP_ERR_BAD_SHAPE;
  if (!is_rows(recv_tokens, g.rows, K) || !is_rows(recv_scales, g.rows, NB) ||
      !is_rows(out, g.rows, glu ? N / 2 : N))
    return EP_ERR_BAD_SHAPE;
  if ((slot_weights == nullptr) != (slot_scales == nullptr)) return EP_ERR_INVALID_ARG;
  const uint8_t *wslot = nullptr;
  const float *swslot = nullptr;
  if (slot_weights) {
    st = check_tensor(slot_weights, EP_TAG_EXPERT_WEIGHTS, EP_DTYPE_FP8_E4M3);
    if (st != EP_OK) return st;
    st = check_tensor(slot_scales, EP_TAG_FP8_SCALES, EP_DTYPE_FP32);
    if (st != EP_OK) return st;
    if (g.layout != EP_LAYOUT_STATIC) return EP_ERR_UNSUPPORTED;
    const int64_t RS = (int64_t)g.R * g.S;
    auto slots_of = [&](const ep_tensor_t *t, int64_t last) {
      return (t->ndim == 4 && t->sizes[0] == g.R && t->sizes[1] == g.S && t->sizes[2] == N &&
              t->sizes[3] == last) ||
             (t->ndim == 3 && t->sizes[0] == RS && t->sizes[1] == N && t->sizes[2] == last);
    };
    if (!slots_of(slot_weights, K) || !slots_of(slot_scales, NB)) return EP_ERR_BAD_SHAPE;
    wslot = static_cast<const uint8_t *>(slot_weights->data);
    swslot = static_cast<const float *>(slot_scales->data);
  }
  if (!h->planned) return EP_ERR_NOT_PLANNED;
  return hip_status(epk::launch_grouped_gemm_fp8(
      g, h->ws, static_cast<const uint8_t *>(recv_tokens->data),
      static_cast<const float *>(recv_scales->data), static_cast<const uint8_t *>(w->data),
      static_cast<const float *>(ws->data), wslot, swslot, (int32_t)K, (int32_t)N,
      static_cast<uint16_t *>(out->data), glu, as_stream(stream)));
}

ep_status_t ep_expert_gemm_fp8(ep_handle_t h, const ep_tensor_t *recv_tokens,
                               const ep_tensor_t *recv_scales, const ep_tensor_t *expert_weights,
                               const ep_tensor_t *expert_scales, const ep_tensor_t *slot_weights,
                               const ep_tensor_t *slot_scales, ep_tensor_t *out, void *stream) {
  return expert_gemm_fp8(h, recv_tokens, recv_scales, expert_weights, expert_scales, slot_weights,
                         slot_scales, out, stream, false);
}

ep_status_t ep_expert_gemm_fp8_swiglu(ep_handle_t h, const ep_tensor_t *recv_tokens,
                                      const ep_tensor_t *recv_scales,
                                      const ep_tensor_t *expert_weights,
                                      const ep_tensor_t *expert_scales,
                                      const ep_tensor_t *slot_weights,
                                      const ep_tensor_t *slot_scales, ep_tensor_t *out,
                                      void *stream) {
  return expert_gemm_fp8(h, recv_tokens, recv_scales, expert_weights, expert_scales, slot_weights,
                         slot_scales, out, stream, true);
}

ep_status_t ep_run_calls(const ep_call_t *calls, int32_t n, int32_t *failed) {
  if (failed != nullptr) *failed = 0;
  if (n < 0 || (n > 0 && calls == nullptr)) return EP_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const ep_call_t &c = calls[i];
    const auto h = static_cast<ep_handle_t>(c.p[0]);
    const auto t = [&c](int k) { return static_cast<ep_tensor_t *>(c.p[k]); };
    ep_status_t st;
    switch (c.op) {
      case EP_OP_ROUTE: st = ep_route(h, t(1), t(2), t(3), c.p[4]); break;
      case EP_OP_ROUTE_PLAN: st = ep_route_plan(h, t(1), t(2), t(3), c.p[4]); break;
      case EP_OP_PLAN: st = ep_plan(h, t(1), c.p[2]); break;
      case EP_OP_DISPATCH: st = ep_dispatch(h, t(1), t(2), t(3), t(4), t(5), t(6), c.p[7]); break;
      case EP_OP_PLAN_DISPATCH:
        st = ep_plan_dispatch(h, t(1), t(2), t(3), t(4), t(5), t(6), t(7), c.p[8]);
        break;
      case EP_OP_QUANTIZE_FP8: st = ep_quantize_fp8(t(0), t(1), t(2), c.i0, c.p[3]); break;
      case EP_OP_COMBINE: st = ep_combine(h, t(1), t(2), t(3), c.p[4]); break;
      case EP_OP_COMBINE_BWD: st = ep_combine_bwd(h, t(1), t(2), t(3), t(4), t(5), c.p[6]); break;
      case EP_OP_DUP_GRAD_REDUCE: st = ep_dup_grad_reduce(h, t(1), t(2), t(3), c.p[4]); break;
      case EP_OP_PREFETCH_REPLICAS: st = ep_prefetch_replicas(h, t(1), t(2), c.p[3]); break;
      case EP_OP_EXPERT_GEMM: st = ep_expert_gemm(h, t(1), t(2), t(3), t(4), c.p[5]); break;
      case EP_OP_EXPERT_GEMM_SWIGLU:
        st = ep_expert_gemm_swiglu(h, t(1), t(2), t(3), t(4), c.p[5]);
        break;
      case EP_OP_EXPERT_GEMM_FP8:
        st = ep_expert_gemm_fp8(h, t(1), t(2), t(3), t(4), t(5), t(6), t(7), c.p[8]);
        break;
      case EP_OP_EXPERT_GEMM_FP8_SWIGLU:
        st = ep_expert_gemm_fp8_swiglu(h, t(1), t(2), t(3), t(4), t(5), t(6), t(7), c.p[8]);
        break;
      default: st = EP_ERR_INVALID_ARG; break;
    }
    if (st != EP_OK) {
      if (failed != nullptr) *failed = i;
      return st;
    }
  }
  if (failed != nullptr) *failed = n;
  return EP_OK;
}

}  // extern "C"
