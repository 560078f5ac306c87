"""Host-side tests of the C ABI: the library loads without a GPU, exports
every entry point include/ep.h declares, and rejects bad arguments on the
host before anything would be enqueued.  No kernel is launched here: every
call either fails validation or is pure bookkeeping."""

from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import combine_ep_plan_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced by these tests


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ep.library_path()):
        from combine_ep_plan_amd import build
        build.build()
    return ep.load_library()


def declared_functions() -> list[str]:
    names = []
    with open(os.path.join(ROOT, "include", "ep.h")) as fh:
        text = fh.read()
    for m in re.finditer(r"^(?:const char \*|ep_status_t )(ep_\w+)\(", text, re.M):
        names.append(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = set(declared_functions())
    for need in ("ep_plan", "ep_dispatch", "ep_combine", "ep_combine_bwd", "ep_dup_grad_reduce",
                 "ep_group_create", "ep_handle_create", "ep_handle_status"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing


def test_status_strings(lib):
    for code, name in enumerate(ep._STATUS):
        assert ep.ep_status_string(code) == name
    assert ep.ep_status_string(99) == "EP_ERR_UNKNOWN"


def cfg(**kw):
    base = dict(num_experts=8, num_ranks=4, hidden=256, top_k=2, max_tokens=64,
                layout=ep.LAYOUT_HT, capacity=0, slots_per_rank=0, slot_mode=0, dispatch_stores=0,
                passes_in_flight=0, fp8_scales=0, combine_stores=0)
    base.update(kw)
    return ep.ep_group_config_t(*[base[f] for f, _ in ep.ep_group_config_t._fields_])


def create(lib, **kw):
    g = ctypes.c_void_p()
    rc = lib.ep_group_create(ctypes.byref(cfg(**kw)), ctypes.byref(g))
    return rc, g


@pytest.mark.parametrize("bad", [
    dict(num_experts=0), dict(num_experts=1025), dict(num_ranks=3), dict(num_ranks=0),
    dict(hidden=12), dict(hidden=0), dict(top_k=0), dict(top_k=17), dict(max_tokens=-1),
    dict(layout=7), dict(layout=ep.LAYOUT_LL, capacity=0), dict(layout=ep.LAYOUT_STATIC, slots_per_rank=-1),
    dict(layout=ep.LAYOUT_STATIC, slot_mode=2), dict(layout=ep.LAYOUT_STATIC, slot_mode=-1),
    dict(dispatch_stores=3), dict(dispatch_stores=-1), dict(passes_in_flight=-1),
    dict(passes_in_flight=65), dict(fp8_scales=3), dict(fp8_scales=-1),
    dict(combine_stores=3), dict(combine_stores=-1),
    dict(slot_mode=ep.SLOTS_INFERENCE),               # the inference slot mode is STATIC only
    dict(layout=ep.LAYOUT_STATIC, num_experts=1024, num_ranks=1024, slots_per_rank=1 << 22),
])
def test_group_config_validation(lib, bad):
    rc, _ = create(lib, **bad)
    assert rc == 1  # EP_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["dispatch_stores", "combine_stores"])
@pytest.mark.parametrize("stores", [ep.STORES_AUTO, ep.STORES_CACHED, ep.STORES_STREAMING])
def test_group_accepts_each_store_kind(lib, field, stores):
    rc, g = create(lib, **{field: stores})
    assert rc == 0
    lib.ep_group_destroy(g)


@pytest.mark.parametrize("f8", [ep.FP8_SCALES_AMAX, ep.FP8_SCALES_POW2, ep.FP8_SCALES_AMAX_POW2_WEIGHTS])
def test_group_accepts_each_fp8_scale_format(lib, f8):
    rc, g = create(lib, fp8_scales=f8)
    assert rc == 0
    lib.ep_group_destroy(g)


def test_group_null_arguments(lib):
    g = ctypes.c_void_p()
    assert lib.ep_group_create(None, ctypes.byref(g)) == 1
    assert lib.ep_group_create(ctypes.byref(cfg()), None) == 1
    assert lib.ep_group_destroy(None) == 1


def test_group_planner_table_limit(lib):
    rc, g = create(lib, num_experts=1024, num_ranks=1024, layout=ep.LAYOUT_STATIC, slots_per_rank=1)
    assert rc == 0
    lib.ep_group_destroy(g)


@pytest.mark.parametrize("layout,kw,T,rows", [
    (ep.LAYOUT_HT, {}, 64, 128),
    (ep.LAYOUT_LL, dict(capacity=64), 64, 8 * 64),
    (ep.LAYOUT_STATIC, dict(slots_per_rank=2), 63, 4 * 32),   # ceil(126/4) = 32
    (ep.LAYOUT_HT, {}, 0, 0),
])
def test_recv_rows_and_workspace(lib, layout, kw, T, rows):
    rc, g = create(lib, layout=layout, **kw)
    assert rc == 0
    r = ctypes.c_int64()
    assert lib.ep_group_recv_rows(g, T, ctypes.byref(r)) == 0 and r.value == rows
    b = ctypes.c_size_t()
    assert lib.ep_handle_workspace_bytes(g, T, ctypes.byref(b)) == 0
    assert b.value >= 4 * rows and b.value % 256 == 0
    assert lib.ep_handle_workspace_bytes(g, 65, ctypes.byref(b)) == 1   # > max_tokens
    lib.ep_group_destroy(g)


def make_handle(lib, T=64, **kw):
    rc, g = create(lib, **kw)
    assert rc == 0
    b = ctypes.c_size_t()
    lib.ep_handle_workspace_bytes(g, T, ctypes.byref(b))
    h = ctypes.c_void_p()
    assert lib.ep_handle_create(g, T, ctypes.c_void_p(FAKE), b.value, ctypes.byref(h)) == 0
    return g, h, b.value


def test_handle_create_validation(lib):
    rc, g = create(lib)
    b = ctypes.c_size_t()
    lib.ep_handle_workspace_bytes(g, 64, ctypes.byref(b))
    h = ctypes.c_void_p()
    assert lib.ep_handle_create(g, 64, None, b.value, ctypes.byref(h)) == 1
    assert lib.ep_handle_create(g, 64, ctypes.c_void_p(FAKE + 8), b.value, ctypes.byref(h)) == 1
    assert lib.ep_handle_create(g, 64, ctypes.c_void_p(FAKE), b.value - 1, ctypes.byref(h)) == 6
    assert lib.ep_handle_create(g, 65, ctypes.c_void_p(FAKE), 1 << 30, ctypes.byref(h)) == 1
    assert lib.ep_handle_create(g, -1, ctypes.c_void_p(FAKE), 1 << 30, ctypes.byref(h)) == 1
    lib.ep_group_destroy(g)


def test_handle_create_static_validation(lib):
    # argument checks of the scratch-backed handle run before any device call;
    # a batch whose workspace exceeds the 16 MiB scratch is refused
    rc, g = create(lib)
    h = ctypes.c_void_p()
    f = lib.ep_handle_create_static
    assert f(None, 64, None, ctypes.byref(h)) == 1
    assert f(g, 64, None, None) == 1
    assert f(g, 65, None, ctypes.byref(h)) == 1       # > max_tokens
    assert f(g, -1, None, ctypes.byref(h)) == 1
    lib.ep_group_destroy(g)
    rc, g = create(lib, num_experts=1024, num_ranks=1, top_k=16, max_tokens=65536)
    assert rc == 0
    b = ctypes.c_size_t()
    lib.ep_handle_workspace_bytes(g, 65536, ctypes.byref(b))
    assert b.value > (16 << 20)
    assert f(g, 65536, None, ctypes.byref(h)) == 6    # EP_ERR_WORKSPACE_TOO_SMALL
    lib.ep_group_destroy(g)


def test_handle_view_points_into_workspace(lib):
    g, h, nbytes = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    v = ep.ep_handle_view_t()
    assert lib.ep_handle_query(h, ctypes.byref(v)) == 0
    assert v.num_tokens == 64 and v.top_k == 2 and v.num_experts == 8 and v.num_ranks == 4
    assert v.recv_rows == 128 and v.rank_rows == 32 and v.max_segments == 12
    for name in ("counts", "offsets", "dst", "recv_src", "status", "keep", "native_row",
                 "seg_first", "seg_count", "segments", "n_segments", "load", "replica",
                 "seg_slot"):
        p = getattr(v, name)
        assert p is not None and FAKE <= p < FAKE + nbytes and p % 256 == 0
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def T(dtype, tag, *sizes, data=FAKE):
    t = ep.ep_tensor_t()
    t.data = data
    t.dtype = dtype
    t.tag = tag
    t.ndim = len(sizes)
    t.reserved = 0
    for i, s in enumerate(sizes):
        t.sizes[i] = s
    return ctypes.pointer(t)


BF16, F32, FP8, I32 = 0, 1, 2, 3


def test_plan_argument_validation(lib):
    g, h, _ = make_handle(lib)
    assert lib.ep_plan(h, None, None) == 1
    assert lib.ep_plan(h, T(I32, ep.TAG_TOKENS, 64, 2), None) == 2
    assert lib.ep_plan(h, T(F32, ep.TAG_TOPK_IDX, 64, 2), None) == 3
    assert lib.ep_plan(h, T(I32, ep.TAG_TOPK_IDX, 64, 3), None) == 4
    assert lib.ep_plan(h, T(I32, ep.TAG_TOPK_IDX, 128), None) == 4
    assert lib.ep_plan(h, T(I32, ep.TAG_TOPK_IDX, 64, 2, data=None), None) == 1
    assert lib.ep_plan(None, T(I32, ep.TAG_TOPK_IDX, 64, 2), None) == 1
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_dispatch_argument_validation(lib):
    g, h, _ = make_handle(lib)
    x = T(BF16, ep.TAG_TOKENS, 64, 256)
    w = T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2)
    recv = T(BF16, ep.TAG_TOKENS, 128, 256)
    D = lib.ep_dispatch
    assert D(h, T(BF16, ep.TAG_TOKENS, 64, 255), w, recv, None, None, None, None) == 4
    assert D(h, x, w, T(BF16, ep.TAG_TOKENS, 127, 256), None, None, None, None) == 4
    assert D(h, x, w, T(F32, ep.TAG_TOKENS, 128, 256), None, None, None, None) == 3
    assert D(h, x, w, T(BF16, ep.TAG_FP8_SCALES, 128, 256), None, None, None, None) == 2
    assert D(h, x, T(F32, ep.TAG_TOPK_WEIGHTS, 64, 3), recv, None, None, None, None) == 4
    # FP8 output needs FP8 rows and H % 128 == 0 (H = 256 here: fine)
    assert D(h, x, w, recv, T(F32, ep.TAG_FP8_SCALES, 128, 2), None, None, None) == 3
    assert D(h, x, w, T(FP8, ep.TAG_TOKENS, 128, 256), T(F32, ep.TAG_FP8_SCALES, 128, 3),
             None, None, None) == 4
    assert D(h, x, None, recv, None, None, T(F32, ep.TAG_TOPK_WEIGHTS, 128), None) == 1
    assert D(h, x, w, recv, None, T(I32, ep.TAG_TOPK_IDX, 127), None, None) == 4
    # valid arguments, but the handle has never been planned
    assert D(h, x, w, recv, None, T(I32, ep.TAG_TOPK_IDX, 128), T(F32, ep.TAG_TOPK_WEIGHTS, 128), None) == 5
    assert D(h, x, w, T(BF16, ep.TAG_TOKENS, 4, 32, 256), None, None, None, None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_fp8_needs_hidden_multiple_of_128(lib):
    g, h, _ = make_handle(lib, hidden=136)
    x = T(BF16, ep.TAG_TOKENS, 64, 136)
    assert lib.ep_dispatch(h, x, None, T(FP8, ep.TAG_TOKENS, 128, 136),
                           T(F32, ep.TAG_FP8_SCALES, 128, 1), None, None, None) == 7
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_combine_and_bwd_argument_validation(lib):
    g, h, _ = make_handle(lib)
    rows = T(BF16, ep.TAG_TOKENS, 128, 256)
    w = T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2)
    y = T(BF16, ep.TAG_TOKENS, 64, 256)
    C = lib.ep_combine
    assert C(h, rows, w, None, None) == 1
    assert C(h, rows, w, T(BF16, ep.TAG_TOKENS, 63, 256), None) == 4
    assert C(h, rows, w, T(I32, ep.TAG_TOKENS, 64, 256), None) == 3
    assert C(h, T(BF16, ep.TAG_TOPK_IDX, 128, 256), w, y, None) == 2
    assert C(h, rows, w, y, None) == 5
    assert C(h, rows, None, T(F32, ep.TAG_TOKENS, 64, 256), None) == 5
    B = lib.ep_combine_bwd
    gw = T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2)
    assert B(h, y, rows, None, rows, gw, None) == 1
    assert B(h, y, rows, w, rows, T(F32, ep.TAG_TOKENS, 64, 2), None) == 2
    assert B(h, y, rows, w, T(BF16, ep.TAG_TOKENS, 128, 128), gw, None) == 4
    assert B(h, y, rows, w, rows, gw, None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_dup_reduce_argument_validation(lib):
    g, h, _ = make_handle(lib)
    rep = T(BF16, ep.TAG_EXPERT_GRADS, 2, 64, 16)
    own = T(F32, ep.TAG_EXPERT_GRADS, 8, 64, 16)
    ids = T(I32, ep.TAG_TOPK_IDX, 2)
    R = lib.ep_dup_grad_reduce
    assert R(h, T(BF16, ep.TAG_TOKENS, 2, 64, 16), ids, own, None) == 2
    assert R(h, rep, ids, T(F32, ep.TAG_EXPERT_GRADS, 8, 64, 8), None) == 4
    assert R(h, rep, T(I32, ep.TAG_TOPK_IDX, 3), own, None) == 4
    assert R(h, rep, None, own, None) == 7      # replica table only exists for STATIC
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)
    g, h, _ = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    assert R(h, T(BF16, ep.TAG_EXPERT_GRADS, 7, 64, 16), None, own, None) == 4   # n != R*S
    assert R(h, T(BF16, ep.TAG_EXPERT_GRADS, 8, 64, 16), None, own, None) == 5   # not planned
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


@pytest.mark.parametrize("entry", ["ep_route", "ep_route_plan"])
def test_route_argument_validation(lib, entry):
    g, h, _ = make_handle(lib)
    lg = T(F32, ep.TAG_ROUTER_LOGITS, 64, 8)
    idx = T(I32, ep.TAG_TOPK_IDX, 64, 2)
    w = T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2)
    Rt = getattr(lib, entry)
    assert Rt(h, T(F32, ep.TAG_TOKENS, 64, 8), idx, w, None) == 2
    assert Rt(h, T(BF16, ep.TAG_ROUTER_LOGITS, 64, 8), idx, w, None) == 3
    assert Rt(h, T(F32, ep.TAG_ROUTER_LOGITS, 64, 9), idx, w, None) == 4
    assert Rt(h, lg, T(I32, ep.TAG_TOPK_IDX, 64, 3), w, None) == 4
    assert Rt(h, lg, idx, T(F32, ep.TAG_TOPK_IDX, 64, 2), None) == 2
    assert Rt(h, lg, idx, None, None) == 1
    assert Rt(None, lg, idx, w, None) == 1
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_inference_slot_mode_accepted(lib):
    rc, g = create(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=1, slot_mode=ep.SLOTS_INFERENCE)
    assert rc == 0
    lib.ep_group_destroy(g)


def test_prefetch_argument_validation(lib):
    P = lib.ep_prefetch_replicas
    W = ep.TAG_EXPERT_WEIGHTS
    g, h, _ = make_handle(lib)                       # HT: no replica slots
    assert P(h, T(BF16, W, 8, 64), T(BF16, W, 4, 2, 64), None) == 7
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)
    g, h, _ = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    w = T(BF16, W, 8, 64)
    sl = T(BF16, W, 4, 2, 64)
    assert P(h, None, sl, None) == 1
    assert P(None, w, sl, None) == 1
    assert P(h, T(BF16, ep.TAG_EXPERT_GRADS, 8, 64), sl, None) == 2
    assert P(h, w, T(F32, W, 4, 2, 64), None) == 3       # dtypes differ
    assert P(h, T(I32, W, 8, 64), T(I32, W, 4, 2, 64), None) == 3
    assert P(h, T(BF16, W, 7, 64), sl, None) == 4        # not E experts
    assert P(h, w, T(BF16, W, 4, 3, 64), None) == 4      # not [R, S, ...]
    assert P(h, w, T(BF16, W, 4, 2, 32), None) == 4      # rows differ
    assert P(h, w, T(BF16, W, 9, 64), None) == 4         # 2-D form needs R*S rows
    assert P(h, T(BF16, W, 8, 1), T(BF16, W, 4, 2, 1), None) == 4   # 2-byte rows
    assert P(h, T(BF16, W, 8, 4), T(BF16, W, 4, 2, 4), None) == 5   # 8-byte rows: the 4-byte path
    assert P(h, w, sl, None) == 5                        # not planned
    assert P(h, w, T(BF16, W, 8, 64), None) == 5         # 2-D form, not planned
    assert P(h, T(FP8, W, 8, 2, 16), T(FP8, W, 4, 2, 2, 16), None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_expert_gemm_argument_validation(lib):
    G = lib.ep_expert_gemm
    W, TK = ep.TAG_EXPERT_WEIGHTS, ep.TAG_TOKENS
    g, h, _ = make_handle(lib)                       # HT, T=64, k=2: 128 rows, E=8
    x = T(BF16, TK, 128, 64)
    w = T(BF16, W, 8, 32, 64)
    y = T(BF16, TK, 128, 32)
    assert G(None, x, w, None, y, None) == 1
    assert G(h, T(BF16, W, 128, 64), w, None, y, None) == 2      # x must be TOKENS
    assert G(h, x, T(F32, W, 8, 32, 64), None, y, None) == 3
    assert G(h, x, T(BF16, W, 7, 32, 64), None, y, None) == 4    # not E matrices
    assert G(h, T(BF16, TK, 128, 48), T(BF16, W, 8, 32, 48), None, T(BF16, TK, 128, 32), None) == 4  # K % 64
    assert G(h, x, w, None, T(BF16, TK, 128, 33), None) == 4      # out columns != N
    assert G(h, T(BF16, TK, 127, 64), w, None, y, None) == 4      # not recv_rows
    assert G(h, x, w, T(BF16, W, 4, 1, 32, 64), y, None) == 7     # slots only for STATIC
    assert G(h, x, w, None, y, None) == 5                         # not planned
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)
    g, h, _ = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    assert G(h, x, w, T(BF16, W, 4, 3, 32, 64), y, None) == 4     # not [R, S, N, K]
    assert G(h, x, w, T(BF16, W, 8, 32, 64), y, None) == 5        # [R*S, N, K] accepted; not planned
    assert G(h, x, w, T(BF16, W, 4, 2, 32, 64), y, None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_expert_gemm_swiglu_argument_validation(lib):
    # out has N/2 columns and N must be a multiple of 16; the rest as for the plain GEMMs
    W, TK, SC = ep.TAG_EXPERT_WEIGHTS, ep.TAG_TOKENS, ep.TAG_FP8_SCALES
    g, h, _ = make_handle(lib)                       # HT, T=64, k=2: 128 rows, E=8
    G = lib.ep_expert_gemm_swiglu
    x, w = T(BF16, TK, 128, 64), T(BF16, W, 8, 32, 64)
    assert G(None, x, w, None, T(BF16, TK, 128, 16), None) == 1
    assert G(h, x, w, None, T(BF16, TK, 128, 32), None) == 4                        # N columns, not N/2
    assert G(h, x, T(BF16, W, 8, 40, 64), None, T(BF16, TK, 128, 20), None) == 4    # N % 16
    assert G(h, x, w, None, T(BF16, TK, 128, 16), None) == 5                        # accepted; not planned
    G8 = lib.ep_expert_gemm_fp8_swiglu
    x8, sx = T(FP8, TK, 128, 128), T(F32, SC, 128, 1)
    w8, sw = T(FP8, W, 8, 32, 128), T(F32, SC, 8, 32, 1)
    assert G8(None, x8, sx, w8, sw, None, None, T(BF16, TK, 128, 16), None) == 1
    assert G8(h, x8, sx, w8, sw, None, None, T(BF16, TK, 128, 32), None) == 4
    assert G8(h, x8, sx, T(FP8, W, 8, 40, 128), T(F32, SC, 8, 40, 1), None, None,
              T(BF16, TK, 128, 20), None) == 4
    assert G8(h, x8, sx, w8, sw, None, None, T(BF16, TK, 128, 16), None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_prefetch_accepts_fp8_weight_scales(lib):
    P = lib.ep_prefetch_replicas
    W, SC = ep.TAG_EXPERT_WEIGHTS, ep.TAG_FP8_SCALES
    g, h, _ = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    assert P(h, T(F32, SC, 8, 4, 2), T(F32, SC, 4, 2, 4, 2), None) == 5   # scales: accepted, not planned
    assert P(h, T(F32, SC, 8, 4, 2), T(F32, W, 4, 2, 4, 2), None) == 2    # tags differ
    assert P(h, T(BF16, SC, 8, 4, 8), T(BF16, SC, 4, 2, 4, 8), None) == 3  # scales are fp32
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_expert_gemm_fp8_argument_validation(lib):
    G = lib.ep_expert_gemm_fp8
    W, TK, SC = ep.TAG_EXPERT_WEIGHTS, ep.TAG_TOKENS, ep.TAG_FP8_SCALES
    g, h, _ = make_handle(lib)                       # HT, T=64, k=2: 128 rows, E=8
    x, sx = T(FP8, TK, 128, 256), T(F32, SC, 128, 2)
    w, sw = T(FP8, W, 8, 32, 256), T(F32, SC, 8, 32, 2)
    y = T(BF16, TK, 128, 32)
    assert G(None, x, sx, w, sw, None, None, y, None) == 1
    assert G(h, T(BF16, TK, 128, 256), sx, w, sw, None, None, y, None) == 3   # codes must be FP8
    assert G(h, x, T(F32, TK, 128, 2), w, sw, None, None, y, None) == 2       # scales tag
    assert G(h, x, sx, T(BF16, W, 8, 32, 256), sw, None, None, y, None) == 3
    assert G(h, x, sx, w, sw, None, None, T(F32, TK, 128, 32), None) == 3     # out is bf16
    assert G(h, T(FP8, TK, 128, 192), T(F32, SC, 128, 1), T(FP8, W, 8, 32, 192),
             T(F32, SC, 8, 32, 1), None, None, y, None) == 4                  # K % 128
    assert G(h, x, T(F32, SC, 128, 1), w, sw, None, None, y, None) == 4       # row scales K/128
    assert G(h, x, sx, w, T(F32, SC, 8, 32, 1), None, None, y, None) == 4     # weight scales K/128
    KB = (1 << 24) + 128                                                      # beyond 32-bit tile offsets
    assert G(h, T(FP8, TK, 128, KB), T(F32, SC, 128, KB // 128), T(FP8, W, 8, 32, KB),
             T(F32, SC, 8, 32, KB // 128), None, None, y, None) == 7
    KM = 1 << 24                                                              # the largest K taken:
    assert G(h, T(FP8, TK, 128, KM), T(F32, SC, 128, KM // 128), T(FP8, W, 8, 32, KM),
             T(F32, SC, 8, 32, KM // 128), None, None, y, None) == 5          # passes the size check
    assert G(h, x, sx, w, T(F32, SC, 7, 32, 2), None, None, y, None) == 4
    assert G(h, x, sx, T(FP8, W, 7, 32, 256), sw, None, None, y, None) == 4   # not E matrices
    assert G(h, T(FP8, TK, 127, 256), sx, w, sw, None, None, y, None) == 4    # not recv_rows
    assert G(h, x, sx, w, sw, None, None, T(BF16, TK, 128, 33), None) == 4    # out columns != N
    assert G(h, x, sx, w, sw, T(FP8, W, 4, 1, 32, 256), None, y, None) == 1   # slot scales missing
    assert G(h, x, sx, w, sw, T(FP8, W, 4, 1, 32, 256), T(F32, SC, 4, 1, 32, 2), y, None) == 7
    assert G(h, x, sx, w, sw, None, None, y, None) == 5                       # not planned
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)
    g, h, _ = make_handle(lib, layout=ep.LAYOUT_STATIC, slots_per_rank=2)
    sl, ssl = T(FP8, W, 4, 2, 32, 256), T(F32, SC, 4, 2, 32, 2)
    assert G(h, x, sx, w, sw, T(FP8, W, 4, 3, 32, 256), ssl, y, None) == 4    # not [R, S, N, K]
    assert G(h, x, sx, w, sw, sl, T(F32, SC, 4, 2, 32, 1), y, None) == 4      # slot scales K/128
    assert G(h, x, sx, w, sw, sl, T(BF16, SC, 4, 2, 32, 2), y, None) == 3
    assert G(h, x, sx, w, sw, sl, ssl, y, None) == 5                          # not planned
    assert G(h, x, sx, w, sw, T(FP8, W, 8, 32, 256), T(F32, SC, 8, 32, 2), y, None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_misaligned_tensor_data_is_rejected(lib):
    g, h, _ = make_handle(lib)                       # HT, T=64, k=2, H=256
    D = lib.ep_dispatch
    recv = T(BF16, ep.TAG_TOKENS, 128, 256)
    # token rows need 16-byte alignment
    assert D(h, T(BF16, ep.TAG_TOKENS, 64, 256, data=FAKE + 8), None, recv, None, None, None, None) == 1
    assert D(h, T(BF16, ep.TAG_TOKENS, 64, 256, data=FAKE + 16), None, recv, None, None, None, None) == 5
    # router weights only 4-byte alignment
    x = T(BF16, ep.TAG_TOKENS, 64, 256)
    assert D(h, x, T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2, data=FAKE + 2), recv, None, None, None, None) == 1
    assert D(h, x, T(F32, ep.TAG_TOPK_WEIGHTS, 64, 2, data=FAKE + 4), recv, None, None, None, None) == 5
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)


def test_binding_refuses_host_tensors():
    # the binding hands raw pointers to the kernels: a host tensor must never
    # reach them
    with pytest.raises(ValueError, match="on the GPU"):
        ep._tensor(torch.zeros(4, 8), ep.TAG_TOKENS)


def test_quantize_fp8_argument_validation(lib):
    def Q(x, q, s, stream, fmt=0):
        return lib.ep_quantize_fp8(x, q, s, fmt, stream)
    TK, SC = ep.TAG_TOKENS, ep.TAG_FP8_SCALES
    x, q, s = T(BF16, TK, 64, 256), T(FP8, TK, 64, 256), T(F32, SC, 64, 2)
    assert Q(None, q, s, None) == 1
    assert Q(x, q, None, None) == 1
    assert Q(T(F32, TK, 64, 256), q, s, None) == 3            # rows are bf16
    assert Q(x, T(BF16, TK, 64, 256), s, None) == 3           # codes are e4m3
    assert Q(x, q, T(F32, TK, 64, 2), None) == 2              # scales tag
    assert Q(T(BF16, TK, 64, 192), T(FP8, TK, 64, 192), T(F32, SC, 64, 1), None) == 4   # K % 128
    assert Q(T(BF16, TK, 256), T(FP8, TK, 256), T(F32, SC, 2), None) == 4              # 1D rows
    assert Q(x, T(FP8, TK, 63, 256), s, None) == 4            # codes not [rows, K]
    assert Q(x, q, T(F32, SC, 64, 3), None) == 4              # scales not [rows, K/128]
    assert Q(x, q, T(F32, SC, 64, 2, data=FAKE + 2), None) == 1
    assert Q(T(BF16, TK, 64, 256, data=FAKE + 8), q, s, None) == 1
    assert Q(x, q, s, None, fmt=2) == 1                      # no such scale format
    assert Q(x, q, s, None, fmt=-1) == 1
    # zero rows, also under a leading shape, pass validation and enqueue nothing
    assert Q(T(BF16, TK, 0, 256, data=None), T(FP8, TK, 0, 256, data=None),
             T(F32, SC, 0, 2, data=None), None) == 0
    assert Q(T(BF16, TK, 4, 0, 256, data=None), T(FP8, TK, 0, 256, data=None),
             T(F32, SC, 0, 2, data=None), None) == 0
    assert Q(T(BF16, TK, 0, 256, data=None), T(FP8, TK, 0, 256, data=None),
             T(F32, SC, 0, 2, data=None), None, fmt=1) == 0


def test_prepare_records_without_enqueueing():
    # nothing recorded: an empty call list; prepare does not nest; the
    # recording state is cleared even when the recorded function raises
    p = ep.prepare(lambda: None)
    assert p.names == () and p() is None
    with pytest.raises(RuntimeError, match="nest"):
        ep.prepare(lambda: ep.prepare(lambda: None))
    with pytest.raises(ValueError, match="on the GPU"):
        ep.prepare(lambda: ep.ep_plan(1, torch.zeros(4, 2, dtype=torch.int32)))
    assert getattr(ep._RECORDING, "calls", None) is None


def _calls(*specs):
    """ep_call_t array from (op, i0, [pointer args]) triples."""
    arr = (ep.ep_call_t * max(len(specs), 1))()
    for k, (op, i0, ptrs) in enumerate(specs):
        arr[k].op, arr[k].i0 = op, i0
        for m, a in enumerate(ptrs):
            arr[k].p[m] = None if a is None else ctypes.cast(a, ctypes.c_void_p).value
    return arr


def test_run_calls_validation(lib):
    failed = ctypes.c_int32(-7)
    R = lib.ep_run_calls
    assert R(_calls(), 0, ctypes.byref(failed)) == 0 and failed.value == 0   # nothing to do
    assert R(None, 0, None) == 0
    assert R(_calls(), -1, ctypes.byref(failed)) == 1
    assert R(None, 2, ctypes.byref(failed)) == 1
    g, h, _ = make_handle(lib)
    hp = h   # already a c_void_p
    # an unknown op stops the list at its index
    assert R(_calls((99, 0, [hp])), 1, ctypes.byref(failed)) == 1 and failed.value == 0
    # each call returns exactly what its entry point returns: the second call
    # here is an ep_plan with the wrong tag (EP_ERR_BAD_TAG), so the list
    # stops there; the first (wrong shape, EP_ERR_BAD_SHAPE) stops it sooner
    bad_tag = T(I32, ep.TAG_TOKENS, 64, 2)
    bad_shape = T(I32, ep.TAG_TOPK_IDX, 64, 3)
    assert lib.ep_plan(h, bad_tag, None) == 2 and lib.ep_plan(h, bad_shape, None) == 4
    assert R(_calls((3, 0, [hp, bad_tag, None])), 1, ctypes.byref(failed)) == 2 and failed.value == 0
    assert R(_calls((3, 0, [hp, bad_shape, None]), (3, 0, [hp, bad_tag, None])), 2,
             ctypes.byref(failed)) == 4 and failed.value == 0
    # ep_quantize_fp8 takes its scale format from i0: 2 is not a format
    x = T(BF16, ep.TAG_TOKENS, 4, 256)
    q = T(FP8, ep.TAG_TOKENS, 4, 256)
    s = T(F32, ep.TAG_FP8_SCALES, 4, 2)
    assert R(_calls((6, 2, [x, q, s, None])), 1, ctypes.byref(failed)) == \
        lib.ep_quantize_fp8(x, q, s, 2, None) == 1
    lib.ep_handle_destroy(h)
    lib.ep_group_destroy(g)
