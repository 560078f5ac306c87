"""MoE expert-parallel token dispatch / combine / static-shape planner for
MI355X (gfx950).

A thin binding over ``libep_mi355x.so`` (C ABI in ``include/ep.h``).  It only
marshals arguments: torch tensors provide device memory and the stream, and
every step of the path runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if the library is missing the calls raise.

The functions ``ep_group_create`` ... ``ep_dup_grad_reduce`` mirror the C
entry points one to one.  ``Group`` / ``Handle`` / ``Buffer`` wrap them in
the group -> handle -> dispatch -> expert -> combine flow of the NCCL EP
paper (listing, Table II and Figure 2), and ``Buffer.dispatch`` returns
``recv_x, recv_i, recv_w, handle, event`` like that paper's Table V.
"""

from __future__ import annotations

import ctypes
import os
import threading
from ctypes import POINTER, c_int32, c_int64, c_size_t, c_uint32, c_void_p

import torch

__all__ = [
    "EpError", "LAYOUT_LL", "LAYOUT_HT", "LAYOUT_STATIC", "FLAG_INDEX_RANGE", "FLAG_CAPACITY",
    "FLAG_SLOT_BUDGET", "FLAG_PLAN_STALL", "FLAG_SCALE_FORMAT", "Group", "Handle", "Buffer", "library_path", "load_library",
    "ep_status_string", "ep_group_create", "ep_group_destroy", "ep_group_recv_rows",
    "ep_handle_workspace_bytes", "ep_handle_create", "ep_handle_create_static", "ep_handle_destroy",
    "ep_handle_query",
    "ep_handle_status", "ep_route", "ep_route_plan", "ep_plan", "ep_dispatch", "ep_plan_dispatch",
    "ep_quantize_fp8", "ep_combine", "ep_combine_bwd", "prepare", "Prepared",
    "ep_dup_grad_reduce", "ep_prefetch_replicas", "ep_expert_gemm", "ep_expert_gemm_fp8",
    "ep_expert_gemm_swiglu", "ep_expert_gemm_fp8_swiglu", "ep_run_calls", "ep_call_t",
    "SLOTS_TRAINING",
    "SLOTS_INFERENCE",
    "STORES_AUTO", "STORES_CACHED", "STORES_STREAMING", "FP8_SCALES_AMAX", "FP8_SCALES_POW2",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libep_mi355x.so"

LAYOUT_LL, LAYOUT_HT, LAYOUT_STATIC = 0, 1, 2
_LAYOUTS = {"ll": LAYOUT_LL, "ht": LAYOUT_HT, "static": LAYOUT_STATIC}
FLAG_INDEX_RANGE, FLAG_CAPACITY, FLAG_SLOT_BUDGET, FLAG_PLAN_STALL, FLAG_SCALE_FORMAT = 1, 2, 4, 8, 16
TAG_TOKENS, TAG_TOPK_IDX, TAG_TOPK_WEIGHTS, TAG_FP8_SCALES, TAG_EXPERT_GRADS = 0, 1, 2, 3, 4
TAG_ROUTER_LOGITS, TAG_EXPERT_WEIGHTS = 5, 6
SLOTS_TRAINING, SLOTS_INFERENCE = 0, 1
_SLOT_MODES = {"training": SLOTS_TRAINING, "inference": SLOTS_INFERENCE}
STORES_AUTO, STORES_CACHED, STORES_STREAMING = 0, 1, 2
_STORES = {"auto": STORES_AUTO, "cached": STORES_CACHED, "streaming": STORES_STREAMING}
FP8_SCALES_AMAX, FP8_SCALES_POW2, FP8_SCALES_AMAX_POW2_WEIGHTS = 0, 1, 2
_FP8_SCALES = {"amax": FP8_SCALES_AMAX, "pow2": FP8_SCALES_POW2,
               "amax_pow2w": FP8_SCALES_AMAX_POW2_WEIGHTS}
_DTYPES = {torch.bfloat16: 0, torch.float32: 1, torch.float8_e4m3fn: 2, torch.int32: 3}
_STATUS = ["EP_OK", "EP_ERR_INVALID_ARG", "EP_ERR_BAD_TAG", "EP_ERR_BAD_DTYPE",
           "EP_ERR_BAD_SHAPE", "EP_ERR_NOT_PLANNED", "EP_ERR_WORKSPACE_TOO_SMALL",
           "EP_ERR_UNSUPPORTED", "EP_ERR_HIP"]


class EpError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        name = _STATUS[code] if 0 <= code < len(_STATUS) else str(code)
        super().__init__(f"{what} failed: {name}")


class ep_tensor_t(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("tag", c_int32), ("ndim", c_int32),
                ("reserved", c_int32), ("sizes", c_int64 * 4)]


class ep_group_config_t(ctypes.Structure):
    _fields_ = [("num_experts", c_int32), ("num_ranks", c_int32), ("hidden", c_int32),
                ("top_k", c_int32), ("max_tokens", c_int32), ("layout", c_int32),
                ("capacity", c_int32), ("slots_per_rank", c_int32), ("slot_mode", c_int32),
                ("dispatch_stores", c_int32), ("passes_in_flight", c_int32),
                ("fp8_scales", c_int32), ("combine_stores", c_int32)]


class ep_call_t(ctypes.Structure):
    """One recorded call for ep_run_calls: op, integer argument, pointers."""
    _fields_ = [("op", c_int32), ("i0", c_int32), ("p", c_void_p * 9)]


_OPS = {"ep_route": 1, "ep_route_plan": 2, "ep_plan": 3, "ep_dispatch": 4, "ep_plan_dispatch": 5,
        "ep_quantize_fp8": 6, "ep_combine": 7, "ep_combine_bwd": 8, "ep_dup_grad_reduce": 9,
        "ep_prefetch_replicas": 10, "ep_expert_gemm": 11, "ep_expert_gemm_swiglu": 12,
        "ep_expert_gemm_fp8": 13, "ep_expert_gemm_fp8_swiglu": 14}


class ep_handle_view_t(ctypes.Structure):
    _fields_ = [("num_tokens", c_int32), ("top_k", c_int32), ("num_experts", c_int32),
                ("num_ranks", c_int32), ("recv_rows", c_int64), ("rank_rows", c_int32),
                ("max_segments", c_int32)] + [
        (n, c_void_p) for n in ("counts", "offsets", "dst", "recv_src", "status", "keep",
                                "native_row", "seg_first", "seg_count", "segments",
                                "n_segments", "load", "replica", "seg_slot")]


_lib = None
_T = POINTER(ep_tensor_t)


def library_path() -> str:
    """The in-tree libep_mi355x.so, or the file EP_MI355X_LIB names (e.g. the
    host-sanitized build of the same sources)."""
    return os.environ.get("EP_MI355X_LIB") or os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libep_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m combine_ep_plan_amd.build`"
                           " (there is no fallback path)")
    lib = ctypes.CDLL(path)
    S = c_int32
    sig = {
        "ep_status_string": (ctypes.c_char_p, [S]),
        "ep_group_create": (S, [POINTER(ep_group_config_t), POINTER(c_void_p)]),
        "ep_group_destroy": (S, [c_void_p]),
        "ep_group_recv_rows": (S, [c_void_p, c_int32, POINTER(c_int64)]),
        "ep_handle_workspace_bytes": (S, [c_void_p, c_int32, POINTER(c_size_t)]),
        "ep_handle_create": (S, [c_void_p, c_int32, c_void_p, c_size_t, POINTER(c_void_p)]),
        "ep_handle_create_static": (S, [c_void_p, c_int32, c_void_p, POINTER(c_void_p)]),
        "ep_handle_destroy": (S, [c_void_p]),
        "ep_handle_query": (S, [c_void_p, POINTER(ep_handle_view_t)]),
        "ep_handle_status": (S, [c_void_p, c_void_p, POINTER(c_uint32)]),
        "ep_route": (S, [c_void_p, _T, _T, _T, c_void_p]),
        "ep_route_plan": (S, [c_void_p, _T, _T, _T, c_void_p]),
        "ep_plan": (S, [c_void_p, _T, c_void_p]),
        "ep_dispatch": (S, [c_void_p, _T, _T, _T, _T, _T, _T, c_void_p]),
        "ep_plan_dispatch": (S, [c_void_p, _T, _T, _T, _T, _T, _T, _T, c_void_p]),
        "ep_quantize_fp8": (S, [_T, _T, _T, c_int32, c_void_p]),
        "ep_combine": (S, [c_void_p, _T, _T, _T, c_void_p]),
        "ep_combine_bwd": (S, [c_void_p, _T, _T, _T, _T, _T, c_void_p]),
        "ep_dup_grad_reduce": (S, [c_void_p, _T, _T, _T, c_void_p]),
        "ep_prefetch_replicas": (S, [c_void_p, _T, _T, c_void_p]),
        "ep_expert_gemm": (S, [c_void_p, _T, _T, _T, _T, c_void_p]),
        "ep_expert_gemm_fp8": (S, [c_void_p, _T, _T, _T, _T, _T, _T, _T, c_void_p]),
        "ep_expert_gemm_swiglu": (S, [c_void_p, _T, _T, _T, _T, c_void_p]),
        "ep_expert_gemm_fp8_swiglu": (S, [c_void_p, _T, _T, _T, _T, _T, _T, _T, c_void_p]),
        "ep_run_calls": (S, [POINTER(ep_call_t), c_int32, POINTER(c_int32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, what: str) -> None:
    if code != 0:
        raise EpError(code, what)


_VIEWS: dict = {}
_VIEWS_MAX = 4096
_RECORDING = threading.local()   # prepare(): the calls being recorded and what they use


def _tensor(t: torch.Tensor | None, tag: int):
    """ep_tensor_t view of a contiguous device tensor (None -> NULL).  A view
    is a pure function of (address, dtype, shape, tag) and the library never
    writes to it, so built views are kept and reused: the marshalling of a
    call that repeats its tensors costs a dictionary lookup."""
    if t is None:
        return None
    keep = getattr(_RECORDING, "keep", None)
    if keep is not None:   # a prepared call holds on to its tensors
        keep.append(t)
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    key = (t.data_ptr(), t.dtype, t.shape, tag)
    v = _VIEWS.get(key)
    if v is not None:
        return v
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError("tensors must have 1..4 dimensions")
    sizes = (c_int64 * 4)(*(int(x) for x in t.shape))
    v = ctypes.pointer(ep_tensor_t(t.data_ptr() if t.numel() > 0 else None, _DTYPES[t.dtype], tag,
                                   t.dim(), 0, sizes))
    if len(_VIEWS) >= _VIEWS_MAX:
        _VIEWS.clear()
    _VIEWS[key] = v
    return v


def _stream(stream) -> c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    keep = getattr(_RECORDING, "keep", None)
    if keep is not None:
        keep.append(stream)
    if isinstance(stream, torch.cuda.Stream):
        return c_void_p(stream.cuda_stream)
    return c_void_p(int(stream))


# Compute entry points only enqueue work, so a call is fully described by the
# C function and its marshalled arguments.  prepare() records them once; its
# result makes the same C calls again without marshalling anything in Python
# (each call still validates its arguments in the library and enqueues its
# kernels).  For launch-bound loops such as low-latency decode, where the
# marshalling costs about as much host time as the launch itself.


def _enqueue(name: str, *args) -> None:
    fn = getattr(load_library(), name)
    calls = getattr(_RECORDING, "calls", None)
    if calls is not None:
        calls.append((fn, args, name))
        return
    _check(fn(*args), name)


class Prepared:
    """Library calls with their arguments marshalled once (see prepare),
    replayed by one ep_run_calls call.  It holds references to the tensors,
    views and streams the calls name; the tensors' storage must not be moved
    (no resize or reallocation) while it is in use."""

    def __init__(self, calls, keep):
        self.calls = tuple(calls)
        self.names = tuple(n for _, _, n in self.calls)
        self._keep = tuple(keep)
        n = len(self.calls)
        self._arr = (ep_call_t * max(n, 1))()
        for k, (_, args, name) in enumerate(self.calls):
            c = self._arr[k]
            c.op = _OPS[name]
            m = 0
            for a in args:
                if isinstance(a, (c_int32, int)):   # ep_quantize_fp8's scale format
                    c.i0 = a.value if isinstance(a, c_int32) else int(a)
                    continue
                c.p[m] = None if a is None else ctypes.cast(a, c_void_p).value
                m += 1
        self._n = c_int32(n)
        self._failed = c_int32(0)
        self._run = load_library().ep_run_calls

    def __call__(self) -> None:
        code = self._run(self._arr, self._n, ctypes.byref(self._failed))
        if code != 0:
            raise EpError(code, self.names[self._failed.value] if self._failed.value < len(self.names)
                          else "ep_run_calls")


def prepare(fn) -> Prepared:
    """Runs ``fn()`` -- a function making compute calls of this module (route,
    plan, dispatch, combine, GEMMs, ...) -- with nothing enqueued, recording
    each C call and its marshalled arguments, and returns a Prepared object
    that repeats them.  Object-creating and querying calls are not recorded
    and must not be made inside ``fn``."""
    if getattr(_RECORDING, "calls", None) is not None:
        raise RuntimeError("prepare() does not nest")
    _RECORDING.calls, _RECORDING.keep = [], []
    try:
        fn()
        return Prepared(_RECORDING.calls, _RECORDING.keep)
    finally:
        _RECORDING.calls = _RECORDING.keep = None


# ---------------------------------------------------------------------------
# one-to-one wrappers of the C entry points
# ---------------------------------------------------------------------------

def ep_run_calls(calls, n: int) -> int:
    """Makes n recorded calls (a ctypes array of ep_call_t) in one entry into
    the library; raises at the first that fails and returns n otherwise."""
    failed = c_int32(0)
    code = load_library().ep_run_calls(calls, int(n), ctypes.byref(failed))
    if code != 0:
        raise EpError(code, f"ep_run_calls (call {failed.value})")
    return failed.value


def ep_status_string(code: int) -> str:
    return load_library().ep_status_string(int(code)).decode()


def ep_group_create(cfg: ep_group_config_t) -> int:
    out = c_void_p()
    _check(load_library().ep_group_create(ctypes.byref(cfg), ctypes.byref(out)), "ep_group_create")
    return out.value


def ep_group_destroy(g: int) -> None:
    _check(load_library().ep_group_destroy(c_void_p(g)), "ep_group_destroy")


def ep_group_recv_rows(g: int, num_tokens: int) -> int:
    out = c_int64()
    _check(load_library().ep_group_recv_rows(c_void_p(g), num_tokens, ctypes.byref(out)),
           "ep_group_recv_rows")
    return out.value


def ep_handle_workspace_bytes(g: int, num_tokens: int) -> int:
    out = c_size_t()
    _check(load_library().ep_handle_workspace_bytes(c_void_p(g), num_tokens, ctypes.byref(out)),
           "ep_handle_workspace_bytes")
    return out.value


def ep_handle_create(g: int, num_tokens: int, workspace_ptr: int, workspace_bytes: int) -> int:
    out = c_void_p()
    _check(load_library().ep_handle_create(c_void_p(g), num_tokens, c_void_p(workspace_ptr),
                                           workspace_bytes, ctypes.byref(out)), "ep_handle_create")
    return out.value


def ep_handle_create_static(g: int, num_tokens: int, stream=None) -> int:
    out = c_void_p()
    _check(load_library().ep_handle_create_static(c_void_p(g), num_tokens, _stream(stream),
                                                  ctypes.byref(out)), "ep_handle_create_static")
    return out.value


def ep_handle_destroy(h: int) -> None:
    _check(load_library().ep_handle_destroy(c_void_p(h)), "ep_handle_destroy")


def ep_handle_query(h: int) -> ep_handle_view_t:
    v = ep_handle_view_t()
    _check(load_library().ep_handle_query(c_void_p(h), ctypes.byref(v)), "ep_handle_query")
    return v


def ep_handle_status(h: int, stream=None) -> int:
    out = c_uint32()
    _check(load_library().ep_handle_status(c_void_p(h), _stream(stream), ctypes.byref(out)),
           "ep_handle_status")
    return out.value


def ep_route(h: int, logits: torch.Tensor, topk_idx: torch.Tensor,
             topk_weights: torch.Tensor, stream=None) -> None:
    _enqueue("ep_route", c_void_p(h), _tensor(logits, TAG_ROUTER_LOGITS),
             _tensor(topk_idx, TAG_TOPK_IDX), _tensor(topk_weights, TAG_TOPK_WEIGHTS),
             _stream(stream))


def ep_route_plan(h: int, logits: torch.Tensor, topk_idx: torch.Tensor,
                  topk_weights: torch.Tensor, stream=None) -> None:
    _enqueue("ep_route_plan", c_void_p(h), _tensor(logits, TAG_ROUTER_LOGITS),
             _tensor(topk_idx, TAG_TOPK_IDX), _tensor(topk_weights, TAG_TOPK_WEIGHTS),
             _stream(stream))


def ep_plan(h: int, topk_idx: torch.Tensor, stream=None) -> None:
    _enqueue("ep_plan", c_void_p(h), _tensor(topk_idx, TAG_TOPK_IDX), _stream(stream))


def ep_dispatch(h: int, tokens: torch.Tensor, topk_weights: torch.Tensor | None,
                recv_tokens: torch.Tensor, recv_scales: torch.Tensor | None = None,
                recv_topk_idx: torch.Tensor | None = None,
                recv_topk_weights: torch.Tensor | None = None, stream=None) -> None:
    _enqueue("ep_dispatch", c_void_p(h), _tensor(tokens, TAG_TOKENS),
             _tensor(topk_weights, TAG_TOPK_WEIGHTS), _tensor(recv_tokens, TAG_TOKENS),
             _tensor(recv_scales, TAG_FP8_SCALES), _tensor(recv_topk_idx, TAG_TOPK_IDX),
             _tensor(recv_topk_weights, TAG_TOPK_WEIGHTS), _stream(stream))


def ep_plan_dispatch(h: int, topk_idx: torch.Tensor, tokens: torch.Tensor,
                     topk_weights: torch.Tensor | None, recv_tokens: torch.Tensor,
                     recv_scales: torch.Tensor | None = None, recv_topk_idx: torch.Tensor | None = None,
                     recv_topk_weights: torch.Tensor | None = None, stream=None) -> None:
    _enqueue("ep_plan_dispatch", c_void_p(h), _tensor(topk_idx, TAG_TOPK_IDX),
             _tensor(tokens, TAG_TOKENS), _tensor(topk_weights, TAG_TOPK_WEIGHTS),
             _tensor(recv_tokens, TAG_TOKENS), _tensor(recv_scales, TAG_FP8_SCALES),
             _tensor(recv_topk_idx, TAG_TOPK_IDX), _tensor(recv_topk_weights, TAG_TOPK_WEIGHTS),
             _stream(stream))


def ep_quantize_fp8(tokens: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None,
                    pow2: bool = False) -> None:
    _enqueue("ep_quantize_fp8", _tensor(tokens, TAG_TOKENS), _tensor(codes, TAG_TOKENS),
             _tensor(scales, TAG_FP8_SCALES), c_int32(FP8_SCALES_POW2 if pow2 else FP8_SCALES_AMAX),
             _stream(stream))


def ep_combine(h: int, expert_out: torch.Tensor, topk_weights: torch.Tensor | None,
               out_tokens: torch.Tensor, stream=None) -> None:
    _enqueue("ep_combine", c_void_p(h), _tensor(expert_out, TAG_TOKENS),
             _tensor(topk_weights, TAG_TOPK_WEIGHTS), _tensor(out_tokens, TAG_TOKENS),
             _stream(stream))


def ep_combine_bwd(h: int, grad_tokens: torch.Tensor, expert_out: torch.Tensor,
                   topk_weights: torch.Tensor, grad_expert_out: torch.Tensor,
                   grad_topk_weights: torch.Tensor, stream=None) -> None:
    _enqueue("ep_combine_bwd", c_void_p(h), _tensor(grad_tokens, TAG_TOKENS),
             _tensor(expert_out, TAG_TOKENS), _tensor(topk_weights, TAG_TOPK_WEIGHTS),
             _tensor(grad_expert_out, TAG_TOKENS), _tensor(grad_topk_weights, TAG_TOPK_WEIGHTS),
             _stream(stream))


def ep_dup_grad_reduce(h: int, replica_grads: torch.Tensor, replica_expert: torch.Tensor | None,
                       owner_grads: torch.Tensor, stream=None) -> None:
    _enqueue("ep_dup_grad_reduce", c_void_p(h), _tensor(replica_grads, TAG_EXPERT_GRADS),
             _tensor(replica_expert, TAG_TOPK_IDX), _tensor(owner_grads, TAG_EXPERT_GRADS),
             _stream(stream))


def ep_prefetch_replicas(h: int, expert_weights: torch.Tensor, slot_weights: torch.Tensor,
                         stream=None, scales: bool = False) -> None:
    """``scales``: the tensors are the fp32 scales of FP8 weights (tag FP8_SCALES)."""
    tag = TAG_FP8_SCALES if scales else TAG_EXPERT_WEIGHTS
    _enqueue("ep_prefetch_replicas", c_void_p(h), _tensor(expert_weights, tag),
             _tensor(slot_weights, tag), _stream(stream))


def ep_expert_gemm(h: int, recv_tokens: torch.Tensor, expert_weights: torch.Tensor,
                   slot_weights: torch.Tensor | None, out: torch.Tensor, stream=None,
                   swiglu: bool = False) -> None:
    name = "ep_expert_gemm_swiglu" if swiglu else "ep_expert_gemm"
    _enqueue(name, c_void_p(h), _tensor(recv_tokens, TAG_TOKENS),
             _tensor(expert_weights, TAG_EXPERT_WEIGHTS),
             _tensor(slot_weights, TAG_EXPERT_WEIGHTS), _tensor(out, TAG_TOKENS), _stream(stream))


def ep_expert_gemm_swiglu(h: int, recv_tokens: torch.Tensor, expert_weights: torch.Tensor,
                          slot_weights: torch.Tensor | None, out: torch.Tensor, stream=None) -> None:
    ep_expert_gemm(h, recv_tokens, expert_weights, slot_weights, out, stream, swiglu=True)


def ep_expert_gemm_fp8(h: int, recv_tokens: torch.Tensor, recv_scales: torch.Tensor,
                       expert_weights: torch.Tensor, expert_scales: torch.Tensor,
                       slot_weights: torch.Tensor | None, slot_scales: torch.Tensor | None,
                       out: torch.Tensor, stream=None, swiglu: bool = False) -> None:
    name = "ep_expert_gemm_fp8_swiglu" if swiglu else "ep_expert_gemm_fp8"
    _enqueue(name, c_void_p(h), _tensor(recv_tokens, TAG_TOKENS),
             _tensor(recv_scales, TAG_FP8_SCALES), _tensor(expert_weights, TAG_EXPERT_WEIGHTS),
             _tensor(expert_scales, TAG_FP8_SCALES), _tensor(slot_weights, TAG_EXPERT_WEIGHTS),
             _tensor(slot_scales, TAG_FP8_SCALES), _tensor(out, TAG_TOKENS), _stream(stream))


def ep_expert_gemm_fp8_swiglu(h: int, recv_tokens: torch.Tensor, recv_scales: torch.Tensor,
                              expert_weights: torch.Tensor, expert_scales: torch.Tensor,
                              slot_weights: torch.Tensor | None, slot_scales: torch.Tensor | None,
                              out: torch.Tensor, stream=None) -> None:
    ep_expert_gemm_fp8(h, recv_tokens, recv_scales, expert_weights, expert_scales, slot_weights,
                       slot_scales, out, stream, swiglu=True)


# ---------------------------------------------------------------------------
# group / handle / buffer objects
# ---------------------------------------------------------------------------

class Group:
    """Long-lived configuration (experts, ranks, hidden size, top-k, layout)."""

    def __init__(self, num_experts: int, num_ranks: int, hidden: int, top_k: int,
                 max_tokens: int, layout: str | int = "ht", capacity: int = 0,
                 slots_per_rank: int = 0, slot_mode: str | int = "training",
                 dispatch_stores: str | int = "auto", passes_in_flight: int = 1,
                 fp8_scales: str | int = "amax", combine_stores: str | int = "auto"):
        self.layout = _LAYOUTS[layout] if isinstance(layout, str) else int(layout)
        mode = _SLOT_MODES[slot_mode] if isinstance(slot_mode, str) else int(slot_mode)
        stores = _STORES[dispatch_stores] if isinstance(dispatch_stores, str) else int(dispatch_stores)
        f8 = _FP8_SCALES[fp8_scales] if isinstance(fp8_scales, str) else int(fp8_scales)
        cstores = _STORES[combine_stores] if isinstance(combine_stores, str) else int(combine_stores)
        self.cfg = ep_group_config_t(num_experts, num_ranks, hidden, top_k, max_tokens,
                                     self.layout, capacity, slots_per_rank, mode, stores,
                                     passes_in_flight, f8, cstores)
        self.ptr = ep_group_create(self.cfg)

    @property
    def num_experts(self):
        return self.cfg.num_experts

    @property
    def hidden(self):
        return self.cfg.hidden

    @property
    def top_k(self):
        return self.cfg.top_k

    def recv_rows(self, num_tokens: int) -> int:
        return ep_group_recv_rows(self.ptr, num_tokens)

    def recv_shape(self, num_tokens: int) -> tuple[int, ...]:
        c = self.cfg
        rows = self.recv_rows(num_tokens)
        if self.layout == LAYOUT_LL:
            return (c.num_experts, c.capacity, c.hidden)
        if self.layout == LAYOUT_STATIC:
            return (c.num_ranks, rows // c.num_ranks, c.hidden)
        return (rows, c.hidden)

    def workspace_bytes(self, num_tokens: int) -> int:
        return ep_handle_workspace_bytes(self.ptr, num_tokens)

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.ep_group_destroy(c_void_p(self.ptr))
            self.ptr = None


class Handle:
    """Per-pass routing state over a device workspace owned by this object."""

    def __init__(self, group: Group, num_tokens: int, device: torch.device | str | None = None):
        self.group = group
        self.num_tokens = num_tokens
        nbytes = group.workspace_bytes(num_tokens)
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.ptr = ep_handle_create(group.ptr, num_tokens, self.workspace.data_ptr(), nbytes)
        self._view = ep_handle_query(self.ptr)

    def route(self, logits: torch.Tensor, stream=None):
        """Top-k routing of this pass: returns (topk_idx int32 [T,k], weights fp32 [T,k])."""
        k = self.group.top_k
        idx = torch.empty((self.num_tokens, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((self.num_tokens, k), dtype=torch.float32, device=logits.device)
        ep_route(self.ptr, logits, idx, w, stream)
        return idx, w

    def route_plan(self, logits: torch.Tensor, stream=None):
        """Routing and the layout of its ids in one pass (ep_route + ep_plan,
        one launch fewer): returns (topk_idx, weights); the handle is planned."""
        k = self.group.top_k
        idx = torch.empty((self.num_tokens, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((self.num_tokens, k), dtype=torch.float32, device=logits.device)
        ep_route_plan(self.ptr, logits, idx, w, stream)
        return idx, w

    def plan(self, topk_idx: torch.Tensor, stream=None) -> "Handle":
        ep_plan(self.ptr, topk_idx, stream)
        return self

    def status(self, stream=None) -> int:
        return ep_handle_status(self.ptr, stream)

    @property
    def recv_rows(self) -> int:
        return self._view.recv_rows

    @property
    def rank_rows(self) -> int:
        return self._view.rank_rows

    def _ws(self, ptr: int | None, count: int) -> torch.Tensor | None:
        if not ptr:
            return None
        off = ptr - self.workspace.data_ptr()
        return self.workspace[off: off + 4 * count].view(torch.int32)

    def tables(self) -> dict[str, torch.Tensor]:
        """Views (no copies) of the layout and plan tables in the workspace."""
        v = self._view
        E, R, T, k = v.num_experts, v.num_ranks, v.num_tokens, v.top_k
        out = {
            "counts": self._ws(v.counts, E),
            "offsets": self._ws(v.offsets, E + 1),
            "dst": self._ws(v.dst, T * k).view(T, k) if T * k else self._ws(v.dst, 0),
            "recv_src": self._ws(v.recv_src, v.recv_rows),
            "status": self._ws(v.status, 1),
        }
        if v.keep:
            S = self.group.cfg.slots_per_rank
            out.update({
                "keep": self._ws(v.keep, E), "native_row": self._ws(v.native_row, E),
                "seg_first": self._ws(v.seg_first, E), "seg_count": self._ws(v.seg_count, E),
                "segments": self._ws(v.segments, 5 * v.max_segments).view(v.max_segments, 5),
                "n_segments": self._ws(v.n_segments, 1), "load": self._ws(v.load, R),
                "replica": self._ws(v.replica, R * S).view(R, S),
                "seg_slot": self._ws(v.seg_slot, v.max_segments),
            })
        return out

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.ep_handle_destroy(c_void_p(self.ptr))
            self.ptr = None


class Buffer:
    """Framework-facing operations (NCCL EP paper listing, Table V)."""

    def __init__(self, group: Group):
        self.group = group

    def handle(self, num_tokens: int, device=None) -> Handle:
        return Handle(self.group, num_tokens, device)

    def dispatch(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor | None,
                 handle: Handle | None = None, fp8: bool = False, recv_meta: bool = True,
                 out: torch.Tensor | None = None, stream=None):
        """Dispatch; with ``handle`` None, first plan ``topk_idx`` on a new
        handle for these tokens (a handle passed in must already be planned).
        Returns ``recv_x, recv_i, recv_w, handle, event`` (plus the FP8 scales
        as ``recv_x = (codes, scales)`` when ``fp8``)."""
        T = x.shape[0]
        plan = handle is None
        if plan:
            handle = Handle(self.group, T, x.device)
        rows = handle.recv_rows
        shape = self.group.recv_shape(T)
        H = self.group.hidden
        scales = None
        if fp8:
            recv = out if out is not None else torch.empty(shape, dtype=torch.float8_e4m3fn, device=x.device)
            scales = torch.empty((rows, H // 128), dtype=torch.float32, device=x.device)
        else:
            recv = out if out is not None else torch.empty(shape, dtype=torch.bfloat16, device=x.device)
        ri = torch.empty(rows, dtype=torch.int32, device=x.device) if recv_meta else None
        rw = torch.empty(rows, dtype=torch.float32, device=x.device) if (recv_meta and topk_weights is not None) else None
        if plan:   # the layout and the dispatch together (one launch for small batches)
            ep_plan_dispatch(handle.ptr, topk_idx, x, topk_weights, recv, scales, ri, rw, stream)
        else:
            ep_dispatch(handle.ptr, x, topk_weights, recv, scales, ri, rw, stream)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream() if stream is None else stream)
        recv_x = (recv, scales) if fp8 else recv
        return recv_x, ri, rw, handle, ev

    def combine(self, expert_out: torch.Tensor, handle: Handle,
                topk_weights: torch.Tensor | None, out_dtype=torch.bfloat16,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        T, H = handle.num_tokens, self.group.hidden
        y = out if out is not None else torch.empty((T, H), dtype=out_dtype, device=expert_out.device)
        ep_combine(handle.ptr, expert_out, topk_weights, y, stream)
        return y

    def dispatch_bwd(self, grad_recv: torch.Tensor, handle: Handle, stream=None) -> torch.Tensor:
        """Gradient of dispatch: sum of each token's received-row gradients."""
        return self.combine(grad_recv, handle, None, stream=stream)

    def combine_bwd(self, grad_y: torch.Tensor, expert_out: torch.Tensor,
                    topk_weights: torch.Tensor, handle: Handle, stream=None):
        grad_out = torch.empty_like(expert_out)
        grad_w = torch.empty_like(topk_weights)
        ep_combine_bwd(handle.ptr, grad_y, expert_out, topk_weights, grad_out, grad_w, stream)
        return grad_out, grad_w

    def prefetch_replicas(self, expert_weights: torch.Tensor, handle: Handle,
                          slots: torch.Tensor | None = None, stream=None,
                          scales: bool = False) -> torch.Tensor:
        """Copy the plan's replica experts' weights ([E, P...]) into their
        prefetch slots ([R, S, P...]); slots the plan leaves empty keep their
        contents (uninitialised if ``slots`` is None).  ``scales``: the
        tensor is the fp32 scales of FP8 weights."""
        c = self.group.cfg
        if slots is None:
            slots = torch.empty((c.num_ranks, c.slots_per_rank) + tuple(expert_weights.shape[1:]),
                                dtype=expert_weights.dtype, device=expert_weights.device)
        ep_prefetch_replicas(handle.ptr, expert_weights, slots, stream, scales=scales)
        return slots

    def expert_gemm(self, recv: torch.Tensor, expert_weights: torch.Tensor, handle: Handle,
                    slots: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    stream=None, swiglu: bool = False) -> torch.Tensor:
        """Grouped GEMM of the experts over the received rows: ``recv``
        [rows, K] (any leading shape) times each group's [N, K] weights.
        With ``swiglu`` the weight rows interleave gate (even) and up (odd)
        projections and the result is [rows, N/2] of silu(gate) * up."""
        N = expert_weights.shape[1]
        rows = handle.recv_rows
        if out is None:
            out = torch.empty((rows, N // 2 if swiglu else N), dtype=torch.bfloat16, device=recv.device)
        ep_expert_gemm(handle.ptr, recv.view(rows, expert_weights.shape[2]), expert_weights, slots,
                       out, stream, swiglu=swiglu)
        return out

    def expert_gemm_fp8(self, recv: torch.Tensor, recv_scales: torch.Tensor,
                        expert_weights: torch.Tensor, expert_scales: torch.Tensor, handle: Handle,
                        slots: torch.Tensor | None = None, slot_scales: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, stream=None,
                        swiglu: bool = False) -> torch.Tensor:
        """The grouped GEMM on FP8 operands: ``recv`` e4m3 [rows, K] with fp32
        ``recv_scales`` [rows, K/128] (the FP8 dispatch output), weights e4m3
        [E, N, K] with fp32 scales [E, N, K/128].  ``swiglu`` as in
        ``expert_gemm``."""
        N, K = expert_weights.shape[1], expert_weights.shape[2]
        rows = handle.recv_rows
        if out is None:
            out = torch.empty((rows, N // 2 if swiglu else N), dtype=torch.bfloat16, device=recv.device)
        ep_expert_gemm_fp8(handle.ptr, recv.view(rows, K), recv_scales.view(rows, K // 128),
                           expert_weights, expert_scales, slots, slot_scales, out, stream,
                           swiglu=swiglu)
        return out

    @staticmethod
    def quantize_fp8(x: torch.Tensor, codes: torch.Tensor | None = None,
                     scales: torch.Tensor | None = None, stream=None, pow2: bool = False):
        """bf16 rows [..., K] (K % 128 == 0) to e4m3 codes of the same shape
        and fp32 scales [..., K/128], bit for bit the FP8 dispatch's
        quantisation (``pow2``: power-of-two scales, as a group with
        fp8_scales="pow2"); for the activation between the two FFN GEMMs,
        or for FP8 weights."""
        K = x.shape[-1]
        if codes is None:
            codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
        if scales is None:
            scales = torch.empty(tuple(x.shape[:-1]) + (K // 128,), dtype=torch.float32, device=x.device)
        ep_quantize_fp8(x, codes, scales, stream, pow2=pow2)
        return codes, scales

    def dup_grad_reduce(self, replica_grads: torch.Tensor, owner_grads: torch.Tensor,
                        handle: Handle, replica_expert: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
        ep_dup_grad_reduce(handle.ptr, replica_grads, replica_expert, owner_grads, stream)
        return owner_grads
