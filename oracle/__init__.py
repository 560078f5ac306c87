"""CPU oracle for the MoE expert-parallel dispatch / combine / planner path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports it, and it never imports the GPU library: the two share no
code, only the seeded inputs of ``workloads``.

The arithmetic lives in ``ep_oracle.c`` (plain C loops, double precision,
one rounding per output); this module only marshals numpy arrays.  See the
header of ``ep_oracle.c`` for the passages each function follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
# EP_ORACLE_SANITIZE=1: build and load an AddressSanitizer +
# UndefinedBehaviorSanitizer build instead (the sanitizer runtimes must be
# preloaded into the interpreter)
_SANITIZE = os.environ.get("EP_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libep_oracle_san.so" if _SANITIZE else "libep_oracle.so")

FLAG_INDEX_RANGE = 1
FLAG_CAPACITY = 2
FLAG_SLOT_BUDGET = 4

LAYOUT_CODE = {"ll": 0, "ht": 1, "static": 2}
SLOTS_TRAINING = 0     # a rank needing more than S slots raises SLOT_BUDGET
SLOTS_INFERENCE = 1    # segments past the S-th slot read the owner directly


def build(force: bool = True) -> str:
    """Compile ep_oracle.c with gcc (no fused multiply-add, OpenMP on)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        if _SANITIZE:
            cmd[1:1] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-g"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        sig = {
            "orc_set_threads": (None, [ctypes.c_int]),
            "orc_get_threads": (ctypes.c_int, []),
            "orc_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_e4m3_from_float": (ctypes.c_uint8, [ctypes.c_float]),
            "orc_e4m3_to_double": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_layout": (u32, [i32, i32, i32, P, P, P, P]),
            "orc_dst_ht_ll": (u32, [i32, i32, i32, i32, P, P, P, P]),
            "orc_plan": (i32, [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P]),
            "orc_prefetch": (i32, [i32, i32, i32, i64, P, P, P]),
            "orc_dst_static": (None, [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P]),
            "orc_dispatch": (None, [i32, i32, i32, P, P, P]),
            "orc_recv_meta": (None, [i32, i32, i64, P, P, P, P, P, P]),
            "orc_quantize_row_fp8": (None, [i32, P, P, P]),
            "orc_quantize_row_fp8_pow2": (None, [i32, P, P, P]),
            "orc_dispatch_fp8": (None, [i32, i32, i32, P, P, P, P]),
            "orc_dispatch_fp8_pow2": (None, [i32, i32, i32, P, P, P, P]),
            "orc_combine": (None, [i32, i32, i32, P, P, P, i32, P]),
            "orc_combine_bwd": (None, [i32, i32, i32, P, P, P, P, P, P]),
            "orc_dup_reduce": (None, [i32, i64, P, P, i32, P]),
            "orc_route": (None, [i32, i32, i32, P, P, P]),
            "orc_grouped_gemm": (None, [i32, P, i32, i32, P, P, P]),
            "orc_grouped_gemm_fp8": (None, [i32, P, i32, i32, P, P, P, P, P]),
            "orc_swiglu": (None, [i64, i32, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    _L().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_L().orc_get_threads())


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_from_double(v: float) -> int:
    return int(_L().orc_bf16_from_double(float(v)))


def bf16_to_double(b: int) -> float:
    return float(_L().orc_bf16_to_double(int(b)))


def e4m3_from_float(v: float) -> int:
    return int(_L().orc_e4m3_from_float(float(v)))


def e4m3_to_double(c: int) -> float:
    return float(_L().orc_e4m3_to_double(int(c)))


def bf16_to_f32_array(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# layout and planner
# --------------------------------------------------------------------------

@dataclass
class Layout:
    counts: np.ndarray     # [E] int32
    offsets: np.ndarray    # [E+1] int32
    pos: np.ndarray        # [T, k] int32 (-1 skipped)
    dst: np.ndarray        # [T, k] int32 (-1 skipped/dropped)
    flags: int
    rows: int              # rows of the receive buffer
    plan: "Plan | None" = None


@dataclass
class Plan:
    C: int
    keep: np.ndarray
    native_row: np.ndarray
    seg_first: np.ndarray
    seg_count: np.ndarray
    segments: np.ndarray   # [n_seg, 5]: expert, rank, pos_begin, len, row_begin
    load: np.ndarray       # [R]
    replica: np.ndarray    # [R, S]
    seg_slot: np.ndarray   # [n_seg] slot of each segment on its rank, -1 if none
    flags: int


def layout_counts(topk_idx: np.ndarray, E: int):
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    pos = np.zeros((T, k), np.int32)
    flags = _L().orc_layout(T, k, E, _p(idx), _p(counts), _p(offsets), _p(pos))
    return counts, offsets, pos, int(flags)


def plan(counts: np.ndarray, R: int, S: int, C: int, slot_mode: int = SLOTS_TRAINING) -> Plan:
    counts = _c(counts, np.int32)
    E = counts.shape[0]
    keep = np.zeros(E, np.int32)
    native_row = np.zeros(E, np.int32)
    seg_first = np.zeros(E, np.int32)
    seg_count = np.zeros(E, np.int32)
    seg = np.zeros(((E + R) * 5,), np.int32)
    n_seg = np.zeros(1, np.int32)
    load = np.zeros(R, np.int32)
    replica = np.zeros(R * S if S > 0 else 1, np.int32)
    seg_slot = np.zeros(E + R, np.int32)
    flags = np.zeros(1, np.uint32)
    rc = _L().orc_plan(E, R, S, C, slot_mode, _p(counts), _p(keep), _p(native_row),
                       _p(seg_first), _p(seg_count), _p(seg), _p(n_seg), _p(load), _p(replica),
                       _p(seg_slot), _p(flags))
    if rc != 0:
        raise ValueError("orc_plan: inconsistent arguments")
    ns = int(n_seg[0])
    return Plan(C, keep, native_row, seg_first, seg_count, seg[: ns * 5].reshape(ns, 5).copy(),
                load, replica[: R * S].reshape(R, S).copy(), seg_slot[:ns].copy(), int(flags[0]))


def static_rows_per_rank(T: int, k: int, R: int) -> int:
    """Static shape of a rank's buffer: ceil(T*k / R) rows (the planner's step 1)."""
    return -(-(T * k) // R) if R > 0 else 0


def layout(topk_idx: np.ndarray, E: int, kind: str, cap: int = 0, R: int = 1,
           S: int = 0, slot_mode: int = SLOTS_TRAINING) -> Layout:
    """Counts, offsets, positions and destination rows for layout ``kind``."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts, offsets, pos, flags = layout_counts(idx, E)
    dst = np.zeros((T, k), np.int32)
    pl = None
    if kind in ("ht", "ll"):
        flags |= int(_L().orc_dst_ht_ll(T, k, LAYOUT_CODE[kind], cap, _p(idx), _p(pos),
                                         _p(offsets), _p(dst)))
        rows = T * k if kind == "ht" else E * cap
    elif kind == "static":
        C = static_rows_per_rank(T, k, R)
        pl = plan(counts, R, S, C, slot_mode)
        flags |= pl.flags
        segflat = np.ascontiguousarray(pl.segments.reshape(-1)) if pl.segments.size else np.zeros(5, np.int32)
        _L().orc_dst_static(T, k, E, R, C, _p(idx), _p(pos), _p(pl.keep), _p(pl.native_row),
                            _p(pl.seg_first), _p(pl.seg_count), _p(segflat), _p(dst))
        rows = R * C
    else:
        raise ValueError(kind)
    return Layout(counts, offsets, pos, dst, flags, rows, pl)


# --------------------------------------------------------------------------
# data movement and arithmetic
# --------------------------------------------------------------------------

def dispatch(x_bits: np.ndarray, dst: np.ndarray, rows: int, fill: int = 0) -> np.ndarray:
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    d = _c(dst, np.int32)
    k = d.shape[1] if d.ndim == 2 else 1
    recv = np.full((rows, H), fill, np.uint16)
    _L().orc_dispatch(T, k, H, _p(x), _p(d), _p(recv))
    return recv


def recv_meta(topk_idx, topk_w, dst, rows: int):
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    w = None if topk_w is None else _c(topk_w, np.float32)
    d = _c(dst, np.int32)
    src = np.zeros(rows, np.int32)
    ridx = np.zeros(rows, np.int32)
    rw = np.zeros(rows, np.float32)
    _L().orc_recv_meta(T, k, rows, _p(idx), _p(w), _p(d), _p(src), _p(ridx), _p(rw))
    return src, ridx, rw


def quantize_row_fp8(x_bits: np.ndarray, pow2: bool = False):
    """One bf16 row to e4m3 codes and one fp32 scale per 128 channels
    (amax / 448, or with ``pow2`` the power of two at or above it)."""
    x = _c(x_bits, np.uint16).reshape(-1)
    H = x.shape[0]
    q = np.zeros(H, np.uint8)
    s = np.zeros(max(H // 128, 1), np.float32)
    fn = _L().orc_quantize_row_fp8_pow2 if pow2 else _L().orc_quantize_row_fp8
    fn(H, _p(x), _p(q), _p(s))
    return q, s[: H // 128]


def dispatch_fp8(x_bits: np.ndarray, dst: np.ndarray, rows: int, pow2: bool = False):
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    d = _c(dst, np.int32)
    k = d.shape[1]
    q = np.zeros((rows, H), np.uint8)
    s = np.zeros((rows, H // 128), np.float32)
    fn = _L().orc_dispatch_fp8_pow2 if pow2 else _L().orc_dispatch_fp8
    fn(T, k, H, _p(x), _p(d), _p(q), _p(s))
    return q, s


def combine(rows_bits: np.ndarray, dst: np.ndarray, w: np.ndarray | None,
            out_fp32: bool = False) -> np.ndarray:
    rows = _c(rows_bits, np.uint16)
    H = rows.shape[-1]
    d = _c(dst, np.int32)
    T, k = d.shape
    wv = None if w is None else _c(w, np.float32)
    y = np.zeros((T, H), np.float32 if out_fp32 else np.uint16)
    _L().orc_combine(T, k, H, _p(rows), _p(d), _p(wv), 1 if out_fp32 else 0, _p(y))
    return y


def combine_bwd(gy_bits: np.ndarray, out_bits: np.ndarray, dst: np.ndarray, w: np.ndarray,
                rows: int | None = None):
    gy = _c(gy_bits, np.uint16)
    out = _c(out_bits, np.uint16)
    d = _c(dst, np.int32)
    T, k = d.shape
    H = gy.shape[1]
    wv = _c(w, np.float32)
    nrows = out.shape[0] if rows is None else rows
    gout = np.zeros((nrows, H), np.uint16)
    gw = np.zeros((T, k), np.float32)
    _L().orc_combine_bwd(T, k, H, _p(gy), _p(out), _p(d), _p(wv), _p(gout), _p(gw))
    return gout, gw


def dup_reduce(rep_bits: np.ndarray, rep_e: np.ndarray, owner: np.ndarray) -> np.ndarray:
    """Returns the updated copy of ``owner`` ([E, P] fp32)."""
    rep = _c(rep_bits, np.uint16)
    n = rep.shape[0]
    P = int(np.prod(rep.shape[1:])) if n else int(np.prod(owner.shape[1:]))
    re = _c(rep_e, np.int32)
    own = np.array(owner, np.float32, copy=True, order="C")
    E = own.shape[0]
    _L().orc_dup_reduce(n, P, _p(rep), _p(re), E, _p(own))
    return own


def prefetch(weights: np.ndarray, replica: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Replica-weight prefetch: returns a copy of ``slots`` ([R, S, ...]) in
    which every slot (r, s) with replica[r, s] = e >= 0 holds expert e's row
    of ``weights`` ([E, ...], any dtype); empty slots keep their contents."""
    w = np.ascontiguousarray(weights)
    out = np.array(slots, copy=True, order="C")
    rep = _c(replica, np.int32)
    R, S = rep.shape
    E = w.shape[0]
    row_bytes = w[0].nbytes if E else 0
    if out.dtype != w.dtype or out.shape[:2] != (R, S) or out.shape[2:] != w.shape[1:]:
        raise ValueError("prefetch: slots must be [R, S] + weights.shape[1:] of the same dtype")
    rc = _L().orc_prefetch(E, R, S, row_bytes, _p(rep), _p(w), _p(out))
    if rc != 0:
        raise ValueError("orc_prefetch: a slot names an expert outside [0, E)")
    return out


def expert_groups(L: Layout, kind: str, E: int, cap: int = 0, R: int = 1, S: int = 0,
                  use_slots: bool = False) -> np.ndarray:
    """Groups of consecutive receive rows that share one weight matrix, as
    rows (row0, rows, widx).  widx < E is an owner expert; E + r*S + s is
    prefetch slot s of rank r (used for a STATIC segment with a slot when
    ``use_slots``; otherwise, and for overflow segments, the owner).
      HT: expert e holds rows [offsets[e], offsets[e+1]).
      LL: expert e holds rows [e*cap, e*cap + min(counts[e], cap)).
      STATIC: e's kept rows on its home rank e // (E/R) at native_row[e],
              and each segment's rows on its receiving rank."""
    g = []
    if kind == "ht":
        for e in range(E):
            n = int(L.offsets[e + 1] - L.offsets[e])
            if n:
                g.append((int(L.offsets[e]), n, e))
    elif kind == "ll":
        for e in range(E):
            n = min(int(L.counts[e]), cap)
            if n:
                g.append((e * cap, n, e))
    elif kind == "static":
        p = L.plan
        m = E // R
        for e in range(E):
            if p.keep[e]:
                g.append(((e // m) * p.C + int(p.native_row[e]), int(p.keep[e]), e))
        for i, (e, r, _, ln, row) in enumerate(p.segments.tolist()):
            sl = int(p.seg_slot[i])
            g.append((r * p.C + row, ln, E + r * S + sl if (use_slots and sl >= 0) else e))
    else:
        raise ValueError(kind)
    return np.array(g, np.int32).reshape(-1, 3)


def grouped_gemm(x_bits: np.ndarray, w_bits: np.ndarray, groups: np.ndarray,
                 y_bits: np.ndarray | None = None) -> np.ndarray:
    """Y[row0+i, n] = bf16(sum_c X[row0+i, c] * W[widx, n, c]) for every group;
    other rows of Y keep ``y_bits`` (zeros if None).  x_bits [rows, K] and
    w_bits [nW, N, K] are bf16 bit patterns."""
    x = _c(x_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    nW, N, K = w.shape
    if x.shape[1] != K:
        raise ValueError("grouped_gemm: X and W disagree on K")
    gr = _c(groups, np.int32).reshape(-1, 3)
    if gr.size and (gr[:, 0].min() < 0 or (gr[:, 0] + gr[:, 1]).max() > x.shape[0]
                    or gr[:, 2].min() < 0 or gr[:, 2].max() >= nW):
        raise ValueError("grouped_gemm: a group is outside X or names no weight matrix")
    y = np.zeros((x.shape[0], N), np.uint16) if y_bits is None else np.array(y_bits, np.uint16, copy=True, order="C")
    _L().orc_grouped_gemm(gr.shape[0], _p(gr), K, N, _p(x), _p(w), _p(y))
    return y


def swiglu(h_bits: np.ndarray) -> np.ndarray:
    """The expert FFN's activation over [rows, 2I] bf16 bit patterns whose
    column pairs (2j, 2j + 1) hold gate and up: [rows, I] bf16 bits of
    bf16(silu(gate) * up)."""
    h = _c(h_bits, np.uint16)
    if h.ndim != 2 or h.shape[1] % 2 != 0:
        raise ValueError("swiglu: h must be [rows, 2I]")
    out = np.zeros((h.shape[0], h.shape[1] // 2), np.uint16)
    _L().orc_swiglu(h.shape[0], h.shape[1] // 2, _p(h), _p(out))
    return out


def quantize_rows_fp8(bits: np.ndarray, pow2: bool = False):
    """Every row of a bf16 matrix (last axis a multiple of 128) quantised as
    ep_dispatch's FP8 path does: e4m3 codes and one fp32 scale per 128
    (``pow2``: power-of-two scales)."""
    b = _c(bits, np.uint16)
    H = b.shape[-1]
    flat = b.reshape(-1, H)
    q = np.zeros(flat.shape, np.uint8)
    s = np.zeros((flat.shape[0], H // 128), np.float32)
    for r in range(flat.shape[0]):
        q[r], s[r] = quantize_row_fp8(flat[r], pow2)
    return q.reshape(b.shape), s.reshape(b.shape[:-1] + (H // 128,))


def grouped_gemm_fp8(x_codes: np.ndarray, x_scales: np.ndarray, w_codes: np.ndarray,
                     w_scales: np.ndarray, groups: np.ndarray,
                     y_bits: np.ndarray | None = None) -> np.ndarray:
    """The grouped GEMM on FP8 operands: codes (e4m3) with one fp32 scale per
    128 of K, for the rows ([rows, K], [rows, K/128]) and for every output row
    of every weight matrix ([nW, N, K], [nW, N, K/128])."""
    x = _c(x_codes, np.uint8)
    sx = _c(x_scales, np.float32)
    w = _c(w_codes, np.uint8)
    sw = _c(w_scales, np.float32)
    nW, N, K = w.shape
    if K % 128 or x.shape[1] != K or sx.shape != (x.shape[0], K // 128) or sw.shape != (nW, N, K // 128):
        raise ValueError("grouped_gemm_fp8: inconsistent shapes")
    gr = _c(groups, np.int32).reshape(-1, 3)
    if gr.size and (gr[:, 0].min() < 0 or (gr[:, 0] + gr[:, 1]).max() > x.shape[0]
                    or gr[:, 2].min() < 0 or gr[:, 2].max() >= nW):
        raise ValueError("grouped_gemm_fp8: a group is outside X or names no weight matrix")
    y = np.zeros((x.shape[0], N), np.uint16) if y_bits is None else np.array(y_bits, np.uint16, copy=True, order="C")
    _L().orc_grouped_gemm_fp8(gr.shape[0], _p(gr), K, N, _p(x), _p(sx), _p(w), _p(sw), _p(y))
    return y


def route(logits: np.ndarray, k: int):
    """Top-k experts per token (descending logit, ties to the lower id) and the
    softmax over the chosen logits.  Returns (topk_idx int32 [T,k], w fp32 [T,k])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    _L().orc_route(T, E, k, _p(lg), _p(idx), _p(w))
    return idx, w
