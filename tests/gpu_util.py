"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device
and results back, building small oracle problems from sampled tokens."""

from __future__ import annotations

import numpy as np
import torch

import combine_ep_plan_amd as ep
import oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def make_group(E, R, H, k, T, kind, cap=0, S=0, mode="training", fp8_scales="amax") -> ep.Group:
    return ep.Group(E, R, H, k, max(T, 1), kind, capacity=cap, slots_per_rank=S, slot_mode=mode,
                    fp8_scales=fp8_scales)


def check_layout(h: ep.Handle, L: "oracle.Layout", kind: str, idx: np.ndarray, w: np.ndarray | None):
    """Bit-exact comparison of every layout / plan table with the oracle."""
    torch.cuda.synchronize()
    tb = {k: (host(v) if v is not None else None) for k, v in h.tables().items()}
    assert np.array_equal(tb["counts"], L.counts), "counts"
    assert np.array_equal(tb["offsets"], L.offsets), "offsets"
    assert np.array_equal(tb["dst"].reshape(L.dst.shape), L.dst), "dst"
    src, _, _ = oracle.recv_meta(idx, w, L.dst, L.rows)
    used = L.dst[L.dst >= 0]          # recv_src is defined on the rows that hold an entry
    assert np.array_equal(tb["recv_src"][used], src[used]), "recv_src"
    assert h.status() == L.flags, "status flags"
    if kind == "static":
        p = L.plan
        ns = int(tb["n_segments"][0])
        assert ns == p.segments.shape[0], "segment count"
        assert np.array_equal(tb["keep"], p.keep), "keep"
        assert np.array_equal(tb["native_row"], p.native_row), "native_row"
        assert np.array_equal(tb["seg_first"], p.seg_first), "seg_first"
        assert np.array_equal(tb["seg_count"], p.seg_count), "seg_count"
        assert np.array_equal(tb["segments"][:ns], p.segments), "segments"
        assert np.array_equal(tb["load"], p.load), "load"
        assert np.array_equal(tb["replica"], p.replica), "replica"
        assert np.array_equal(tb["seg_slot"][:ns], p.seg_slot), "seg_slot"
        assert h.rank_rows == p.C


def sample_problem(dst: np.ndarray, tokens: np.ndarray, rows: torch.Tensor):
    """Rows used by ``tokens`` gathered from the device buffer ``rows``
    ([n_rows, H] view) plus their dst remapped to the gathered order, so the
    oracle can recompute those tokens' outputs on its own."""
    d = dst[tokens]                                   # [n, k]
    used = np.unique(d[d >= 0])
    remap = np.full(int(d.max(initial=-1)) + 2, -1, np.int64)
    remap[used] = np.arange(used.size)
    local = np.where(d >= 0, remap[np.maximum(d, 0)], -1).astype(np.int32)
    if used.size:
        g = rows.index_select(0, torch.from_numpy(used).cuda())
        gb = host_bits(g)
    else:
        gb = np.zeros((0, rows.shape[-1]), np.uint16)
    return local, gb, used


def same_up_to_zero_sign_np(a: np.ndarray, b: np.ndarray) -> bool:
    """bf16 bit patterns equal once -0 (0x8000) is read as +0."""
    a = np.where(a == 0x8000, 0, a)
    b = np.where(b == 0x8000, 0, b)
    return bool(np.array_equal(a, b))


def same_up_to_zero_sign(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Device version for bf16 tensors of equal shape."""
    ai, bi = a.view(torch.int16), b.view(torch.int16)
    neg0 = torch.tensor(-32768, dtype=torch.int16, device=a.device)
    zero = torch.zeros((), dtype=torch.int16, device=a.device)
    return bool(torch.equal(torch.where(ai == neg0, zero, ai), torch.where(bi == neg0, zero, bi)))
