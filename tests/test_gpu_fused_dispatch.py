"""GPU parity of ep_plan_dispatch, the layout and the dispatch in one call
(one launch for LL and HT batches of at most 2048 entries: the low-latency
decode regime of the NCCL EP paper listing, abstract and Table III).

Every case checks, bit for bit: every layout table (counts, offsets, dst,
recv_src, status flags) against the oracle; the dispatched rows (bf16, and
FP8 codes and scales) and the per-row expert and weight against the oracle;
and every output against ep_plan followed by ep_dispatch on the same inputs.
Cases above 2048 entries and STATIC layouts take the two-launch path and
must agree as well."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import check_layout, dev_bf16, dev_f32, dev_i32, host, host_bits, make_group

pytestmark = pytest.mark.gpu

SENT = 0x7F7F

# name, T, H, E, k, layout, cap, R, S, mask, bad, dup, skew, seed
CASES = [
    ("decode_ll", 128, 7168, 256, 8, "ll", 128, 32, 0, 0.0, 0.0, 0.0, 0.0, 21),
    ("decode_ll_masked_bad", 128, 1024, 256, 8, "ll", 128, 32, 0, 0.1, 0.03, 0.0, 0.0, 22),
    ("decode_ht", 128, 512, 256, 8, "ht", 0, 32, 0, 0.0, 0.0, 0.0, 1.1, 23),
    ("tiny_ll", 64, 256, 8, 2, "ll", 64, 4, 0, 0.0, 0.0, 0.0, 0.0, 24),
    ("ll_overflow", 200, 128, 16, 8, "ll", 50, 4, 0, 0.0, 0.0, 0.0, 1.5, 25),
    ("ht_dup_k4", 300, 64, 16, 4, "ht", 0, 2, 0, 0.0, 0.0, 0.3, 0.0, 26),
    ("ht_k3_ragged", 333, 136, 37, 3, "ht", 0, 1, 0, 0.05, 0.02, 0.0, 0.8, 27),
    ("ll_k16_e1024_full_tile", 128, 256, 1024, 16, "ll", 4, 8, 0, 0.0, 0.0, 0.0, 1.2, 28),
    ("ht_e1000", 200, 128, 1000, 8, "ht", 0, 8, 0, 0.0, 0.0, 0.0, 0.0, 29),
    ("single", 1, 8, 1, 1, "ht", 0, 1, 0, 0.0, 0.0, 0.0, 0.0, 30),
    ("single_masked", 1, 128, 4, 2, "ll", 2, 2, 0, 1.0, 0.0, 0.0, 0.0, 31),
    ("empty_ht", 0, 64, 8, 2, "ht", 0, 2, 0, 0.0, 0.0, 0.0, 0.0, 32),
    ("empty_ll", 0, 64, 8, 2, "ll", 4, 2, 0, 0.0, 0.0, 0.0, 0.0, 33),
    ("k1_ll", 513, 24, 5, 1, "ll", 200, 5, 0, 0.0, 0.0, 0.0, 0.5, 34),
    # two-launch fallbacks: more than one layout tile, or the static layout
    ("ht_two_tiles", 300, 64, 64, 8, "ht", 0, 8, 0, 0.0, 0.0, 0.0, 1.0, 35),
    ("static_small", 200, 128, 32, 4, "static", 0, 8, 4, 0.0, 0.0, 0.0, 1.2, 36),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def _inputs(c):
    name, T, H, E, k, kind, cap, R, S, mask, bad, dup, skew, seed = c
    idx, w, x = workloads.random_case(2000 + seed, T, H, E, k, mask_frac=mask, bad_frac=bad,
                                      dup_frac=dup, skew=skew)
    return T, H, E, k, kind, cap, R, S, idx, w, x


def _run(g, T, H, idx, w, x, fused, fp8):
    h = ep.Handle(g, T)
    rows = h.recv_rows
    if fp8:
        recv = torch.full((rows, H), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        sc = torch.full((rows, H // 128), -1.0, dtype=torch.float32, device="cuda")
    else:
        recv = torch.full((rows, H), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        sc = None
    ri = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    rw = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
    di, dw, dx = dev_i32(idx), dev_f32(w), dev_bf16(x)
    if fused:
        ep.ep_plan_dispatch(h.ptr, di, dx, dw, recv, sc, ri, rw)
    else:
        ep.ep_plan(h.ptr, di)
        ep.ep_dispatch(h.ptr, dx, dw, recv, sc, ri, rw)
    torch.cuda.synchronize()
    out = {"recv": host(recv.view(torch.uint8)), "ri": host(ri), "rw": host(rw)}
    if fp8:
        out["sc"] = host(sc)
    return h, out


# every case in bf16; in FP8 those whose hidden size is a multiple of 128
# (the FP8 format's block), the only sizes the FP8 dispatch accepts
_PAIRS = [(c, f) for f in (False, True) for c in CASES if not (f and c[2] % 128)]


@pytest.mark.parametrize("c,fp8", _PAIRS, ids=[f"{c[0]}-{'fp8' if f else 'bf16'}" for c, f in _PAIRS])
def test_plan_dispatch_matches_oracle_and_two_calls(c, fp8):
    T, H, E, k, kind, cap, R, S, idx, w, x = _inputs(c)
    print(f"[plan_dispatch] {c[0]} fp8={fp8} T={T} E={E} k={k}", flush=True)
    g = make_group(E, R, H, k, T, kind, cap, S)
    h, got = _run(g, T, H, idx, w, x, True, fp8)
    L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S)
    check_layout(h, L, kind, idx, w)
    used = L.dst[L.dst >= 0]
    if fp8:
        wq, ws = oracle.dispatch_fp8(x, L.dst, L.rows)
        assert np.array_equal(got["recv"].reshape(L.rows, H)[used], wq[used])
        assert np.array_equal(got["sc"].reshape(L.rows, -1)[used], ws[used])
    else:
        want = oracle.dispatch(x, L.dst, L.rows)
        assert np.array_equal(got["recv"].view(np.uint16).reshape(L.rows, H)[used], want[used])
    _, widx, ww = oracle.recv_meta(idx, w, L.dst, L.rows)
    assert np.array_equal(got["ri"], widx)
    assert np.array_equal(got["rw"], ww)
    _, two = _run(g, T, H, idx, w, x, False, fp8)
    for key in got:
        assert np.array_equal(got[key], two[key]), key


def test_plan_dispatch_then_combine_and_backward():
    # the handle planned by the fused call serves combine and its backward
    T, H, E, k, kind, cap, R, S, idx, w, x = _inputs(CASES[0])
    g = make_group(E, R, H, k, T, kind, cap, S)
    buf = ep.Buffer(g)
    recv, _, _, h, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), dev_f32(w))   # plans as it dispatches
    y = buf.combine(recv, h, dev_f32(w))
    torch.cuda.synchronize()
    L = oracle.layout(idx, E, kind, cap=cap)
    check_layout(h, L, kind, idx, w)
    ref = oracle.combine(oracle.dispatch(x, L.dst, L.rows), L.dst, w)
    from tests.helpers import bf16_bits_to_f32, rel_err
    assert rel_err(bf16_bits_to_f32(host_bits(y)), bf16_bits_to_f32(ref)) <= 2e-3
