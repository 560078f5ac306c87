"""GPU test of ep_handle_create_static, the entry point for callers that
cannot allocate device memory: a handle whose workspace is the library's
static device scratch must give exactly what a handle over a caller-owned
workspace (ep_handle_create) gives, and what the oracle gives, on two calls
in a row, the second with a smaller batch (the scratch keeps the first
call's contents)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, host_bits, make_group
from tests.helpers import bf16_bits_to_f32, rel_err

pytestmark = pytest.mark.gpu

SENT = 0x7F7F   # rows no entry maps to keep this pattern

# (layout, E, R, H, k, cap, S, T first, T second)
CASES = [
    ("ht", 64, 8, 512, 8, 0, 0, 3000, 700),          # 12 resident tiles, then 3
    ("static", 64, 8, 256, 4, 0, 8, 5000, 300),      # 10 resident tiles, then one
    ("ll", 32, 4, 256, 2, 160, 0, 1500, 100),        # 2 tiles, then one; capacity drops
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def chain(hptr, rows, H, x, idx, w, gy):
    """plan -> dispatch (with per-row expert and weight) -> combine -> combine
    backward on one handle; every output buffer starts from a sentinel."""
    T, k = idx.shape
    recv = torch.full((rows, H), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ri = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    rw = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    gout = torch.full((rows, H), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    gw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ep.ep_plan(hptr, idx)
    ep.ep_dispatch(hptr, x, w, recv, None, ri, rw)
    ep.ep_combine(hptr, recv, w, y)
    ep.ep_combine_bwd(hptr, gy, recv, w, gout, gw)
    torch.cuda.synchronize()
    return {"recv": host_bits(recv), "ri": host(ri), "rw": host(rw), "y": host_bits(y),
            "gout": host_bits(gout), "gw": host(gw), "status": ep.ep_handle_status(hptr)}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_static_scratch_handle_matches_workspace_handle(case):
    kind, E, R, H, k, cap, S, T1, T2 = case
    g = make_group(E, R, H, k, T1, kind, cap, S)
    for call, T in enumerate((T1, T2)):
        print(f"[no-alloc] {kind} call {call} T={T}", flush=True)
        idx_np, w_np, x_np = workloads.random_case(700 + 10 * call + len(kind), T, H, E, k,
                                                   skew=1.5 if call == 0 else 0.0)
        gy_np = workloads.f32_to_bf16_bits(
            np.random.default_rng(800 + call).standard_normal((T, H)).astype(np.float32))
        idx, w, x, gy = dev_i32(idx_np), dev_f32(w_np), dev_bf16(x_np), dev_bf16(gy_np)
        rows = g.recv_rows(T)
        ref_h = ep.Handle(g, T)
        want = chain(ref_h.ptr, rows, H, x, idx, w, gy)
        sh = ep.ep_handle_create_static(g.ptr, T)
        got = chain(sh, rows, H, x, idx, w, gy)
        for key in want:
            assert np.array_equal(np.asarray(got[key]), np.asarray(want[key])), (call, key)
        # and the oracle's layout and rows
        L = oracle.layout(idx_np, E, kind, cap=cap, R=R, S=S)
        assert got["status"] == L.flags
        used = L.dst[L.dst >= 0]
        recv = got["recv"].reshape(rows, H)
        assert np.array_equal(recv[used], oracle.dispatch(x_np, L.dst, L.rows)[used])
        flat = np.flatnonzero(L.dst.ravel() >= 0)
        assert np.array_equal(got["ri"][L.dst.ravel()[flat]], idx_np.ravel()[flat])
        ref_y = oracle.combine(oracle.dispatch(x_np, L.dst, L.rows), L.dst, w_np)
        assert rel_err(bf16_bits_to_f32(got["y"]).astype(np.float64),
                       bf16_bits_to_f32(ref_y).astype(np.float64)) <= 2e-3
        ep.ep_handle_destroy(sh)   # static storage: does nothing


def test_static_scratch_rejects_a_batch_beyond_the_scratch():
    # E = 1024, k = 16 at T = 65536: T*k = 2^20 entries need more than 16 MiB
    g = ep.Group(1024, 1, 8, 16, 65536, "ht")
    need = g.workspace_bytes(65536)
    assert need > (16 << 20)
    with pytest.raises(ep.EpError) as ex:
        ep.ep_handle_create_static(g.ptr, 65536)
    assert ex.value.code == 6   # EP_ERR_WORKSPACE_TOO_SMALL
