"""GPU checks of prepared calls (combine_ep_plan_amd.prepare): the library's C
calls recorded once with their marshalled arguments and replayed.  A replay
makes the same C calls on the same buffers, so it must give bit for bit what
the plain calls give, and it must follow new data written in place into the
same tensors (the pointers are what was recorded)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_i32, host, host_bits, make_group

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


# name, T, H, E, k, layout, cap, R, S
CASES = [
    ("decode_ll", 128, 1024, 256, 8, "ll", 128, 32, 0),   # layout + dispatch in one launch
    ("ht_three_tiles", 700, 256, 64, 8, "ht", 0, 8, 0),   # layout, then dispatch
    ("static", 400, 128, 32, 4, "static", 0, 8, 4),       # planner tables
]


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_prepared_chain_matches_plain_calls_and_follows_new_data(c):
    name, T, H, E, k, kind, cap, R, S = c
    print(f"[prepared] {name}", flush=True)
    g = make_group(E, R, H, k, T, kind, cap, S)
    h = ep.Handle(g, T)
    idx1, w1, x1 = workloads.random_case(4100, T, H, E, k, skew=1.0)
    idx2, w2, x2 = workloads.random_case(4101, T, H, E, k, skew=0.5)
    idx, w = dev_i32(idx1), torch.from_numpy(w1).cuda()
    x = dev_bf16(x1)
    recv = torch.empty(g.recv_shape(T), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream()

    def chain():
        ep.ep_plan_dispatch(h.ptr, idx, x, None, recv, None, None, None, s)
        ep.ep_combine(h.ptr, recv, w, y, s)

    chain()   # plain calls
    torch.cuda.synchronize()
    recv_plain, y_plain = host_bits(recv).copy(), host_bits(y).copy()
    recv.zero_()
    y.zero_()
    p = ep.prepare(chain)
    assert p.names == ("ep_plan_dispatch", "ep_combine")
    p()
    p()   # twice: the handshake words of the layout carry no state between calls
    torch.cuda.synchronize()
    assert h.status() == 0
    # receive rows no entry uses (LL capacity rows) are never written: the
    # plain run left whatever the allocation held there, so compare used rows
    L1 = oracle.layout(idx1, E, kind, cap=cap, R=R, S=S)
    used1 = L1.dst[L1.dst >= 0]
    assert np.array_equal(host_bits(recv).reshape(L1.rows, H)[used1], recv_plain.reshape(L1.rows, H)[used1])
    assert np.array_equal(host_bits(y), y_plain)
    # a new batch written in place into the same tensors
    idx.copy_(dev_i32(idx2))
    w.copy_(torch.from_numpy(w2).cuda())
    x.copy_(dev_bf16(x2))
    p()
    torch.cuda.synchronize()
    L = oracle.layout(idx2, E, kind, cap=cap, R=R, S=S)
    tb = {key: host(v) for key, v in h.tables().items() if v is not None}
    assert np.array_equal(tb["dst"].reshape(L.dst.shape), L.dst)
    want_recv = oracle.dispatch(x2, L.dst, L.rows)
    used = L.dst[L.dst >= 0]
    assert np.array_equal(host_bits(recv).reshape(L.rows, H)[used], want_recv[used])
    want_y = oracle.combine(want_recv, L.dst, w2)
    got = host_bits(y)
    diff = np.abs(oracle.bf16_to_f32_array(got).astype(np.float64) -
                  oracle.bf16_to_f32_array(want_y).astype(np.float64))
    ulp = np.abs(oracle.bf16_to_f32_array(want_y).astype(np.float64)) * 2.0 ** -7 + 1e-30
    assert np.all(diff <= ulp)
