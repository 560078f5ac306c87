"""GPU parity of several micro-batches in flight: the one-GPU form of
double-buffered dispatch/combine ([NCCL-EP] Table II and Figure 2: LL mode
overlaps the dispatch and combine phases of consecutive batches through
double buffers).  Each micro-batch has its own handle, receive and output
buffers and runs on its own stream; the launches are interleaved op by op,
so one micro-batch's plan and dispatch run beside another's combine.  Every
micro-batch must match the oracle (layout and dispatched rows bit-exact,
combine as in the parity tests) and be bit-identical to the same
micro-batches run one after another on one stream."""

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


# name, T, H, E, k, kind, cap, R, S, micro-batches, fp8
CASES = [
    ("ll_double", 96, 512, 32, 4, "ll", 40, 1, 0, 2, False),
    ("ll_triple_fp8", 96, 512, 32, 4, "ll", 40, 1, 0, 3, True),
    ("ht_double", 700, 256, 16, 8, "ht", 0, 1, 0, 2, False),
    ("static_triple", 900, 256, 32, 4, "static", 0, 8, 4, 3, False),
]


def _microbatches(c):
    name, T, H, E, k, kind, cap, R, S, M, fp8 = c
    g = make_group(E, R, H, k, T, kind, cap, S)
    mbs = []
    for i in range(M):
        idx, w, x = workloads.random_case(7000 + 17 * i + T, T, H, E, k, skew=1.0 + 0.3 * i)
        mbs.append((idx, w, x))
    return g, mbs


def _run(g, mbs, fp8, streams):
    """Launch every micro-batch's plan -> dispatch (-> FP8 dispatch) ->
    combine, op by op across the micro-batches, micro-batch i on streams[i]."""
    buf = ep.Buffer(g)
    T = mbs[0][0].shape[0]
    H = g.hidden
    state = []
    for (idx, w, x), st in zip(mbs, streams):
        h = ep.Handle(g, T)
        recv = torch.empty(g.recv_shape(T), dtype=torch.bfloat16, device="cuda")
        q = torch.empty(g.recv_shape(T), dtype=torch.float8_e4m3fn, device="cuda") if fp8 else None
        s = torch.empty((h.recv_rows, H // 128), dtype=torch.float32, device="cuda") if fp8 else None
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        state.append((h, dev_i32(idx), dev_f32(w), dev_bf16(x), recv, q, s, y, st))
    torch.cuda.synchronize()
    start = torch.cuda.Event()
    start.record(torch.cuda.current_stream())
    for *_, st in state:
        st.wait_stream(torch.cuda.current_stream())
    for h, idx, w, x, recv, q, s, y, st in state:
        ep.ep_plan(h.ptr, idx, st)
    for h, idx, w, x, recv, q, s, y, st in state:
        ep.ep_dispatch(h.ptr, x, None, recv, None, None, None, st)
    if fp8:
        for h, idx, w, x, recv, q, s, y, st in state:
            ep.ep_dispatch(h.ptr, x, None, q, s, None, None, st)
    for h, idx, w, x, recv, q, s, y, st in state:
        ep.ep_combine(h.ptr, recv, w, y, st)
    torch.cuda.synchronize()
    return state


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_microbatches_overlapped_match_oracle_and_serial(c):
    name, T, H, E, k, kind, cap, R, S, M, fp8 = c
    print(f"[overlap] {name} M={M} T={T} H={H} E={E} k={k} {kind} fp8={fp8}", flush=True)
    g, mbs = _microbatches(c)
    over = _run(g, mbs, fp8, [torch.cuda.Stream() for _ in range(M)])
    serial = _run(g, mbs, fp8, [torch.cuda.current_stream()] * M)
    for (idx, w, x), a, b in zip(mbs, over, serial):
        h, _, _, _, recv, q, s, y, _ = a
        L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S)
        assert np.array_equal(host(h.tables()["dst"]).reshape(L.dst.shape), L.dst)
        assert h.status() == L.flags
        used = L.dst[L.dst >= 0]
        want = oracle.dispatch(x, L.dst, L.rows)
        assert np.array_equal(host_bits(recv).reshape(L.rows, H)[used], want[used])
        if fp8:
            oq, osc = oracle.dispatch_fp8(x, L.dst, L.rows)
            assert np.array_equal(q.view(torch.uint8).cpu().numpy().reshape(L.rows, H)[used], oq[used])
            assert np.array_equal(host(s)[used], osc[used])
        ref = bf16_bits_to_f32(oracle.combine(want, L.dst, w)).astype(np.float64)
        got = bf16_bits_to_f32(host_bits(y)).astype(np.float64)
        assert rel_err(got, ref) <= 2e-3
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)   # one bf16 ulp
        # bit-identical to the same micro-batch run in turn on one stream
        for u, v in zip(a[4:8], b[4:8]):
            if u is None:
                continue
            uu = u.view(torch.uint8) if u.dtype == torch.float8_e4m3fn else u
            vv = v.view(torch.uint8) if v.dtype == torch.float8_e4m3fn else v
            if uu.dtype == torch.bfloat16:
                uu, vv = uu.view(torch.int16), vv.view(torch.int16)
            if u is recv or u is q or (s is not None and u is s):
                rows = torch.from_numpy(used.astype(np.int64)).cuda()
                uu, vv = uu.reshape(L.rows, -1)[rows], vv.reshape(L.rows, -1)[rows]
            assert torch.equal(uu, vv)
