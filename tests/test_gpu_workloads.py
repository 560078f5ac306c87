"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (same library calls, same shapes).

Layout and plan tables are compared with the oracle in full.  Dispatched
rows are checked in full on the device against the gather that defines them
(row dst[t*k+j] holds x[t]) once dst is proven equal to the oracle's, and on
sampled tokens against the oracle's own dispatch.  Combine, its backward and
the dispatch backward are compared with the oracle on sampled tokens (the
oracle recomputes those tokens from the gathered rows), and in full through
closed forms that hold at any size: with identity experts and weights summing
to 1, combine(dispatch(x)) == x bit for bit up to the sign of zero (the sum
starts from +0, so a -0 input comes back as +0, in the oracle as on the GPU),
and every copy of a token gets the same grad_w."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import (check_layout, dev_bf16, dev_f32, dev_i32, host, host_bits,
                            make_group, same_up_to_zero_sign, same_up_to_zero_sign_np,
                            sample_problem)
from tests.helpers import bf16_bits_to_f32, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def _run_forward(inp, kind_override=None, cap=None, S=None):
    c = inp.cfg
    kind = kind_override or c.layout
    cap = c.cap if cap is None else cap
    S = c.S if S is None else S
    print(f"[workload] {c.name} rho={c.rho} T={c.T} H={c.H} E={c.E} k={c.k} layout={kind}", flush=True)
    g = make_group(c.E, c.R, c.H, c.k, c.T, kind, cap, S)
    h = ep.Handle(g, c.T)
    buf = ep.Buffer(g)
    x = dev_bf16(inp.x)
    idx = dev_i32(inp.topk_idx)
    w = dev_f32(inp.topk_w)
    h.plan(idx)
    recv, ri, rw, _, _ = buf.dispatch(x, idx, w, handle=h, recv_meta=False)
    L = oracle.layout(inp.topk_idx, c.E, kind, cap=cap, R=c.R, S=S)
    return g, h, buf, x, idx, w, recv, L


def _check_dispatch_full(inp, recv, L, x):
    c = inp.cfg
    d = L.dst.reshape(-1)
    f = np.nonzero(d >= 0)[0]
    rows = recv.view(L.rows, c.H).view(torch.int16)
    got = rows.index_select(0, torch.from_numpy(d[f].astype(np.int64)).cuda())
    want = x.view(torch.int16).index_select(0, torch.from_numpy(f // c.k).cuda())
    assert torch.equal(got, want)
    # sampled tokens against the oracle's own dispatch
    rng = np.random.default_rng(c.T)
    toks = np.sort(rng.choice(c.T, size=min(c.T, 64), replace=False))
    sub_dst = L.dst[toks]
    for t_i, t in enumerate(toks):
        for j in range(c.k):
            if sub_dst[t_i, j] >= 0:
                row = host_bits(recv.view(L.rows, c.H)[int(sub_dst[t_i, j])])
                ref = oracle.dispatch(inp.x[t:t + 1], sub_dst[t_i:t_i + 1, j:j + 1] * 0, 1)
                assert np.array_equal(row, ref[0])


def _check_combine_sampled(inp, L, rows, y, w_np, n=512, out_fp32=False):
    c = inp.cfg
    rng = np.random.default_rng(c.T + 1)
    toks = np.sort(rng.choice(c.T, size=min(c.T, n), replace=False))
    local, gb, _ = sample_problem(L.dst, toks, rows.view(L.rows, c.H))
    ref = oracle.combine(gb, local, None if w_np is None else w_np[toks], out_fp32=out_fp32)
    if out_fp32:
        got = host(y)[toks]
        assert rel_err(got, ref) <= TOL
    else:
        got = bf16_bits_to_f32(host_bits(y)[toks])
        assert rel_err(got, bf16_bits_to_f32(ref)) <= TOL


def test_tiny_ll_and_planner():
    inp = workloads.make_inputs("tiny")
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, "ll", inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w, out_dtype=torch.float32)
    local, gb, _ = sample_problem(L.dst, np.arange(c.T), recv.view(L.rows, c.H))
    ref = oracle.combine(gb, local, inp.topk_w, out_fp32=True)
    assert rel_err(host(y), ref) <= TOL
    # the static planner on the same routing (4 ranks x 2 experts, 2 slots)
    g2, h2, buf2, _, _, _, recv2, L2 = _run_forward(inp, kind_override="static")
    check_layout(h2, L2, "static", inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv2, L2, x)
    y2 = buf2.combine(recv2, h2, w)
    assert same_up_to_zero_sign_np(host_bits(y2), inp.x)


def test_decode_ll_bf16_and_fp8():
    inp = workloads.make_inputs("decode")
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, "ll", inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w)
    _check_combine_sampled(inp, L, recv, y, inp.topk_w, n=c.T)
    assert same_up_to_zero_sign_np(host_bits(y), inp.x)
    (q, s), _, _, _, _ = buf.dispatch(x, idx, None, handle=h, fp8=True, recv_meta=False)
    torch.cuda.synchronize()
    wq, wsc = oracle.dispatch_fp8(inp.x, L.dst, L.rows)
    used = L.dst[L.dst >= 0]
    gq = q.view(torch.uint8).view(L.rows, c.H)[torch.from_numpy(used.astype(np.int64)).cuda()]
    assert np.array_equal(gq.cpu().numpy(), wq[used])
    assert np.array_equal(host(s)[used], wsc[used])
    # dequantised rows within 1e-2 of the oracle's dequantised rows (expected: exact)
    deq = lambda qq, ss: (torch.from_numpy(qq).view(torch.float8_e4m3fn).float().numpy()
                          .reshape(-1, 128) * ss.reshape(-1, 1))
    assert rel_err(deq(gq.cpu().numpy(), host(s)[used]), deq(wq[used], wsc[used])) <= 1e-2


def test_prefill_ht():
    inp = workloads.make_inputs("prefill")
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, "ht", inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w)
    _check_combine_sampled(inp, L, recv, y, inp.topk_w, n=1024)
    assert same_up_to_zero_sign_np(host_bits(y), inp.x)   # identity experts, weights sum to 1
    # the oracle makes the same choice for the sign of zero
    neg0 = np.argwhere(inp.x == 0x8000)
    if len(neg0):
        t = int(neg0[0][0])
        local, gb, _ = sample_problem(L.dst, np.array([t]), recv.view(L.rows, c.H))
        ref = oracle.combine(gb, local, inp.topk_w[t:t + 1])
        assert np.array_equal(host_bits(y)[t], ref[0])


@pytest.mark.parametrize("rho", workloads.SWEEP_RHOS)
def test_sweep_static(rho):
    inp = workloads.make_inputs("sweep", rho=rho)
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, "static", inp.topk_idx, inp.topk_w)
    assert L.flags == 0
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w)
    _check_combine_sampled(inp, L, recv, y, inp.topk_w)
    assert same_up_to_zero_sign(y, x)


def test_training_fwd_bwd_and_dup_reduce():
    inp = workloads.make_inputs("training")
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, "static", inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w)
    assert same_up_to_zero_sign(y, x)
    # backward: combine_bwd with identity experts, then dispatch_bwd
    gy_bits = workloads.make_grad(c, 0, (c.T, c.H), 1)
    gy = dev_bf16(gy_bits)
    gout, gw = buf.combine_bwd(gy, recv, w, h)
    gx = buf.dispatch_bwd(gout, h)
    torch.cuda.synchronize()
    gwh = host(gw)
    assert np.all(gwh == gwh[:, :1])          # same dot product for every copy
    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(c.T, size=512, replace=False))
    local, gb, used = sample_problem(L.dst, toks, recv.view(L.rows, c.H))
    rgo, rgw = oracle.combine_bwd(gy_bits[toks], gb, local, inp.topk_w[toks], rows=gb.shape[0])
    got_rows = host_bits(gout.view(L.rows, c.H).index_select(0, torch.from_numpy(used).cuda()))
    assert np.array_equal(got_rows, rgo)
    assert rel_err(gwh[toks], rgw) <= TOL
    # dispatch backward of the sampled tokens, from the gathered grad rows
    ref_gx = oracle.combine(got_rows, local, None)
    assert rel_err(bf16_bits_to_f32(host_bits(gx)[toks]), bf16_bits_to_f32(ref_gx)) <= TOL
    # duplicated-expert reduce: 2 bf16 replicas of the hottest expert's [4096, 1536]
    # weight gradient folded into its fp32 owner slot
    hot = int(np.argmax(L.counts))
    rep_bits = workloads.make_grad(c, 0, (2, 4096, 1536), 2)
    owner_hot = workloads.make_owner(c, 0, (1, 4096, 1536))
    owner = torch.zeros((c.E, 4096, 1536), dtype=torch.float32, device="cuda")
    owner[hot] = dev_f32(owner_hot[0])
    ep.ep_dup_grad_reduce(h.ptr, dev_bf16(rep_bits), dev_i32(np.array([hot, hot], np.int32)), owner)
    want = oracle.dup_reduce(rep_bits.reshape(2, -1), np.array([0, 0], np.int32),
                             owner_hot.reshape(1, -1))
    assert np.array_equal(host(owner[hot]).reshape(1, -1), want)
    assert float(owner[(hot + 1) % c.E].abs().max()) == 0.0
    assert h.status() == 0


@pytest.mark.parametrize("name,s", [(n, s) for n in ("tiny", "decode", "prefill", "sweep", "training")
                                    for s in (1, 2)])
def test_workload_other_seeds(name, s):
    # seeds 1 and 2 of every workload: layout and plan in full, dispatch in
    # full, combine on sampled tokens
    inp = workloads.make_inputs(name, s, 8.0) if name == "sweep" else workloads.make_inputs(name, s)
    c = inp.cfg
    g, h, buf, x, idx, w, recv, L = _run_forward(inp)
    check_layout(h, L, c.layout, inp.topk_idx, inp.topk_w)
    _check_dispatch_full(inp, recv, L, x)
    y = buf.combine(recv, h, w, out_dtype=torch.float32 if c.out_fp32 else torch.bfloat16)
    _check_combine_sampled(inp, L, recv, y, inp.topk_w, n=256, out_fp32=c.out_fp32)


@pytest.mark.parametrize("name", ["prefill", "training"])
def test_fp8_dispatch_at_full_sizes(name):
    # prefill writes 242 MB of codes and scales (cached stores), training 553 MB
    # (non-temporal stores): sampled tokens bit-exact against the oracle, and in
    # full on the device every copy of a token equal to its first copy
    inp = workloads.make_inputs(name)
    c = inp.cfg
    print(f"[workload fp8] {name} T={c.T} H={c.H} E={c.E} k={c.k} layout={c.layout}", flush=True)
    g = make_group(c.E, c.R, c.H, c.k, c.T, c.layout, c.cap, c.S)
    h = ep.Handle(g, c.T)
    buf = ep.Buffer(g)
    h.plan(dev_i32(inp.topk_idx))
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(inp.x), None, None, handle=h, fp8=True, recv_meta=False)
    torch.cuda.synchronize()
    L = oracle.layout(inp.topk_idx, c.E, c.layout, cap=c.cap, R=c.R, S=c.S)
    qr = q.view(torch.uint8).view(L.rows, c.H)
    sr = s.view(L.rows, c.H // 128)
    d = torch.from_numpy(L.dst.astype(np.int64)).cuda()            # [T, k]
    ok = d >= 0
    first = d[:, :1].expand_as(d)
    assert bool(ok[:, 0].all())                                       # no entry masked here
    assert torch.equal(qr[d[ok]], qr[first[ok]])
    assert torch.equal(sr[d[ok]], sr[first[ok]])
    rng = np.random.default_rng(c.T + 7)
    for t in np.sort(rng.choice(c.T, size=64, replace=False)):
        wq, ws = oracle.dispatch_fp8(inp.x[t:t + 1], np.zeros((1, 1), np.int32), 1)
        for j in range(c.k):
            r = int(L.dst[t, j])
            assert np.array_equal(qr[r].cpu().numpy(), wq[0]), (t, j)
            assert np.array_equal(sr[r].cpu().numpy(), ws[0]), (t, j)
    assert h.status() == 0
