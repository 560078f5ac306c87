"""GPU parity of every step of the path against the CPU oracle, at sizes the
oracle finishes in seconds that still span several layout tiles (2048
entries each) and a ragged tail, plus edge cases: empty batch, single entry,
masked / out-of-range / duplicate expert ids, LL capacity overflow, replica
slot overflow, k outside the specialised set, the largest E.

Bars: layout, plan, dispatched rows, FP8 codes and scales, combine-backward
rows and the duplicated-expert reduce are bit-exact; combine, dispatch
backward and grad_w agree within a norm-wise relative error of 2e-3 (and
elementwise within one bf16 rounding of the exact value plus fp32
accumulation slack).  All calls go through the C ABI."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import (check_layout, dev_bf16, dev_f32, dev_i32, host, host_bits,
                            make_group, same_up_to_zero_sign_np)
from tests.helpers import bf16_bits_to_f32, rel_err

pytestmark = pytest.mark.gpu

COMBINE_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()   # raises if the HIP library has not been built
    oracle.build(force=False)


# name, T, H, E, k, layout, cap, R, S, mask, bad, dup, skew, seed
CASES = [
    ("tiny_ll", 64, 256, 8, 2, "ll", 64, 4, 2, 0.0, 0.0, 0.0, 0.0, 1),
    ("ragged_ht", 1000, 136, 37, 8, "ht", 0, 1, 0, 0.0, 0.0, 0.0, 0.8, 2),
    ("ll_overflow", 1000, 64, 37, 8, "ll", 150, 1, 0, 0.0, 0.0, 0.0, 1.5, 3),
    ("masked_bad_k6", 777, 200, 100, 6, "ht", 0, 4, 0, 0.1, 0.02, 0.0, 0.0, 4),
    ("dup_k4", 300, 64, 16, 4, "ht", 0, 2, 0, 0.0, 0.0, 0.3, 0.0, 5),
    ("static_skew", 2000, 128, 64, 8, "static", 0, 8, 8, 0.0, 0.0, 0.0, 1.0, 6),
    ("static_slot_budget", 999, 96, 12, 3, "static", 0, 4, 1, 0.05, 0.0, 0.0, 2.0, 7),
    ("static_masked_k16", 400, 64, 1024, 16, "static", 0, 1024, 1, 0.1, 0.0, 0.0, 1.2, 8),
    ("ht_k16_e1024", 300, 64, 1024, 16, "ht", 0, 1, 0, 0.0, 0.0, 0.0, 0.0, 9),
    ("empty", 0, 64, 8, 2, "ht", 0, 2, 0, 0.0, 0.0, 0.0, 0.0, 10),
    ("empty_static", 0, 64, 8, 2, "static", 0, 2, 2, 0.0, 0.0, 0.0, 0.0, 11),
    ("single", 1, 8, 1, 1, "ht", 0, 1, 0, 0.0, 0.0, 0.0, 0.0, 12),
    ("k1_ll", 513, 24, 5, 1, "ll", 200, 5, 0, 0.0, 0.0, 0.0, 0.5, 13),
    ("exact_tile", 512, 32, 256, 8, "static", 0, 32, 8, 0.0, 0.0, 0.0, 1.1, 14),
    ("one_full_tile", 256, 40, 64, 8, "ht", 0, 8, 0, 0.0, 0.0, 0.0, 1.0, 15),
    ("ll_multi_tile_masked", 700, 48, 96, 8, "ll", 90, 8, 0, 0.08, 0.01, 0.0, 1.3, 16),
    # 274 layout tiles: the finishing workgroup scans hundreds of tile histograms
    ("many_tiles_ht", 70000, 8, 64, 8, "ht", 0, 8, 0, 0.02, 0.0, 0.0, 1.0, 17),
    ("many_tiles_static", 70000, 8, 64, 8, "static", 0, 8, 4, 0.0, 0.0, 0.0, 1.5, 18),
]


def _case(c):
    name, T, H, E, k, kind, cap, R, S, mask, bad, dup, skew, seed = c
    idx, w, x = workloads.random_case(1000 + seed, T, H, E, k, mask_frac=mask, bad_frac=bad,
                                      dup_frac=dup, skew=skew)
    return dict(name=name, T=T, H=H, E=E, k=k, kind=kind, cap=cap, R=R, S=S, idx=idx, w=w, x=x)


def _setup(c):
    g = make_group(c["E"], c["R"], c["H"], c["k"], c["T"], c["kind"], c["cap"], c["S"])
    h = ep.Handle(g, c["T"])
    L = oracle.layout(c["idx"], c["E"], c["kind"], cap=c["cap"], R=c["R"], S=c["S"])
    return g, h, L


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_layout_and_plan(c):
    c = _case(c)
    g, h, L = _setup(c)
    idx = dev_i32(c["idx"])
    h.plan(idx)
    check_layout(h, L, c["kind"], c["idx"], c["w"])
    # re-planning the same handle gives the same tables (ticket and status reset)
    h.plan(idx)
    check_layout(h, L, c["kind"], c["idx"], c["w"])


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_dispatch_combine(c):
    c = _case(c)
    g, h, L = _setup(c)
    T, H, k = c["T"], c["H"], c["k"]
    buf = ep.Buffer(g)
    x = dev_bf16(c["x"])
    w = dev_f32(c["w"])
    h.plan(dev_i32(c["idx"]))
    recv, ri, rw, _, _ = buf.dispatch(x, dev_i32(c["idx"]), w, handle=h)
    torch.cuda.synchronize()
    want = oracle.dispatch(c["x"], L.dst, L.rows)
    used = L.dst[L.dst >= 0]
    got = host_bits(recv).reshape(L.rows, H)
    assert np.array_equal(got[used], want[used])
    src, widx, ww = oracle.recv_meta(c["idx"], c["w"], L.dst, L.rows)
    assert np.array_equal(host(ri), widx)
    assert np.array_equal(host(rw), ww)

    # combine of arbitrary expert outputs (not the dispatched rows)
    rng = np.random.default_rng(c["T"] + 17)
    eo_bits = workloads.f32_to_bf16_bits(rng.standard_normal((L.rows, H)).astype(np.float32))
    eo = dev_bf16(eo_bits).view(recv.shape)
    for out_fp32 in (False, True):
        y = buf.combine(eo, h, w, out_dtype=torch.float32 if out_fp32 else torch.bfloat16)
        ref = oracle.combine(eo_bits, L.dst, c["w"], out_fp32=out_fp32)
        gy = host(y) if out_fp32 else bf16_bits_to_f32(host_bits(y))
        rf = ref if out_fp32 else bf16_bits_to_f32(ref)
        assert rel_err(gy, rf) <= COMBINE_TOL
        # elementwise: within one bf16 ulp of the oracle's (rounded) value
        scale = np.abs(bf16_bits_to_f32(eo_bits)).max(initial=0.0) * k
        assert np.all(np.abs(gy - rf) <= np.abs(rf) * 2.0 ** -7 + scale * 2.0 ** -20 + 1e-30)
    # dispatch backward = unit-weight combine
    gx = buf.dispatch_bwd(eo, h)
    ref = oracle.combine(eo_bits, L.dst, None)
    assert rel_err(bf16_bits_to_f32(host_bits(gx)), bf16_bits_to_f32(ref)) <= COMBINE_TOL


@pytest.mark.parametrize("c", [c for c in CASES if c[2] % 128 == 0],
                         ids=lambda c: c[0])
def test_dispatch_fp8(c):
    c = _case(c)
    g, h, L = _setup(c)
    buf = ep.Buffer(g)
    h.plan(dev_i32(c["idx"]))
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(c["x"]), dev_i32(c["idx"]), None, handle=h,
                                      fp8=True, recv_meta=False)
    torch.cuda.synchronize()
    wq, ws = oracle.dispatch_fp8(c["x"], L.dst, L.rows)
    used = L.dst[L.dst >= 0]
    gq = q.view(torch.uint8).cpu().numpy().reshape(L.rows, c["H"])
    assert np.array_equal(gq[used], wq[used])
    assert np.array_equal(host(s)[used], ws[used])


def test_fp8_encoder_all_bf16_patterns():
    """Every finite bf16 value, quantised in blocks whose amax is 448 (scale
    exactly 1): the GPU's codes equal the oracle's for all 65 536 patterns."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(pats)
    pats = pats[np.isfinite(f) & (np.abs(f) <= 448)]
    per = 127
    nblk = -(-pats.size // per)
    H = 128 * 8
    T = -(-nblk // 8)
    x = np.zeros((T * 8, 128), np.uint16)
    x[:, 0] = workloads.f32_to_bf16_bits(np.float32([448.0]))[0]
    flat = np.zeros(T * 8 * per, np.uint16)
    flat[: pats.size] = pats
    x[:, 1:] = flat.reshape(T * 8, per)
    x = x.reshape(T, H)
    idx = np.zeros((T, 1), np.int32)
    L = oracle.layout(idx, 1, "ht")
    g = make_group(1, 1, H, 1, T, "ht")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    buf = ep.Buffer(g)
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True,
                                      recv_meta=False)
    wq, ws = oracle.dispatch_fp8(x, L.dst, L.rows)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy().reshape(wq.shape), wq)
    assert np.all(host(s) == 1.0) and np.all(ws == 1.0)


@pytest.mark.parametrize("c", [c for c in CASES if c[0] in
                               ("tiny_ll", "ragged_ht", "masked_bad_k6", "static_skew", "dup_k4",
                                "static_masked_k16", "empty", "single")],
                         ids=lambda c: c[0])
def test_combine_bwd(c):
    c = _case(c)
    g, h, L = _setup(c)
    T, H = c["T"], c["H"]
    buf = ep.Buffer(g)
    h.plan(dev_i32(c["idx"]))
    rng = np.random.default_rng(T + 5)
    eo_bits = workloads.f32_to_bf16_bits(rng.standard_normal((L.rows, H)).astype(np.float32))
    gy_bits = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    eo = dev_bf16(eo_bits)
    gout, gw = buf.combine_bwd(dev_bf16(gy_bits), eo, dev_f32(c["w"]), h)
    torch.cuda.synchronize()
    rgo, rgw = oracle.combine_bwd(gy_bits, eo_bits, L.dst, c["w"])
    used = L.dst[L.dst >= 0]
    assert np.array_equal(host_bits(gout)[used], rgo[used])
    assert rel_err(host(gw), rgw) <= COMBINE_TOL
    assert np.all(host(gw)[L.dst < 0] == 0)


@pytest.mark.parametrize("P", [4096, 1000, 8, 13, 8200, 4100])
def test_dup_reduce(P):
    rng = np.random.default_rng(P)
    E = 6
    owner = rng.standard_normal((E, P)).astype(np.float32)
    rep_e = np.array([4, 1, 4, -1, 1, 4, 0], np.int32)
    rep = workloads.f32_to_bf16_bits(rng.standard_normal((rep_e.size, P)).astype(np.float32))
    g = make_group(8, 2, 64, 2, 4, "ht")
    h = ep.Handle(g, 4)
    own = dev_f32(owner)
    ep.ep_dup_grad_reduce(h.ptr, dev_bf16(rep), dev_i32(rep_e), own)
    want = oracle.dup_reduce(rep, rep_e, owner)
    assert np.array_equal(host(own), want)
    assert h.status() == 0


def test_dup_reduce_index_range_flag():
    g = make_group(8, 2, 64, 2, 4, "ht")
    h = ep.Handle(g, 4)
    owner = np.ones((3, 64), np.float32)
    rep = workloads.f32_to_bf16_bits(np.ones((2, 64), np.float32))
    own = dev_f32(owner)
    ep.ep_dup_grad_reduce(h.ptr, dev_bf16(rep), dev_i32(np.array([2, 7], np.int32)), own)
    assert h.status() & ep.FLAG_INDEX_RANGE
    assert np.array_equal(host(own), oracle.dup_reduce(rep[:1], np.array([2], np.int32), owner))


def test_dup_reduce_from_plan_table():
    c = _case(CASES[5])   # static_skew: replicas exist
    g, h, L = _setup(c)
    h.plan(dev_i32(c["idx"]))
    R, S = c["R"], c["S"]
    P = 512
    rng = np.random.default_rng(3)
    rep = workloads.f32_to_bf16_bits(rng.standard_normal((R * S, P)).astype(np.float32))
    owner = rng.standard_normal((c["E"], P)).astype(np.float32)
    own = dev_f32(owner)
    ep.ep_dup_grad_reduce(h.ptr, dev_bf16(rep), None, own)
    want = oracle.dup_reduce(rep, L.plan.replica.reshape(-1), owner)
    assert (L.plan.replica >= 0).any()
    assert np.array_equal(host(own), want)


def test_deterministic_repeat():
    c = _case(CASES[5])
    g, h, L = _setup(c)
    buf = ep.Buffer(g)
    x, idx, w = dev_bf16(c["x"]), dev_i32(c["idx"]), dev_f32(c["w"])
    outs = []
    for _ in range(2):
        h.plan(idx)
        recv, ri, rw, _, _ = buf.dispatch(x, idx, w, handle=h)
        y = buf.combine(recv, h, w)
        torch.cuda.synchronize()
        outs.append((host(h.tables()["dst"]).copy(), host_bits(recv).copy(), host_bits(y).copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_identity_experts_roundtrip_small():
    c = _case(CASES[1])
    g, h, L = _setup(c)
    buf = ep.Buffer(g)
    x = dev_bf16(c["x"])
    h.plan(dev_i32(c["idx"]))
    recv, _, _, _, _ = buf.dispatch(x, dev_i32(c["idx"]), dev_f32(c["w"]), handle=h)
    y = buf.combine(recv, h, dev_f32(c["w"]))
    assert same_up_to_zero_sign_np(host_bits(y), c["x"])


def test_deterministic_on_two_streams():
    # the whole chain on two streams at once, each with its own handle: every
    # output bit-identical (no atomics order any result)
    c = _case(CASES[5])
    g = make_group(c["E"], c["R"], c["H"], c["k"], c["T"], c["kind"], c["cap"], c["S"])
    buf = ep.Buffer(g)
    x, idx, w = dev_bf16(c["x"]), dev_i32(c["idx"]), dev_f32(c["w"])
    gy = dev_bf16(workloads.f32_to_bf16_bits(
        np.random.default_rng(3).standard_normal((c["T"], c["H"])).astype(np.float32)))
    torch.cuda.synchronize()
    outs = []
    for st in (torch.cuda.Stream(), torch.cuda.Stream()):
        with torch.cuda.stream(st):
            h = ep.Handle(g, c["T"])
            h.plan(idx, st)
            recv, _, _, _, _ = buf.dispatch(x, idx, w, handle=h, recv_meta=False, stream=st)
            y = buf.combine(recv, h, w, stream=st)
            gout, gw = buf.combine_bwd(gy, recv, w, h, stream=st)
            gx = buf.dispatch_bwd(gout, h, stream=st)
            outs.append((h, recv, y, gout, gw, gx))
    torch.cuda.synchronize()
    a, b = outs
    assert np.array_equal(host(a[0].tables()["dst"]), host(b[0].tables()["dst"]))
    for u, v in zip(a[1:], b[1:]):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_hip_graph_replays_match_eager():
    # plan -> dispatch -> combine captured once as a HIP graph; new routing and
    # tokens are copied into the captured buffers before each replay, with
    # eager work in between, and every replay must equal the eager calls
    name, T, H, E, k, kind, cap, R, S = CASES[5][:9]   # static, 8 layout tiles
    g = make_group(E, R, H, k, T, kind, cap, S)
    buf = ep.Buffer(g)
    h = ep.Handle(g, T)
    idx0, w0, x0 = workloads.random_case(5000, T, H, E, k, skew=1.0)
    idx, w, x = dev_i32(idx0), dev_f32(w0), dev_bf16(x0)
    recv = torch.empty(g.recv_shape(T), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def chain(hh, rv, yy, st):
        ep.ep_plan(hh.ptr, idx, st)
        ep.ep_dispatch(hh.ptr, x, None, rv, None, None, None, st)
        ep.ep_combine(hh.ptr, rv, w, yy, st)

    chain(h, recv, y, None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(h, recv, y, torch.cuda.current_stream())
    torch.cuda.synchronize()
    h_ref = ep.Handle(g, T)
    recv_ref, y_ref = torch.empty_like(recv), torch.empty_like(y)
    for seed in range(3):
        i1, w1, x1 = workloads.random_case(5001 + seed, T, H, E, k, skew=0.5 + seed)
        idx.copy_(dev_i32(i1))
        w.copy_(dev_f32(w1))
        x.copy_(dev_bf16(x1))
        graph.replay()
        torch.cuda.synchronize()
        got = (host(h.tables()["dst"]).copy(), host_bits(recv).copy(), host_bits(y).copy())
        _ = torch.ones(1 << 20, device="cuda").sum()          # eager work between replays
        chain(h_ref, recv_ref, y_ref, None)
        torch.cuda.synchronize()
        L = oracle.layout(i1, E, kind, cap=cap, R=R, S=S)
        assert np.array_equal(got[0], L.dst)
        assert np.array_equal(host(h_ref.tables()["dst"]), L.dst)
        used = L.dst[L.dst >= 0]
        assert np.array_equal(got[1].reshape(L.rows, H)[used], host_bits(recv_ref).reshape(L.rows, H)[used])
        assert np.array_equal(got[2], host_bits(y_ref))
        assert h.status() == 0


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_dispatch_store_kinds_give_identical_rows(fp8):
    # the group's dispatch_stores choice changes only how rows are written:
    # cached, non-temporal and the size-chosen default give the same bytes
    T, H, E, k = 700, 512, 32, 4
    idx, w, x = workloads.random_case(4242, T, H, E, k, skew=1.0)
    L = oracle.layout(idx, E, "ht")
    used = L.dst[L.dst >= 0]
    outs = []
    for stores in ("auto", "cached", "streaming"):
        g = ep.Group(E, 4, H, k, T, "ht", dispatch_stores=stores)
        h = ep.Handle(g, T)
        h.plan(dev_i32(idx))
        recv, _, _, _, _ = ep.Buffer(g).dispatch(dev_bf16(x), None, None, handle=h, fp8=fp8, recv_meta=False)
        torch.cuda.synchronize()
        if fp8:
            q, s = recv
            outs.append((q.view(torch.uint8).cpu().numpy().reshape(L.rows, H)[used], host(s)[used]))
        else:
            outs.append((host_bits(recv).reshape(L.rows, H)[used],))
    if fp8:
        oq, osc = oracle.dispatch_fp8(x, L.dst, L.rows)
        want = (oq[used], osc[used])
    else:
        want = (oracle.dispatch(x, L.dst, L.rows)[used],)
    for o in outs:
        for a, b in zip(o, want):
            assert np.array_equal(a, b)


def test_combine_store_kinds_give_identical_rows():
    # the group's combine_stores choice changes only how the token rows are
    # written: weighted (bf16 and fp32 out) and unit-weight combines give the
    # same bytes with cached, non-temporal and default stores
    T, H, E, k = 700, 512, 32, 4
    idx, w, _ = workloads.random_case(4343, T, H, E, k, skew=1.0)
    L = oracle.layout(idx, E, "ht")
    rng = np.random.default_rng(4343)
    eo_bits = workloads.f32_to_bf16_bits(rng.standard_normal((L.rows, H)).astype(np.float32))
    outs = []
    for stores in ("auto", "cached", "streaming"):
        g = ep.Group(E, 4, H, k, T, "ht", combine_stores=stores)
        h = ep.Handle(g, T)
        h.plan(dev_i32(idx))
        buf = ep.Buffer(g)
        eo = dev_bf16(eo_bits)
        y16 = buf.combine(eo, h, dev_f32(w))
        y32 = buf.combine(eo, h, dev_f32(w), out_dtype=torch.float32)
        gx = buf.dispatch_bwd(eo, h)
        torch.cuda.synchronize()
        outs.append((host_bits(y16), host(y32).view(np.uint32), host_bits(gx)))
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert np.array_equal(a, b)
    ref = oracle.combine(eo_bits, L.dst, w, out_fp32=True)
    assert rel_err(outs[0][1].view(np.float32), ref) <= COMBINE_TOL
    ref = oracle.combine(eo_bits, L.dst, None)
    assert rel_err(bf16_bits_to_f32(outs[0][2]), bf16_bits_to_f32(ref)) <= COMBINE_TOL
