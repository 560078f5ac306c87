"""GPU parity of the replica-weight prefetch and of the planner's two slot
modes (MoonEP article, paragraph 5) against the oracle, through the C ABI.

Bars: every plan table (seg_slot included) and the status flags bit-exact;
prefetched slots byte-exact, and slots the plan leaves empty untouched.
Weights are random bytes, so the copy is checked as bytes whatever the
dtype the tensor is tagged with (bf16, fp32, FP8)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import check_layout, dev_i32, host, make_group

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


# name, T, E, k, R, S, skew, seed, slot mode
PLANS = [
    ("skew_training", 2000, 64, 8, 8, 8, 1.0, 21, "training"),
    ("skew_inference_s1", 2000, 64, 8, 8, 1, 1.5, 22, "inference"),
    ("budget_training", 999, 12, 3, 4, 1, 2.0, 23, "training"),
    ("budget_inference", 999, 12, 3, 4, 1, 2.0, 23, "inference"),
    ("e1024_r1024_inference", 400, 1024, 16, 1024, 1, 1.2, 24, "inference"),
    ("no_slots_inference", 500, 16, 4, 4, 0, 2.0, 25, "inference"),
    ("empty", 0, 8, 2, 2, 2, 0.0, 26, "training"),
]
MODE = {"training": oracle.SLOTS_TRAINING, "inference": oracle.SLOTS_INFERENCE}


def _planned(c):
    name, T, E, k, R, S, skew, seed, mode = c
    idx, w, _ = workloads.random_case(2000 + seed, T, 8, E, k, skew=skew)
    g = make_group(E, R, 8, k, T, "static", 0, S, mode)
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, "static", R=R, S=S, slot_mode=MODE[mode])
    return g, h, L, idx, w


@pytest.mark.parametrize("c", PLANS, ids=[c[0] for c in PLANS])
def test_plan_slot_modes(c):
    print(f"[prefetch] plan {c[0]}", flush=True)
    g, h, L, idx, w = _planned(c)
    check_layout(h, L, "static", idx, w)
    if c[8] == "inference":
        assert L.flags & oracle.FLAG_SLOT_BUDGET == 0
    if c[0].startswith("budget") or c[0].startswith("skew_inference"):
        assert np.any(L.plan.seg_slot < 0)           # the case has overflow segments


def _dev(b: np.ndarray, dtype, *shape) -> torch.Tensor:
    """Device tensor of ``dtype`` and ``shape`` holding the bytes ``b``."""
    if b.size == 0:
        return torch.empty(shape, dtype=dtype, device="cuda")
    return torch.from_numpy(np.ascontiguousarray(b)).cuda().view(dtype).view(*shape)


def _bytes_case(E, R, S, row_bytes, seed):
    rng = np.random.default_rng(seed)
    wb = rng.integers(0, 256, (E, row_bytes), dtype=np.uint8)
    sb = rng.integers(0, 256, (R, S, row_bytes), dtype=np.uint8)
    return wb, sb


@pytest.mark.parametrize("dtype,P", [(torch.bfloat16, 8), (torch.bfloat16, 20000),
                                     (torch.float32, 12), (torch.float8_e4m3fn, 70000),
                                     # rows that are not a multiple of 16 bytes (4-byte path)
                                     (torch.float32, 3), (torch.bfloat16, 6), (torch.float32, 5003)])
@pytest.mark.parametrize("c", PLANS, ids=[c[0] for c in PLANS])
def test_prefetch_parity(c, dtype, P):
    print(f"[prefetch] copy {c[0]} {dtype} P={P}", flush=True)
    g, h, L, _, _ = _planned(c)
    E, R, S = c[2], c[4], c[5]
    esz = torch.empty(0, dtype=dtype).element_size()
    wb, sb = _bytes_case(E, R, S, P * esz, 1000 * c[7] + P)
    wt = _dev(wb, dtype, E, P)
    st = _dev(sb, dtype, R, S, P)
    buf = ep.Buffer(g)
    buf.prefetch_replicas(wt, h, st)
    torch.cuda.synchronize()
    want = oracle.prefetch(wb, L.plan.replica, sb)
    got = st.cpu().view(torch.uint8).numpy().reshape(want.shape)
    assert np.array_equal(got, want)
    # the 2-D slot form [R*S, P] gives the same bytes
    st2 = _dev(sb, dtype, R * S, P)
    ep.ep_prefetch_replicas(h.ptr, wt, st2)
    torch.cuda.synchronize()
    assert np.array_equal(st2.cpu().view(torch.uint8).numpy().reshape(want.shape), want)


def test_prefetch_follows_a_new_plan():
    # the same handle re-planned with other routing fills other slots
    E, R, S, k, T = 32, 8, 4, 4, 600
    g = make_group(E, R, 8, k, T, "static", 0, S, "inference")
    h = ep.Handle(g, T)
    buf = ep.Buffer(g)
    wb, sb = _bytes_case(E, R, S, 4096, 77)
    wt = torch.from_numpy(wb).cuda().view(torch.bfloat16).view(E, 2048)
    for seed, skew in ((31, 2.0), (32, 0.7)):
        idx, _, _ = workloads.random_case(seed, T, 8, E, k, skew=skew)
        h.plan(dev_i32(idx))
        st = torch.from_numpy(sb).cuda().view(torch.bfloat16).view(R, S, 2048)
        buf.prefetch_replicas(wt, h, st)
        torch.cuda.synchronize()
        L = oracle.layout(idx, E, "static", R=R, S=S, slot_mode=oracle.SLOTS_INFERENCE)
        assert np.array_equal(host(h.tables()["replica"]), L.plan.replica)
        want = oracle.prefetch(wb, L.plan.replica, sb)
        assert np.array_equal(st.view(torch.uint8).cpu().numpy().reshape(R, S, -1), want)


def test_prefetch_training_workload_full_size():
    # training shapes: 128 experts' [4096, 1536] bf16 projections into 16 ranks x 8 slots
    inp = workloads.make_inputs("training")
    c = inp.cfg
    P = 4096 * 1536
    g = make_group(c.E, c.R, c.H, c.k, c.T, "static", 0, c.S)
    h = ep.Handle(g, c.T)
    h.plan(dev_i32(inp.topk_idx))
    L = oracle.layout(inp.topk_idx, c.E, "static", R=c.R, S=c.S)
    rep = L.plan.replica
    assert np.array_equal(host(h.tables()["replica"]), rep)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5005)
    wt = torch.randint(-32768, 32767, (c.E, P), dtype=torch.int16, device="cuda", generator=gen)
    st = torch.full((c.R, c.S, P), 0x5A5A, dtype=torch.int16, device="cuda")
    ep.Buffer(g).prefetch_replicas(wt.view(torch.bfloat16), h, st.view(torch.bfloat16))
    torch.cuda.synchronize()
    filled = np.argwhere(rep >= 0)
    assert filled.shape[0] > 0
    for r, s in filled:                                # every filled slot, compared on the device
        assert torch.equal(st[r, s], wt[int(rep[r, s])]), (r, s)
    for r, s in np.argwhere(rep < 0)[:8]:               # empty slots untouched
        assert bool((st[r, s] == 0x5A5A).all())
    # two filled slots against the oracle on the host, byte for byte
    for r, s in filled[:: max(1, filled.shape[0] // 2)][:2]:
        e = int(rep[r, s])
        wb = wt[e].cpu().numpy().view(np.uint8)[None]
        got = st[r, s].cpu().numpy().view(np.uint8)
        want = oracle.prefetch(wb, np.array([[0]], np.int32), np.zeros((1, 1, wb.shape[1]), np.uint8))
        assert np.array_equal(got, want[0, 0])
    assert h.status() == 0


def test_prefetch_fp8_weight_scales():
    # the fp32 scales of FP8 weights, tagged FP8_SCALES: [E, N, K/128] rows of
    # 131 * 2 * 4 = 1048 bytes (not a multiple of 16)
    c = PLANS[0]
    g, h, L, _, _ = _planned(c)
    E, R, S = c[2], c[4], c[5]
    rng = np.random.default_rng(77)
    ws = rng.random((E, 131, 2)).astype(np.float32)
    ss = rng.random((R, S, 131, 2)).astype(np.float32)
    st = torch.from_numpy(ss).cuda()
    ep.Buffer(g).prefetch_replicas(torch.from_numpy(ws).cuda(), h, st, scales=True)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), oracle.prefetch(ws, L.plan.replica, ss))
