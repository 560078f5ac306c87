"""GPU parity of top-k routing (router logits -> top-k experts and the
softmax over the chosen logits) with the oracle: indices bit-exact (the
selection compares fp32 logits exactly on both sides, equal logits go to
the lower expert id), weights within 1e-5 relative (fp32 exp and division
against the oracle's double).  Also the whole pass from logits: route ->
plan -> dispatch -> combine with identity experts returns x."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_f32, host, host_bits, make_group, same_up_to_zero_sign_np

pytestmark = pytest.mark.gpu
W_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def _route_gpu(lg: np.ndarray, k: int, R: int = 1):
    T, E = lg.shape
    g = make_group(E, R, 8, k, T, "ht")
    h = ep.Handle(g, T)
    idx, w = h.route(dev_f32(lg))
    torch.cuda.synchronize()
    return host(idx), host(w)


def _check(lg, k):
    gi, gw = _route_gpu(lg, k)
    ri, rw = oracle.route(lg, k)
    assert np.array_equal(gi, ri)
    m = ri >= 0
    assert np.all(gw[~m] == 0)
    assert np.all(np.abs(gw[m] - rw[m]) <= W_TOL * rw[m] + 1e-30)


@pytest.mark.parametrize("name,rho", [("tiny", 1.0), ("decode", 1.0), ("prefill", 1.0),
                                      ("sweep", 8.0), ("training", 1.0)])
def test_route_workloads(name, rho):
    inp = workloads.make_inputs(name, rho=rho) if name == "sweep" else workloads.make_inputs(name)
    print(f"[route] {name} T={inp.cfg.T} E={inp.cfg.E} k={inp.cfg.k}", flush=True)
    _check(inp.logits, inp.cfg.k)
    gi, _ = _route_gpu(inp.logits, inp.cfg.k)
    assert np.array_equal(gi, inp.topk_idx)          # the routing the workloads were drawn with


# up to 1024 tokens a token takes a whole wave, above that a 16-lane row
@pytest.mark.parametrize("T,E,k", [(777, 1024, 16), (300, 384, 8), (129, 65, 3), (50, 5, 7),
                                   (33, 1, 1), (0, 16, 4), (1000, 64, 1), (1024, 256, 8),
                                   (1025, 65, 3), (2000, 1024, 16), (1500, 5, 7), (3001, 1, 1)])
def test_route_shapes_and_ties(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if T and E > 3:
        lg[:, E - 1] = lg[:, 0]                          # exact ties across lanes
        lg[: T // 2, 1:4] = 2.5                          # exact ties inside the top-k
        lg[T // 2:, :] = np.round(lg[T // 2:, :])        # many ties
    _check(lg, k)


def test_route_then_the_whole_pass():
    inp = workloads.make_inputs("prefill")
    c = inp.cfg
    g = make_group(c.E, c.R, c.H, c.k, c.T, "ht")
    h = ep.Handle(g, c.T)
    buf = ep.Buffer(g)
    idx, w = h.route(dev_f32(inp.logits))
    h.plan(idx)
    x = dev_bf16(inp.x)
    recv, _, _, _, _ = buf.dispatch(x, idx, w, handle=h, recv_meta=False)
    y = buf.combine(recv, h, w)
    assert same_up_to_zero_sign_np(host_bits(y), inp.x)
    assert h.status() == 0


def test_route_signed_zero_and_infinities():
    # -0 and +0 compare equal (the lower expert id first); -inf logits are
    # chosen only when nothing larger is left and get weight exp(-inf) = 0.
    T, E, k = 96, 48, 6
    lg = np.zeros((T, E), np.float32)
    lg[:, ::2] = -0.0
    lg[::3, 5] = 1.0
    lg[1::3, 7:20] = -np.inf
    lg[2::3, 3:] = -np.inf
    _check(lg, k)
    big = np.zeros((8, E), np.float32)
    big[:, 9] = np.inf
    big[:, 30] = -0.0
    gi, _ = _route_gpu(big, k)
    ri, _ = oracle.route(big, k)
    assert np.array_equal(gi, ri)


# ---------------------------------------------------------------------------
# routing fused into the layout launch (ep_route_plan)
# ---------------------------------------------------------------------------

from tests.gpu_util import check_layout  # noqa: E402


# name, T, E, k, layout, cap, R, S, logit skew
FUSED = [
    ("decode_ll", 128, 256, 8, "ll", 64, 1, 0, 1.0),
    ("prefill_ht_tiles", 4096, 256, 8, "ht", 0, 1, 0, 1.1),
    ("static_k3_split_tokens", 1500, 64, 3, "static", 0, 8, 4, 1.5),   # 2048 % 3 != 0: tokens span tiles
    ("static_k6_inference", 1000, 48, 6, "static", 0, 6, 1, 2.0),
    ("ht_e384_per32", 700, 384, 8, "ht", 0, 1, 0, 0.5),
    ("ll_e1024_unfused", 300, 1024, 16, "ll", 8, 1, 0, 1.0),            # E > 512: two launches
    ("ht_e5_k7", 50, 5, 7, "ht", 0, 1, 0, 0.0),                        # fewer experts than k
    ("empty", 0, 16, 4, "ht", 0, 1, 0, 0.0),
]


@pytest.mark.parametrize("c", FUSED, ids=[c[0] for c in FUSED])
def test_route_plan_matches_route_then_plan_and_oracle(c):
    name, T, E, k, kind, cap, R, S, skew = c
    print(f"[route_plan] {name} T={T} E={E} k={k} {kind}", flush=True)
    rng = np.random.default_rng(4000 + T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if skew:
        lg += workloads.zipf_bias(E, skew)[None, :].astype(np.float32)
    lg[: T // 4, :: 7] = np.round(lg[: T // 4, :: 7], 1)   # ties inside a token
    mode = "inference" if "inference" in name else "training"
    g = make_group(E, R, 8, k, T, kind, cap, S, mode)
    hf, hs = ep.Handle(g, T), ep.Handle(g, T)
    logits = dev_f32(lg)
    fi, fw = hf.route_plan(logits)
    si, sw = hs.route(logits)
    hs.plan(si)
    torch.cuda.synchronize()
    assert np.array_equal(host(fi), host(si))
    assert np.array_equal(host(fw).view(np.uint32), host(sw).view(np.uint32))
    tf = {key: host(v) for key, v in hf.tables().items()}
    ts = {key: host(v) for key, v in hs.tables().items()}
    ns = int(tf["n_segments"][0]) if "n_segments" in tf else 0
    used = tf["dst"][tf["dst"] >= 0]
    for key in tf:
        a, b = tf[key], ts[key]
        if key in ("segments", "seg_slot"):      # defined up to n_segments
            a, b = a[:ns], b[:ns]
        elif key == "recv_src":                  # defined on the rows that hold an entry
            a, b = a[used], b[used]
        assert np.array_equal(a, b), key
    assert hf.status() == hs.status()
    ri, rw = oracle.route(lg, k)
    assert np.array_equal(host(fi), ri)
    m = ri >= 0
    assert np.all(np.abs(host(fw)[m] - rw[m]) <= W_TOL * rw[m] + 1e-30)
    L = oracle.layout(ri, E, kind, cap=cap, R=R, S=S,
                      slot_mode=oracle.SLOTS_INFERENCE if mode == "inference" else oracle.SLOTS_TRAINING)
    check_layout(hf, L, kind, ri, None)


def test_route_plan_then_the_whole_pass():
    # route+plan fused, dispatch, combine with identity experts: x comes back
    inp = workloads.make_inputs("prefill")
    c = inp.cfg
    g = make_group(c.E, c.R, c.H, c.k, c.T, "ht")
    h = ep.Handle(g, c.T)
    idx, w = h.route_plan(dev_f32(inp.logits))
    buf = ep.Buffer(g)
    x = dev_bf16(inp.x)
    recv, _, _, _, _ = buf.dispatch(x, idx, w, handle=h, recv_meta=False)
    y = buf.combine(recv, h, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), inp.topk_idx)
    assert same_up_to_zero_sign_np(host_bits(y), inp.x)


def test_route_large_logits():
    # logits near +-1000: the softmax over the chosen ones must use their
    # differences (exp of the raw values overflows fp32)
    rng = np.random.default_rng(91)
    lg = (rng.standard_normal((300, 64)) + 1000.0 * rng.choice([-1.0, 1.0], size=(300, 1))).astype(np.float32)
    _check(lg, 6)
    _, gw = _route_gpu(lg, 6)
    assert np.all(np.isfinite(gw))
