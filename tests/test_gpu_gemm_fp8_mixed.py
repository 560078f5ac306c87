"""GPU parity of the FP8 grouped GEMM in a group with
fp8_scales="amax_pow2w": rows with any positive fp32 scales (the amax/448
format of the FP8 dispatch) against weights whose scales are powers of two.
The 128 x 128 FP8 kernel then gives the matrix cores the weight columns'
exponents as block scales and folds only the row scale per 128-channel
block.  The tolerance is the FP8 GEMM's (tests/test_gpu_gemm_fp8.py):
applying a power-of-two scale is exact, so the bound is unchanged.  A weight
scale that is not a power of two raises EP_FLAG_SCALE_FORMAT; the rows' FP8
dispatch keeps the amax format bit for bit."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, host_bits, make_group
from tests.test_gpu_gemm_fp8 import SENTINEL, check_gemm_fp8, dev_u8, finite_codes, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def amax_like_scales(rng, shape):
    """Positive fp32 scales with arbitrary mantissas over a few binades."""
    return (rng.uniform(1.0, 2.0, shape) * np.ldexp(1.0, rng.integers(-10, -2, shape))).astype(np.float32)


def pow2_scales(rng, shape, lo, hi):
    return np.ldexp(1.0, rng.integers(lo, hi, shape)).astype(np.float32)


# name, T, E, k, layout, cap, R, S, mode, K, N, skew, seed, use_slots
CASES = [
    ("ht", 300, 16, 4, "ht", 0, 1, 0, "training", 256, 96, 1.0, 61, False),
    ("ht_large_groups", 2000, 8, 4, "ht", 0, 1, 0, "training", 384, 320, 1.0, 62, False),
    ("ll_capacity", 400, 16, 4, "ll", 60, 1, 0, "training", 128, 136, 1.5, 63, False),
    ("static_slots", 900, 32, 4, "static", 0, 8, 4, "training", 256, 160, 1.5, 64, True),
    ("inference_overflow", 800, 32, 8, "static", 0, 8, 1, "inference", 128, 128, 1.8, 65, True),
    ("n_not_multiple_of_8", 300, 8, 4, "ht", 0, 1, 0, "training", 128, 37, 1.0, 66, False),
]


def _run(c, sw_override=None):
    name, T, E, k, kind, cap, R, S, mode, K, N, skew, seed, use_slots = c
    print(f"[gemm_fp8_mixed] {name} T={T} E={E} k={k} {kind} K={K} N={N}", flush=True)
    idx, _, _ = workloads.random_case(6100 + seed, T, 8, E, k, skew=skew)
    g = make_group(E, R, 8, k, T, kind, cap, S, mode, fp8_scales="amax_pow2w")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S,
                      slot_mode=oracle.SLOTS_INFERENCE if mode == "inference" else oracle.SLOTS_TRAINING)
    rng = np.random.default_rng(seed)
    NB = K // 128
    x = finite_codes(rng, (L.rows, K))
    sx = amax_like_scales(rng, (L.rows, NB))
    w = finite_codes(rng, (E, N, K))
    sw = pow2_scales(rng, (E, N, NB), -12, -6) if sw_override is None else sw_override(rng, (E, N, NB))
    buf = ep.Buffer(g)
    slots_t = slot_sc_t = None
    w_all, sw_all = w, sw
    if use_slots:
        slots_t = buf.prefetch_replicas(dev_u8(w), h, dev_u8(np.zeros((R, S, N, K), np.uint8)))
        slot_sc_t = buf.prefetch_replicas(dev_f32(sw), h, torch.ones((R, S, N, NB), device="cuda"),
                                          scales=True)
        torch.cuda.synchronize()
        w_all = np.concatenate([w, host_u8(slots_t).reshape(R * S, N, K)])
        sw_all = np.concatenate([sw, host(slot_sc_t).reshape(R * S, N, NB)])
    y = torch.full((L.rows, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    buf.expert_gemm_fp8(dev_u8(x), dev_f32(sx), dev_u8(w), dev_f32(sw), h, slots_t, slot_sc_t, out=y)
    torch.cuda.synchronize()
    groups = oracle.expert_groups(L, kind, E, cap=cap, R=R, S=S, use_slots=use_slots)
    ref = oracle.grouped_gemm_fp8(x, sx, w_all, sw_all, groups, np.full((L.rows, N), SENTINEL, np.uint16))
    return host_bits(y), ref, (x, sx, w_all, sw_all), groups, L, h


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_grouped_gemm_fp8_mixed_parity(c):
    yb, ref, ops, groups, L, h = _run(c)
    covered = np.zeros(L.rows, bool)
    for r0, n, _ in groups:
        covered[r0:r0 + n] = True
    assert np.all(yb[~covered] == SENTINEL)
    check_gemm_fp8(yb, ref, *ops, groups, norm=True, separable=L.rows > 2048)
    assert h.status() & ep.FLAG_SCALE_FORMAT == 0
    if c[13]:
        assert np.any(groups[:, 2] >= c[2])


def test_grouped_gemm_fp8_mixed_flags_weight_scales_that_are_not_powers_of_two():
    def skewed(rng, shape):
        s = pow2_scales(rng, shape, -12, -6)
        s[3, 7, 0] *= 1.5
        return s
    c = ("flag", 300, 8, 4, "ht", 0, 1, 0, "training", 128, 64, 1.0, 67, False)
    _, _, _, _, _, h = _run(c, sw_override=skewed)
    assert h.status() & ep.FLAG_SCALE_FORMAT


def test_fp8_dispatch_keeps_amax_scales_in_the_mixed_format():
    # the rows' format is AMAX: codes and scales bit for bit the oracle's amax quantiser
    T, E, k, H = 300, 16, 4, 256
    idx, _, _ = workloads.random_case(6200, T, 8, E, k, skew=1.0)
    x = workloads.f32_to_bf16_bits(np.random.default_rng(68).standard_normal((T, H)).astype(np.float32))
    g = make_group(E, 1, H, k, T, "ht", fp8_scales="amax_pow2w")
    h = ep.Handle(g, T)
    buf = ep.Buffer(g)
    h.plan(dev_i32(idx))
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True,
                                      recv_meta=False)
    torch.cuda.synchronize()
    L = oracle.layout(idx, E, "ht")
    wq, ws = oracle.dispatch_fp8(x, L.dst, L.rows, pow2=False)
    used = L.dst[L.dst >= 0]
    assert np.array_equal(host_u8(q).reshape(L.rows, H)[used], wq[used])
    assert np.array_equal(host(s).reshape(L.rows, -1)[used], ws[used])
