"""GPU parity of the FP8 path with power-of-two scales (a group with
fp8_scales="pow2"): the FP8 dispatch and ep_quantize_fp8 write power-of-two
scales bit for bit as the oracle's quantiser does, and the grouped GEMM of
large groups runs the 256 x 256 kernel whose matrix cores apply the scales
(v_mfma_scale_f32_32x32x64_f8f6f4 block exponents) with no per-block
rescaling on the vector ALU.

The GEMM's tolerance is the one of the FP8 GEMM tests (tests/test_gpu_gemm_fp8.py):
products exact, groups of 8 K truncated inside the MFMA relative to the
group's largest exponent sum, fp32 accumulation, one bf16 rounding on each
side; the scales are powers of two, so applying them is exact.  Small
integer codes with power-of-two scales are exact end to end."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, host_bits, make_group
from tests.helpers import bf16_bits_to_f32, rel_err
from tests.test_gpu_gemm_fp8 import SENTINEL, check_gemm_fp8, dev_u8, finite_codes, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def pow2_scales(rng, shape, lo, hi):
    return np.ldexp(1.0, rng.integers(lo, hi, shape)).astype(np.float32)


# name, T, E, k, layout, cap, R, S, mode, K, N, skew, seed, use_slots
# (the first ones have at least 128 rows per expert on average and N >= 256:
# the 256 x 256 kernel; the last two the 128 x 128 kernel in the same format)
CASES = [
    ("wide_ht", 2000, 8, 4, "ht", 0, 1, 0, "training", 384, 320, 1.0, 31, False),
    ("wide_ht_skewed", 3000, 16, 8, "ht", 0, 1, 0, "training", 256, 256, 1.5, 32, False),
    ("wide_ll", 2100, 8, 2, "ll", 600, 1, 0, "training", 640, 288, 0.8, 33, False),
    ("wide_static_slots", 3000, 16, 4, "static", 0, 4, 2, "training", 256, 384, 1.5, 34, True),
    ("wide_static_owner", 3000, 16, 4, "static", 0, 4, 2, "training", 128, 272, 1.5, 35, False),
    ("wide_inference_overflow", 2500, 16, 8, "static", 0, 8, 1, "inference", 512, 256, 1.8, 36, True),
    ("wide_n_not_multiple_of_8", 2000, 8, 4, "ht", 0, 1, 0, "training", 256, 262, 1.0, 37, False),
    ("narrow_ht", 300, 16, 4, "ht", 0, 1, 0, "training", 256, 96, 1.0, 38, False),
    ("small_groups", 200, 16, 2, "ht", 0, 1, 0, "training", 128, 512, 1.0, 39, False),
]


def _run(c, glu=None, sx_lo=-8, sx_hi=2):
    name, T, E, k, kind, cap, R, S, mode, K, N, skew, seed, use_slots = c
    print(f"[gemm_fp8_pow2] {name} T={T} E={E} k={k} {kind} K={K} N={N}", flush=True)
    idx, _, _ = workloads.random_case(5600 + seed, T, 8, E, k, skew=skew)
    g = make_group(E, R, 8, k, T, kind, cap, S, mode, fp8_scales="pow2")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S,
                      slot_mode=oracle.SLOTS_INFERENCE if mode == "inference" else oracle.SLOTS_TRAINING)
    rng = np.random.default_rng(seed)
    NB = K // 128
    x = finite_codes(rng, (L.rows, K))
    sx = pow2_scales(rng, (L.rows, NB), sx_lo, sx_hi)
    w = finite_codes(rng, (E, N, K))
    sw = pow2_scales(rng, (E, N, NB), -12, -6)
    buf = ep.Buffer(g)
    slots_t = slot_sc_t = None
    w_all, sw_all = w, sw
    if use_slots:
        slots_t = buf.prefetch_replicas(dev_u8(w), h, dev_u8(np.zeros((R, S, N, K), np.uint8)))
        slot_sc_t = buf.prefetch_replicas(dev_f32(sw), h, torch.zeros((R, S, N, NB), device="cuda"),
                                          scales=True)
        torch.cuda.synchronize()
        w_all = np.concatenate([w, host_u8(slots_t).reshape(R * S, N, K)])
        sw_all = np.concatenate([sw, host(slot_sc_t).reshape(R * S, N, NB)])
    y = torch.full((L.rows, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    xd, sxd, wd, swd = dev_u8(x), dev_f32(sx), dev_u8(w), dev_f32(sw)
    buf.expert_gemm_fp8(xd, sxd, wd, swd, h, slots_t, slot_sc_t, out=y)
    if glu is not None:
        a = torch.full((L.rows, N // 2), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        buf.expert_gemm_fp8(xd, sxd, wd, swd, h, slots_t, slot_sc_t, out=a, swiglu=True)
    torch.cuda.synchronize()
    if glu is not None:
        glu.append(host_bits(a))
    groups = oracle.expert_groups(L, kind, E, cap=cap, R=R, S=S, use_slots=use_slots)
    ref = oracle.grouped_gemm_fp8(x, sx, w_all, sw_all, groups, np.full((L.rows, N), SENTINEL, np.uint16))
    return host_bits(y), ref, (x, sx, w_all, sw_all), groups, L, h


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_grouped_gemm_fp8_pow2_parity(c):
    yb, ref, ops, groups, L, h = _run(c)
    covered = np.zeros(L.rows, bool)
    for r0, n, _ in groups:
        covered[r0:r0 + n] = True
    assert np.all(yb[~covered] == SENTINEL)
    check_gemm_fp8(yb, ref, *ops, groups, separable=L.rows > 2048)
    assert h.status() & ep.FLAG_SCALE_FORMAT == 0


@pytest.mark.parametrize("name", ["wide_ht", "wide_static_slots"])
def test_grouped_gemm_fp8_pow2_swiglu(name):
    c = next(c for c in CASES if c[0] == name)
    glu = []
    yb, ref, ops, groups, L, _ = _run(c, glu)
    act = glu[0]
    rows = np.concatenate([np.arange(r0, r0 + n) for r0, n, _ in groups])
    # against the kernel's own plain output put through SwiGLU in double:
    # one bf16 rounding (the SwiGLU store reads the same staged bf16 tile)
    h_ = bf16_bits_to_f32(yb[rows]).astype(np.float64)
    g_, u_ = h_[:, 0::2], h_[:, 1::2]
    with np.errstate(over="ignore"):
        own = g_ / (1.0 + np.exp(-g_)) * u_
    got = bf16_bits_to_f32(act[rows]).astype(np.float64)
    assert np.all(np.abs(got - own) <= np.abs(own) * 2.0 ** -8 * 1.01 + 2.0 ** -133)
    covered = np.zeros(L.rows, bool)
    covered[rows] = True
    assert np.all(act[~covered] == SENTINEL)


def test_grouped_gemm_fp8_pow2_small_integers_are_exact():
    # codes 0, +-1 .. +-4 and scales 2^-2 .. 2^2: every product is a multiple
    # of 2^-4 below 2^8, so every partial sum over K = 384 (below 2^17) is
    # exact in fp32 and both sides round the same exact value to bf16 once
    T, E, k, K, N = 2000, 8, 4, 384, 264
    idx, _, _ = workloads.random_case(5700, T, 8, E, k, skew=1.0)
    g = make_group(E, 1, 8, k, T, "ht", fp8_scales="pow2")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, "ht")
    rng = np.random.default_rng(57)
    small = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8], np.uint8)  # 0, +-1 .. +-4
    x = small[rng.integers(0, small.size, (L.rows, K))]
    w = small[rng.integers(0, small.size, (E, N, K))]
    sx = pow2_scales(rng, (L.rows, K // 128), -2, 3)
    sw = pow2_scales(rng, (E, N, K // 128), -2, 3)
    y = ep.Buffer(g).expert_gemm_fp8(dev_u8(x), dev_f32(sx), dev_u8(w), dev_f32(sw), h)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm_fp8(x, sx, w, sw, oracle.expert_groups(L, "ht", E))
    assert np.array_equal(host_bits(y), ref)
    assert h.status() == 0


def test_grouped_gemm_fp8_pow2_flags_other_scales():
    # a scale that is not a power of two raises EP_FLAG_SCALE_FORMAT
    T, E, k, K, N = 2000, 8, 4, 256, 256
    idx, _, _ = workloads.random_case(5800, T, 8, E, k)
    g = make_group(E, 1, 8, k, T, "ht", fp8_scales="pow2")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, "ht")
    rng = np.random.default_rng(58)
    x, w = finite_codes(rng, (L.rows, K)), finite_codes(rng, (E, N, K))
    sx = pow2_scales(rng, (L.rows, 2), -4, 2)
    sw = pow2_scales(rng, (E, N, 2), -8, -4)
    sw[3, 7, 1] *= 1.5
    ep.Buffer(g).expert_gemm_fp8(dev_u8(x), dev_f32(sx), dev_u8(w), dev_f32(sw), h)
    torch.cuda.synchronize()
    assert h.status() & ep.FLAG_SCALE_FORMAT


@pytest.mark.parametrize("kind,T", [("ht", 700), ("ll", 128), ("static", 900)])
def test_fp8_dispatch_and_quantiser_pow2_bit_exact(kind, T):
    E, k, H, R, S = 32, 4, 512, 8, 2
    cap = 40 if kind == "ll" else 0
    print(f"[dispatch_fp8_pow2] {kind} T={T}", flush=True)
    rng = np.random.default_rng(59)
    idx, _, _ = workloads.random_case(5900, T, 8, E, k, skew=1.0)
    mag = np.exp2(rng.integers(-140, 120, (T, H // 128, 1)).astype(np.float64))
    x = workloads.f32_to_bf16_bits((rng.standard_normal((T, H // 128, 128)) * mag)
                                   .reshape(T, H).astype(np.float32))
    x[3, :128] = 0                                   # an all-zero block
    g = make_group(E, R if kind == "static" else 1, H, k, T, kind, cap, S if kind == "static" else 0,
                   fp8_scales="pow2")
    h = ep.Handle(g, T)
    buf = ep.Buffer(g)
    h.plan(dev_i32(idx))
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True,
                                      recv_meta=False)
    torch.cuda.synchronize()
    L = oracle.layout(idx, E, kind, cap=cap, R=R if kind == "static" else 1, S=S if kind == "static" else 0)
    wq, ws = oracle.dispatch_fp8(x, L.dst, L.rows, pow2=True)
    used = L.dst[L.dst >= 0]
    assert np.array_equal(host_u8(q).reshape(L.rows, H)[used], wq[used])
    assert np.array_equal(host(s).reshape(L.rows, -1)[used], ws[used])
    cq, cs = ep.Buffer.quantize_fp8(dev_bf16(x), pow2=True)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rows_fp8(x, pow2=True)
    assert np.array_equal(host_u8(cq), oq) and np.array_equal(host(cs), os_)


def test_fp8_dispatch_pow2_fused_decode():
    # the decode path (layout and dispatch in one launch) writes the same
    T, E, k, H, cap = 128, 256, 8, 1024, 128
    idx, _, x = workloads.random_case(6000, T, H, E, k)
    g = make_group(E, 32, H, k, T, "ll", cap, fp8_scales="pow2")
    h = ep.Handle(g, T)
    q = torch.empty(g.recv_shape(T), dtype=torch.float8_e4m3fn, device="cuda")
    s = torch.empty((h.recv_rows, H // 128), dtype=torch.float32, device="cuda")
    ep.ep_plan_dispatch(h.ptr, dev_i32(idx), dev_bf16(x), None, q, s)
    torch.cuda.synchronize()
    L = oracle.layout(idx, E, "ll", cap=cap)
    wq, ws = oracle.dispatch_fp8(x, L.dst, L.rows, pow2=True)
    used = L.dst[L.dst >= 0]
    assert np.array_equal(host_u8(q).reshape(L.rows, H)[used], wq[used])
    assert np.array_equal(host(s).reshape(L.rows, -1)[used], ws[used])


def test_expert_ffn_all_fp8_pow2():
    """The whole FFN on FP8 operands with power-of-two scales: FP8 dispatch,
    the SwiGLU GEMM and the second GEMM on the 256 x 256 kernel, the
    activation quantised by ep_quantize_fp8 in the same format."""
    T, E, k, H, I, H2 = 2000, 8, 4, 256, 256, 384
    idx, _, _ = workloads.random_case(6100, T, 8, E, k, skew=1.0)
    g = make_group(E, 1, H, k, T, "ht", fp8_scales="pow2")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, "ht")
    groups = oracle.expert_groups(L, "ht", E)
    rng = np.random.default_rng(61)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1, sw1 = oracle.quantize_rows_fp8(
        workloads.f32_to_bf16_bits((rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)).astype(np.float32)), pow2=True)
    w2, sw2 = oracle.quantize_rows_fp8(
        workloads.f32_to_bf16_bits((rng.standard_normal((E, H2, I)) / np.sqrt(I)).astype(np.float32)), pow2=True)
    buf = ep.Buffer(g)
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True, recv_meta=False)
    act = torch.zeros((L.rows, I), dtype=torch.bfloat16, device="cuda")
    buf.expert_gemm_fp8(q, s, dev_u8(w1), dev_f32(sw1), h, out=act, swiglu=True)
    qa, sa = buf.quantize_fp8(act, pow2=True)
    out = buf.expert_gemm_fp8(qa, sa, dev_u8(w2), dev_f32(sw2), h)
    torch.cuda.synchronize()
    assert h.status() == 0
    rows = np.concatenate([np.arange(r0, r0 + n) for r0, n, _ in groups])
    xq, xs = oracle.dispatch_fp8(x, L.dst, L.rows, pow2=True)
    assert np.array_equal(host_u8(q).reshape(L.rows, H)[rows], xq[rows])
    act_ref = oracle.swiglu(oracle.grouped_gemm_fp8(xq, xs, w1, sw1, groups))
    ga = host_bits(act)
    a_got = bf16_bits_to_f32(ga[rows]).astype(np.float64)
    a_want = bf16_bits_to_f32(act_ref[rows]).astype(np.float64)
    assert rel_err(a_got, a_want) <= 4e-3
    oq, os_ = oracle.quantize_rows_fp8(ga, pow2=True)
    assert np.array_equal(host_u8(qa)[rows], oq[rows]) and np.array_equal(host(sa)[rows], os_[rows])
    got = bf16_bits_to_f32(host_bits(out)[rows]).astype(np.float64)
    ref2 = bf16_bits_to_f32(oracle.grouped_gemm_fp8(oq, os_, w2, sw2, groups)[rows]).astype(np.float64)
    assert rel_err(got, ref2) <= 2e-3
    assert float(got.ravel() @ ref2.ravel() / (np.linalg.norm(got) * np.linalg.norm(ref2))) > 0.999


def test_wide_fp8_gemm_graph_replays_match_eager():
    """The 256 x 256 FP8 kernel (tile table + GEMM) captured once as a HIP
    graph; new codes and scales are copied into the captured buffers before
    each replay, with eager work in between, and every replay must equal the
    same call made eagerly, bit for bit (the kernel's slab loads and waits are
    its own, so a replay must see the same pipeline as an eager launch)."""
    T, E, k, K, N = 2000, 8, 4, 384, 320
    print(f"[gemm_fp8_pow2] graph replay T={T} E={E} K={K} N={N}", flush=True)
    idx, _, _ = workloads.random_case(6200, T, 8, E, k, skew=1.0)
    g = make_group(E, 1, 8, k, T, "ht", fp8_scales="pow2")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, "ht")
    rng = np.random.default_rng(62)
    NB = K // 128
    x = dev_u8(finite_codes(rng, (L.rows, K)))
    sx = dev_f32(pow2_scales(rng, (L.rows, NB), -8, 2))
    w = dev_u8(finite_codes(rng, (E, N, K)))
    sw = dev_f32(pow2_scales(rng, (E, N, NB), -12, -6))
    y = torch.zeros((L.rows, N), dtype=torch.bfloat16, device="cuda")
    y_ref = torch.zeros_like(y)
    call = lambda out, st: ep.ep_expert_gemm_fp8(h.ptr, x, sx, w, sw, None, None, out, st)
    call(y, None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(y, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for seed in range(3):
        x.copy_(dev_u8(finite_codes(rng, (L.rows, K))))
        sx.copy_(dev_f32(pow2_scales(rng, (L.rows, NB), -8, 2)))
        graph.replay()
        torch.cuda.synchronize()
        got = host_bits(y).copy()
        _ = torch.ones(1 << 20, device="cuda").sum()          # eager work between replays
        call(y_ref, None)
        torch.cuda.synchronize()
        assert np.array_equal(got, host_bits(y_ref)), f"replay {seed}"
        assert h.status() == 0
