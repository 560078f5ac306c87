"""GPU parity of the expert FFN: the grouped GEMM with the SwiGLU store
(bf16 and FP8 operands) and the whole FFN, first GEMM with the activation
then the second GEMM ("Ultra-Large MoE Models" article, section 3.1: the
grouped GEMM is the core of the expert computation; the activation is read
as SwiGLU over weight rows that interleave gate and up projections).

Each case runs the plain GEMM and the SwiGLU one on the same inputs and
checks: rows no group covers are not written; the activation against the
oracle's (its own GEMM, then its SwiGLU in double) norm-wise, the error of
the GEMM carried through silu(g) * u; and, elementwise, against the plain
kernel's own output put through silu(g) * u in double, within one bf16
rounding over the whole range, subnormal results included (the kernel
evaluates e^-g and the reciprocal in fp32, and g * u * e^g in double below
g = -64).

The FP8 FFN's activation goes through ep_quantize_fp8 (the FP8 dispatch's
quantiser as its own entry point) before the second GEMM: its codes and
scales are compared bit for bit with the oracle's quantiser, and the whole
FP8 FFN (FP8 dispatch, FP8 SwiGLU GEMM, quantiser, FP8 GEMM) with the same
chain in the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, host_bits, make_group
from tests.helpers import bf16_bits_to_f32, rel_err
from tests.test_gpu_gemm import CASES as BF16_CASES, SENTINEL, _bits, _run as run_bf16
from tests.test_gpu_gemm_fp8 import CASES as FP8_CASES, _run as run_fp8, dev_u8, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def check_glu(act, y_plain, ref_plain, groups, rows):
    covered = np.zeros(rows, bool)
    for r0, n, _ in groups:
        covered[r0:r0 + n] = True
    assert act.shape == (rows, y_plain.shape[1] // 2)
    assert np.all(act[~covered] == SENTINEL)
    if not covered.any():
        return
    got = bf16_bits_to_f32(act[covered]).astype(np.float64)
    want = bf16_bits_to_f32(oracle.swiglu(ref_plain[covered])).astype(np.float64)
    assert rel_err(got, want) <= 4e-3
    cos = float(got.ravel() @ want.ravel() / (np.linalg.norm(got) * np.linalg.norm(want) + 1e-300))
    assert cos > 0.999 or np.linalg.norm(want) == 0
    h = bf16_bits_to_f32(y_plain[covered]).astype(np.float64)
    g, u = h[:, 0::2], h[:, 1::2]
    with np.errstate(over="ignore"):
        own = g / (1.0 + np.exp(-g)) * u
    # one bf16 rounding: 2^-8 relative for normal results, one step of the
    # subnormal bf16 grid (2^-133) below 2^-126
    bad = np.abs(got - own) > np.abs(own) * 2.0 ** -8 * 1.01 + 2.0 ** -133
    if bad.any():
        at = tuple(np.argwhere(bad)[:6].T)
        raise AssertionError(f"got {got[at]} own {own[at]} gate {g[at]} up {u[at]}")


BF16_GLU = ["ht_small", "ll_capacity", "static_slots", "static_inference_overflow", "empty",
            "wide_ht_k384_n320", "wide_ll_k128_n256", "wide_static_inference_k192_n512",
            "wide_skewed_k192_n256"]
FP8_GLU = ["ht_small", "ht_many_empty", "ll_capacity", "static_slots", "static_inference_overflow",
           "empty", "wide_ll", "wide_static_slots", "wide_inference_overflow"]


@pytest.mark.parametrize("name", BF16_GLU)
def test_swiglu_gemm_parity(name):
    c = next(c for c in BF16_CASES if c[0] == name)
    glu = []
    yb, ref, _, _, groups, L = run_bf16(c, glu)
    check_glu(glu[0], yb, ref, groups, L.rows)


@pytest.mark.parametrize("name", FP8_GLU)
def test_swiglu_gemm_fp8_parity(name):
    c = next(c for c in FP8_CASES if c[0] == name)
    glu = []
    yb, ref, _, groups, L = run_fp8(c, glu)
    check_glu(glu[0], yb, ref, groups, L.rows)


def test_swiglu_gemm_rejects_n_not_a_multiple_of_16():
    T, E, k, K, N = 64, 4, 2, 64, 264
    idx, _, _ = workloads.random_case(3300, T, 8, E, k)
    g = make_group(E, 1, 8, k, T, "ht")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    x = torch.zeros((h.recv_rows, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((E, N, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ep.EpError):
        ep.Buffer(g).expert_gemm(x, w, h, swiglu=True)
    w256 = torch.zeros((E, 256, K), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((h.recv_rows, 256), dtype=torch.bfloat16, device="cuda")   # N/2 columns expected
    with pytest.raises(ep.EpError):
        ep.ep_expert_gemm_swiglu(h.ptr, x, w256, None, out)


@pytest.mark.parametrize("kind", ["ht", "static"])
def test_expert_ffn_two_gemms(kind):
    # x [rows, K] -> SwiGLU GEMM over [E, 2I, K] -> [rows, I] -> GEMM over [E, H2, I]
    T, E, k, R, S, K, I, H2 = 700, 8, 2, 4, 2, 128, 128, 192
    print(f"[ffn] {kind} T={T} E={E} K={K} I={I} H2={H2}", flush=True)
    idx, _, _ = workloads.random_case(3400, T, 8, E, k, skew=1.0)
    g = make_group(E, R if kind == "static" else 1, 8, k, T, kind, 0, S if kind == "static" else 0)
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, kind, R=R if kind == "static" else 1, S=S if kind == "static" else 0)
    rng = np.random.default_rng(41)
    xb = _bits(rng.standard_normal((L.rows, K)))
    w1 = _bits(rng.standard_normal((E, 2 * I, K)) / np.sqrt(K))
    w2 = _bits(rng.standard_normal((E, H2, I)) / np.sqrt(I))
    buf = ep.Buffer(g)
    act = buf.expert_gemm(dev_bf16(xb), dev_bf16(w1.reshape(E, -1)).view(E, 2 * I, K), h, swiglu=True)
    out = buf.expert_gemm(act, dev_bf16(w2.reshape(E, -1)).view(E, H2, I), h)
    torch.cuda.synchronize()
    groups = oracle.expert_groups(L, kind, E, R=R if kind == "static" else 1, S=S if kind == "static" else 0)
    ref = oracle.grouped_gemm(oracle.swiglu(oracle.grouped_gemm(xb, w1, groups)), w2, groups)
    rows = np.concatenate([np.arange(r0, r0 + n) for r0, n, _ in groups]) if len(groups) else np.zeros(0, int)
    got = bf16_bits_to_f32(host_bits(out)[rows]).astype(np.float64)
    want = bf16_bits_to_f32(ref[rows]).astype(np.float64)
    assert got.size > 0
    assert rel_err(got, want) <= 1e-2
    assert float(got.ravel() @ want.ravel() / (np.linalg.norm(got) * np.linalg.norm(want))) > 0.9995


def _block_values(rng, rows, K):
    """bf16 rows whose 128-wide blocks span the whole range: per block a
    random binary exponent from subnormal bf16 (2^-133) to 2^126, all-zero
    blocks, blocks with a single nonzero, negative zeros, and blocks holding
    the largest finite bf16."""
    nb = K // 128
    e = rng.integers(-140, 120, (rows, nb, 1))
    v = rng.standard_normal((rows, nb, 128)) * np.exp2(e.astype(np.float64))
    kind = rng.integers(0, 12, (rows, nb))
    v[kind == 0] = 0.0
    one = kind == 1
    v[one] = 0.0
    v[one, 0] = rng.standard_normal(int(one.sum())) * 2.0 ** 40
    v[kind == 2] = -0.0
    big = kind == 3
    v[big, 5] = 3.3895313892515355e38
    v[big, 9] = -3.3895313892515355e38
    return workloads.f32_to_bf16_bits(v.reshape(rows, K).astype(np.float32))


@pytest.mark.parametrize("shape", [(1, 128), (3, 256), (1000, 1024), (37, 7168), (4, 9, 384), (0, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_quantize_fp8_bit_exact(shape):
    print(f"[quantize_fp8] {shape}", flush=True)
    rng = np.random.default_rng(5100 + sum(shape))
    K = shape[-1]
    rows = int(np.prod(shape[:-1]))
    x = _block_values(rng, rows, K).reshape(shape)
    codes, scales = ep.Buffer.quantize_fp8(dev_bf16(x))
    torch.cuda.synchronize()
    assert codes.shape == shape and scales.shape == shape[:-1] + (K // 128,)
    wq, ws = oracle.quantize_rows_fp8(x)
    assert np.array_equal(host_u8(codes), wq)
    assert np.array_equal(host(scales).view(np.uint32), ws.view(np.uint32))


def test_quantize_fp8_equals_fp8_dispatch():
    # the same rows quantised by the dispatch (k = 2 copies each) and by the
    # standalone quantiser: identical codes and scales
    T, E, k, H = 300, 8, 2, 512
    rng = np.random.default_rng(5200)
    x = _block_values(rng, T, H)
    idx, _, _ = workloads.random_case(5201, T, 8, E, k)
    g = make_group(E, 1, H, k, T, "ht")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    (q, s), _, _, _, _ = ep.Buffer(g).dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True,
                                               recv_meta=False)
    cq, cs = ep.Buffer.quantize_fp8(dev_bf16(x))
    torch.cuda.synchronize()
    dst = host(h.tables()["dst"]).reshape(T, k)
    qd, sd = host_u8(q).reshape(-1, H), host(s).reshape(-1, H // 128)
    for j in range(k):
        sel = dst[:, j] >= 0
        assert np.array_equal(qd[dst[sel, j]], host_u8(cq)[sel])
        assert np.array_equal(sd[dst[sel, j]], host(cs)[sel])


@pytest.mark.parametrize("kind", ["ht", "ll", "static"])
def test_expert_ffn_all_fp8(kind):
    """tokens -> FP8 dispatch -> FP8 GEMM [E, 2I, H] with SwiGLU -> bf16
    [rows, I] -> ep_quantize_fp8 -> FP8 GEMM [E, H2, I] -> bf16 [rows, H2]."""
    T, E, k, R, S, H, I, H2 = 600, 8, 2, 4, 2, 256, 256, 384
    cap = 96 if kind == "ll" else 0
    print(f"[ffn_fp8] {kind} T={T} E={E} H={H} I={I} H2={H2}", flush=True)
    idx, _, _ = workloads.random_case(5300, T, 8, E, k, skew=1.0)
    Rk = R if kind == "static" else 1
    Sk = S if kind == "static" else 0
    g = make_group(E, Rk, H, k, T, kind, cap, Sk)
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    L = oracle.layout(idx, E, kind, cap=cap, R=Rk, S=Sk)
    groups = oracle.expert_groups(L, kind, E, cap=cap, R=Rk, S=Sk)
    rng = np.random.default_rng(43)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1, sw1 = oracle.quantize_rows_fp8(
        workloads.f32_to_bf16_bits((rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)).astype(np.float32)))
    w2, sw2 = oracle.quantize_rows_fp8(
        workloads.f32_to_bf16_bits((rng.standard_normal((E, H2, I)) / np.sqrt(I)).astype(np.float32)))
    buf = ep.Buffer(g)
    (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True, recv_meta=False)
    act = torch.zeros((L.rows, I), dtype=torch.bfloat16, device="cuda")
    buf.expert_gemm_fp8(q, s, dev_u8(w1), dev_f32(sw1), h, out=act, swiglu=True)
    qa, sa = buf.quantize_fp8(act)
    out = buf.expert_gemm_fp8(qa, sa, dev_u8(w2), dev_f32(sw2), h)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(r0, r0 + n) for r0, n, _ in groups]) if len(groups) else np.zeros(0, int)
    assert rows.size > 0
    # the chain in the oracle
    xq, xs = oracle.dispatch_fp8(x, L.dst, L.rows)
    assert np.array_equal(host_u8(q).reshape(L.rows, H)[rows], xq[rows])
    assert np.array_equal(host(s).reshape(L.rows, -1)[rows], xs[rows])
    act_ref = oracle.swiglu(oracle.grouped_gemm_fp8(xq, xs, w1, sw1, groups))
    # the quantiser on the GPU's own activation: bit for bit the oracle's
    ga = host_bits(act)
    oq, os_ = oracle.quantize_rows_fp8(ga)
    assert np.array_equal(host_u8(qa)[rows], oq[rows])
    assert np.array_equal(host(sa)[rows], os_[rows])
    # activations agree within the FP8 GEMM's bound carried through SwiGLU
    a_got = bf16_bits_to_f32(ga[rows]).astype(np.float64)
    a_want = bf16_bits_to_f32(act_ref[rows]).astype(np.float64)
    assert rel_err(a_got, a_want) <= 4e-3
    # the second GEMM on the GPU's quantised activation: the FP8 GEMM's
    # operator bar on quantised data (norm-wise 2e-3, cosine above 0.999)
    got = bf16_bits_to_f32(host_bits(out)[rows]).astype(np.float64)
    ref2 = bf16_bits_to_f32(oracle.grouped_gemm_fp8(oq, os_, w2, sw2, groups)[rows]).astype(np.float64)
    assert rel_err(got, ref2) <= 2e-3
    assert float(got.ravel() @ ref2.ravel() / (np.linalg.norm(got) * np.linalg.norm(ref2))) > 0.999
    # the whole chain against the oracle's: an activation one bf16 step off
    # can land in the next e4m3 bin, more often for values far below their
    # block's amax (coarser e4m3 steps there); with a third of the
    # activations one step off, the oracle alone puts about 3% of the codes
    # one step apart and the outputs 1.5e-2 apart norm-wise; the bar is 3e-2
    aq, as_ = oracle.quantize_rows_fp8(act_ref)
    want = bf16_bits_to_f32(oracle.grouped_gemm_fp8(aq, as_, w2, sw2, groups)[rows]).astype(np.float64)
    assert rel_err(got, want) <= 3e-2
    assert float(got.ravel() @ want.ravel() / (np.linalg.norm(got) * np.linalg.norm(want))) > 0.999
