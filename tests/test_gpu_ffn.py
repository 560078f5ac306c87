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
g = -64)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import dev_bf16, dev_i32, host_bits, make_group
from tests.helpers import bf16_bits_to_f32, rel_err
from tests.test_gpu_gemm import CASES as BF16_CASES, SENTINEL, _bits, _run as run_bf16
from tests.test_gpu_gemm_fp8 import CASES as FP8_CASES, _run as run_fp8

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
