"""GPU parity on a seeded sweep of random configurations: expert counts,
ranks, top-k (specialised and generic kernels), layouts, LL capacities,
replica slots and slot modes, batch sizes from empty to several layout
tiles, masked / out-of-range / duplicate ids and skewed routing, drawn from
one seed per case.  Each case goes through plan -> dispatch (bf16, and FP8
when H allows) -> combine -> combine backward -> dispatch backward via the C
ABI and is compared with the oracle: tables, dispatched rows, FP8 codes and
scales and combine-backward rows bit-exact; combine, dispatch backward and
grad_w as in the parity tests (one bf16 ulp elementwise and 2e-3
norm-wise).  A second sweep runs both grouped GEMMs (bf16 and FP8) on random
K, N, layouts and prefetch slots, to the GEMM tests' tolerances, and, where N
is a multiple of 16, the same GEMMs with the SwiGLU store."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_ep_plan_amd as ep
import oracle
import workloads
from tests.gpu_util import check_layout, dev_bf16, dev_f32, dev_i32, host, host_bits, make_group
from tests.helpers import bf16_bits_to_f32, rel_err

pytestmark = pytest.mark.gpu

N_CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.load_library()
    oracle.build(force=False)


def draw(seed: int) -> dict:
    """One random configuration (pure function of the seed)."""
    rng = np.random.default_rng(90_000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    m = int(rng.choice([1, 2, 3, 5, 8, 16]))
    E = min(R * m, 1024)
    E -= E % R
    k = min(int(rng.choice([1, 2, 3, 4, 6, 8, 9, 16])), E)
    kind = str(rng.choice(["ll", "ht", "static"]))
    T = int(rng.choice([0, 1, 7, 64, 255, 1000, 3000, 5000]))
    H = int(rng.choice([8, 64, 128, 136, 256, 384]))
    cap = int(rng.integers(1, max(2, (T * k) // max(E, 1) + 8))) if kind == "ll" else 0
    S = int(rng.integers(0, m + 2)) if kind == "static" else 0
    mode = str(rng.choice(["training", "inference"])) if kind == "static" else "training"
    return dict(seed=seed, R=R, E=E, k=k, kind=kind, T=T, H=H, cap=cap, S=S, mode=mode,
                mask=float(rng.choice([0.0, 0.05])), bad=float(rng.choice([0.0, 0.01])),
                dup=float(rng.choice([0.0, 0.1])), skew=float(rng.choice([0.0, 1.0, 2.0])))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    c = draw(seed)
    print(f"[random] {c}", flush=True)
    E, R, H, k, T, kind, cap, S = c["E"], c["R"], c["H"], c["k"], c["T"], c["kind"], c["cap"], c["S"]
    idx, w, x = workloads.random_case(5000 + seed, T, H, E, k, mask_frac=c["mask"], bad_frac=c["bad"],
                                      dup_frac=c["dup"], skew=c["skew"])
    g = make_group(E, R, H, k, T, kind, cap, S, c["mode"])
    h = ep.Handle(g, T)
    slot_mode = oracle.SLOTS_INFERENCE if c["mode"] == "inference" else oracle.SLOTS_TRAINING
    L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S, slot_mode=slot_mode)
    h.plan(dev_i32(idx))
    check_layout(h, L, kind, idx, w)

    buf = ep.Buffer(g)
    wt = dev_f32(w)
    recv, _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), wt, handle=h, recv_meta=False)
    torch.cuda.synchronize()
    used = L.dst[L.dst >= 0]
    want = oracle.dispatch(x, L.dst, L.rows)
    assert np.array_equal(host_bits(recv).reshape(L.rows, H)[used], want[used])
    if H % 128 == 0:
        (q, s), _, _, _, _ = buf.dispatch(dev_bf16(x), dev_i32(idx), None, handle=h, fp8=True,
                                          recv_meta=False)
        torch.cuda.synchronize()
        oq, osc = oracle.dispatch_fp8(x, L.dst, L.rows)
        assert np.array_equal(q.view(torch.uint8).cpu().numpy().reshape(L.rows, H)[used], oq[used])
        assert np.array_equal(host(s)[used], osc[used])

    # combine of arbitrary expert outputs, its backward and dispatch backward
    rng = np.random.default_rng(seed)
    eo_bits = workloads.f32_to_bf16_bits(rng.standard_normal((L.rows, H)).astype(np.float32))
    eo = dev_bf16(eo_bits).view(recv.shape)
    y = buf.combine(eo, h, wt)
    ref = bf16_bits_to_f32(oracle.combine(eo_bits, L.dst, w)).astype(np.float64)
    got = bf16_bits_to_f32(host_bits(y)).astype(np.float64)
    scale = np.abs(bf16_bits_to_f32(eo_bits)).max(initial=0.0) * k
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + scale * 2.0 ** -20 + 1e-30)
    assert rel_err(got, ref) <= 2e-3
    gy_bits = workloads.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gout, gw = buf.combine_bwd(dev_bf16(gy_bits), eo, wt, h)
    torch.cuda.synchronize()
    rg, rgw = oracle.combine_bwd(gy_bits, eo_bits, L.dst, w, L.rows)
    assert np.array_equal(host_bits(gout).reshape(L.rows, H)[used], rg[used])
    assert rel_err(host(gw).astype(np.float64), rgw.astype(np.float64)) <= 2e-3
    gx = buf.dispatch_bwd(eo, h)
    rx = bf16_bits_to_f32(oracle.combine(eo_bits, L.dst, None)).astype(np.float64)
    assert rel_err(bf16_bits_to_f32(host_bits(gx)).astype(np.float64), rx) <= 2e-3
    assert h.status() == L.flags


# ---------------------------------------------------------------------------
# grouped GEMMs (bf16 and FP8) on random shapes and layouts
# ---------------------------------------------------------------------------

N_GEMM = 48


def draw_gemm(seed: int) -> dict:
    rng = np.random.default_rng(91_000 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    E = R * int(rng.choice([1, 2, 4, 8]))
    k = min(int(rng.choice([1, 2, 4, 8])), E)
    kind = str(rng.choice(["ll", "ht", "static"]))
    T = int(rng.choice([0, 1, 33, 200, 700, 1500]))
    cap = int(rng.integers(1, max(2, (T * k) // E + 8))) if kind == "ll" else 0
    S = int(rng.integers(0, 3)) if kind == "static" else 0
    mode = str(rng.choice(["training", "inference"])) if kind == "static" else "training"
    K = 128 * int(rng.integers(1, 5))
    N = int(rng.choice([1, 8, 37, 64, 128, 160, 200, 257, 272, 320]))
    return dict(R=R, E=E, k=k, kind=kind, T=T, cap=cap, S=S, mode=mode, K=K, N=N,
                skew=float(rng.choice([0.0, 1.5])), slots=bool(kind == "static" and S > 0 and rng.random() < 0.7))


@pytest.mark.parametrize("fp8", [False, True, "pow2"], ids=["bf16", "fp8", "fp8_pow2"])
@pytest.mark.parametrize("seed", range(N_GEMM))
def test_random_grouped_gemm(seed, fp8):
    """bf16, FP8 with any fp32 scales, and FP8 in the power-of-two scale
    format (groups with enough rows per expert and N >= 256 run the 256 x 256
    kernel whose matrix cores apply the scales)."""
    from tests.test_gpu_gemm import check_gemm
    from tests.test_gpu_gemm_fp8 import check_gemm_fp8, dev_u8, finite_codes, host_u8
    c = draw_gemm(seed)
    print(f"[random gemm] fp8={fp8} {c}", flush=True)
    E, R, k, kind, T, cap, S, K, N = c["E"], c["R"], c["k"], c["kind"], c["T"], c["cap"], c["S"], c["K"], c["N"]
    idx, _, _ = workloads.random_case(6000 + seed, T, 8, E, k, skew=c["skew"])
    g = make_group(E, R, 8, k, T, kind, cap, S, c["mode"], fp8_scales="pow2" if fp8 == "pow2" else "amax")
    h = ep.Handle(g, T)
    h.plan(dev_i32(idx))
    slot_mode = oracle.SLOTS_INFERENCE if c["mode"] == "inference" else oracle.SLOTS_TRAINING
    L = oracle.layout(idx, E, kind, cap=cap, R=R, S=S, slot_mode=slot_mode)
    groups = oracle.expert_groups(L, kind, E, cap=cap, R=R, S=S, use_slots=c["slots"])
    rng = np.random.default_rng(seed)
    buf = ep.Buffer(g)
    SENT = 0x7F7F
    y = torch.full((L.rows, N), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if not fp8:
        xb = workloads.f32_to_bf16_bits(rng.standard_normal((L.rows, K)).astype(np.float32))
        wb = workloads.f32_to_bf16_bits((rng.standard_normal((E, N, K)) / np.sqrt(K)).astype(np.float32))
        wt = dev_bf16(wb.reshape(E, N * K)).view(E, N, K)
        slots = buf.prefetch_replicas(wt, h) if c["slots"] else None
        buf.expert_gemm(dev_bf16(xb), wt, h, slots, out=y)
        glu_call = lambda a: buf.expert_gemm(dev_bf16(xb), wt, h, slots, out=a, swiglu=True)
        torch.cuda.synchronize()
        w_all = wb
        if c["slots"]:
            w_all = np.concatenate([wb, host_bits(slots).reshape(R * S, N, K)])
        ref = oracle.grouped_gemm(xb, w_all, groups, np.full((L.rows, N), SENT, np.uint16))
        check_gemm(host_bits(y), ref, xb, w_all, groups)
    else:
        NB = K // 128
        x = finite_codes(rng, (L.rows, K))
        if fp8 == "pow2":
            sx = np.ldexp(1.0, rng.integers(-9, -2, (L.rows, NB))).astype(np.float32)
        else:
            sx = (rng.random((L.rows, NB)) * 2.0 ** -3).astype(np.float32)
        w = finite_codes(rng, (E, N, K))
        if fp8 == "pow2":
            sw = np.ldexp(1.0, rng.integers(-12, -7, (E, N, NB))).astype(np.float32)
        else:
            sw = (rng.random((E, N, NB)) * 2.0 ** -8).astype(np.float32)
        wt, swt = dev_u8(w), dev_f32(sw)
        slots = slot_sc = None
        if c["slots"]:
            slots = buf.prefetch_replicas(wt, h)
            slot_sc = buf.prefetch_replicas(swt, h, scales=True)
        buf.expert_gemm_fp8(dev_u8(x), dev_f32(sx), wt, swt, h, slots, slot_sc, out=y)
        glu_call = lambda a: buf.expert_gemm_fp8(dev_u8(x), dev_f32(sx), wt, swt, h, slots, slot_sc, out=a,
                                                 swiglu=True)
        torch.cuda.synchronize()
        w_all, sw_all = w, sw
        if c["slots"]:
            w_all = np.concatenate([w, host_u8(slots).reshape(R * S, N, K)])
            sw_all = np.concatenate([sw, host(slot_sc).reshape(R * S, N, NB)])
        ref = oracle.grouped_gemm_fp8(x, sx, w_all, sw_all, groups, np.full((L.rows, N), SENT, np.uint16))
        check_gemm_fp8(host_bits(y), ref, x, sx, w_all, sw_all, groups)
        assert h.status() == L.flags, "only the layout's own flags: no scale-format flag"
    covered = np.zeros(L.rows, bool)
    for r0, n, _ in groups:
        covered[r0:r0 + n] = True
    assert np.all(host_bits(y)[~covered] == SENT)
    if N % 16 == 0:   # the same GEMM with the expert FFN's SwiGLU store
        from tests.test_gpu_ffn import check_glu
        a = torch.full((L.rows, N // 2), SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        glu_call(a)
        torch.cuda.synchronize()
        check_glu(host_bits(a), host_bits(y), ref, groups, L.rows)
