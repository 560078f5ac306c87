"""Seeded synthetic inputs for the MoE expert-parallel dispatch / combine path.

This module only *draws* inputs: router logits, top-k routing, activations,
upstream gradients and duplicated-expert gradient replicas.  It holds none of
the arithmetic of the method itself (no histogram, offset, permutation,
planning, quantisation or reduction of the path), so that both the CPU oracle
and the GPU path can consume the same inputs without sharing any code.

Shapes follow the five workloads of the path:

* ``tiny``     T=64,    H=256,  E=8,   top-2, 4 ranks x 2 experts, LL cap 64.
* ``decode``   T=128,   H=7168, E=256, top-8, 32 ranks x 8 experts, LL cap 128.
* ``prefill``  T=4096,  H=7168, E=256, top-8, Zipf(1.1)-skewed expert loads, HT.
* ``sweep``    T=8192,  H=7168, E=384, top-8, 48 ranks x 8 experts, hot-expert
  bias chosen so that max/mean expert load is rho in {1, 2, 4, 8}; STATIC.
* ``training`` T=16384, H=4096, E=128, top-8, logits ~ N(0, 1.5^2),
  16 ranks x 8 experts; STATIC; plus bf16 weight-gradient replicas.

Routing (top-k by descending logit, ties to the lower expert id, weights a
softmax over the k chosen logits) is how the NCCL EP paper's callers produce
``topk_idx`` / ``topk_weights`` (Table IV of the NCCL EP listing names these as
inputs); the "Ultra-Large MoE Models" article, section 2.1, describes the top-k
gate.  Here it is input preparation done on the host, fed to both sides.

Every draw uses numpy's PCG64 with seed ``1000 * config_number + s``; the draw
order is logits, x, gy, replica grads, owner grads.
"""

from __future__ import annotations

import dataclasses
import functools

import numpy as np

# Layout codes shared by name only (each side defines its own enum).
LAYOUT_LL = "ll"
LAYOUT_HT = "ht"
LAYOUT_STATIC = "static"


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    number: int          # 1..5, the seed base is 1000 * number
    T: int               # tokens
    H: int               # hidden size (bf16 channels)
    E: int               # experts
    k: int               # top-k
    R: int               # logical ranks (E % R == 0)
    layout: str          # "ll" | "ht" | "static"
    cap: int = 0         # LL rows per expert
    S: int = 0           # STATIC replica slots per rank
    logit_std: float = 1.0
    bias: str = "none"   # "none" | "zipf" | "hot"
    rho: float = 1.0     # target max/mean expert load for bias == "hot"
    out_fp32: bool = False
    fp8: bool = False

    @property
    def m(self) -> int:
        return self.E // self.R


CONFIGS = {
    "tiny": Config("tiny", 1, T=64, H=256, E=8, k=2, R=4, layout=LAYOUT_LL, cap=64, S=2,
                   out_fp32=True),
    "decode": Config("decode", 2, T=128, H=7168, E=256, k=8, R=32, layout=LAYOUT_LL, cap=128,
                     fp8=True),
    "prefill": Config("prefill", 3, T=4096, H=7168, E=256, k=8, R=32, layout=LAYOUT_HT,
                      bias="zipf"),
    "training": Config("training", 5, T=16384, H=4096, E=128, k=8, R=16, layout=LAYOUT_STATIC,
                       S=8, logit_std=1.5),
}
SWEEP_RHOS = (1.0, 2.0, 4.0, 8.0)


def sweep_config(rho: float) -> Config:
    return Config("sweep", 4, T=8192, H=7168, E=384, k=8, R=48, layout=LAYOUT_STATIC, S=8,
                  bias="hot", rho=float(rho))


def get_config(name: str, rho: float = 1.0) -> Config:
    if name == "sweep":
        return sweep_config(rho)
    return CONFIGS[name]


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------

def rng_for(cfg: Config, s: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg.number + s))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's CPU cast (a library
    conversion used only to store the drawn activations in bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def route_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k routing: experts by descending logit (ties -> lower id, j=0 is the
    largest), weights = softmax over the k chosen logits (fp64, stored fp32)."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def _topk_set_counts(logits: np.ndarray, k: int, E: int) -> np.ndarray:
    part = np.argpartition(-logits, k - 1, axis=1)[:, :k]
    return np.bincount(part.ravel(), minlength=E)


def zipf_bias(E: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit bias -s*ln(e+1): the log of a Zipf(s) pmf up to a constant,
    expert 0 hottest."""
    return (-s * np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)


def hot_bias(base: np.ndarray, k: int, m: int, rho: float, steps: int = 30) -> float:
    """Bias b added to experts [0, m) (the first rank's experts) so that the
    realised max/mean expert load equals rho, found by bisection."""
    if rho <= 1.0:
        return 0.0
    T, E = base.shape
    mean = T * k / E

    def ratio(b: float) -> float:
        lg = base.copy()
        lg[:, :m] += np.float32(b)
        return _topk_set_counts(lg, k, E).max() / mean

    lo, hi = 0.0, 8.0
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if ratio(mid) < rho:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# ---------------------------------------------------------------------------
# per-config inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    cfg: Config
    logits: np.ndarray       # [T, E] fp32
    topk_idx: np.ndarray     # [T, k] int32
    topk_w: np.ndarray       # [T, k] fp32
    x: np.ndarray            # [T, H] bf16 bits (uint16)
    bias_value: float = 0.0


def _logits(cfg: Config, rng: np.random.Generator) -> tuple[np.ndarray, float]:
    lg = (rng.standard_normal((cfg.T, cfg.E), dtype=np.float32) * np.float32(cfg.logit_std))
    b = 0.0
    if cfg.bias == "zipf":
        lg = lg + zipf_bias(cfg.E)[None, :]
    elif cfg.bias == "hot":
        b = hot_bias(lg, cfg.k, cfg.m, cfg.rho)
        lg[:, : cfg.m] += np.float32(b)
    return lg.astype(np.float32), b


@functools.lru_cache(maxsize=8)
def make_inputs(name: str, s: int = 0, rho: float = 1.0, T: int | None = None) -> Inputs:
    """Inputs of workload ``name`` with seed offset ``s``.  ``T`` optionally
    truncates to the first T tokens (same draws, prefix of the batch)."""
    cfg = get_config(name, rho)
    rng = rng_for(cfg, s)
    lg, b = _logits(cfg, rng)
    x = rng.standard_normal((cfg.T, cfg.H), dtype=np.float32)
    idx, w = route_topk(lg, cfg.k)
    xb = f32_to_bf16_bits(x)
    if T is not None:
        lg, idx, w, xb = lg[:T], idx[:T], w[:T], xb[:T]
    return Inputs(cfg, lg, np.ascontiguousarray(idx), np.ascontiguousarray(w),
                  np.ascontiguousarray(xb), b)


def make_grad(cfg: Config, s: int, shape: tuple[int, ...], stream: int) -> np.ndarray:
    """bf16 N(0,1) bits for upstream gradients (stream=1: gy, 2: replica grads)."""
    rng = np.random.Generator(np.random.PCG64([1000 * cfg.number + s, stream]))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_owner(cfg: Config, s: int, shape: tuple[int, ...]) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([1000 * cfg.number + s, 3]))
    return rng.standard_normal(shape, dtype=np.float32)


# ---------------------------------------------------------------------------
# small / adversarial inputs for edge-case tests
# ---------------------------------------------------------------------------

def random_case(seed: int, T: int, H: int, E: int, k: int, mask_frac: float = 0.0,
                bad_frac: float = 0.0, dup_frac: float = 0.0, skew: float = 0.0):
    """Random routing with optional masked (-1) entries, out-of-range ids and
    duplicate experts inside a token.  Returns (topk_idx, topk_w, x_bits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lg = rng.standard_normal((T, E), dtype=np.float32)
    if skew:
        lg = lg + zipf_bias(E, skew)[None, :]
    idx, w = route_topk(lg, k) if T > 0 else (np.zeros((0, k), np.int32), np.zeros((0, k), np.float32))
    idx = idx.copy()
    if T > 0 and dup_frac > 0 and k > 1:
        sel = rng.random(T) < dup_frac
        idx[sel, 1] = idx[sel, 0]
    if T > 0 and mask_frac > 0:
        idx[rng.random((T, k)) < mask_frac] = -1
    if T > 0 and bad_frac > 0:
        bad = rng.random((T, k)) < bad_frac
        idx[bad] = np.where(rng.random(bad.sum()) < 0.5, E + rng.integers(0, 5, bad.sum()),
                            -2 - rng.integers(0, 5, bad.sum())).astype(np.int32)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    return np.ascontiguousarray(idx, dtype=np.int32), np.ascontiguousarray(w), x

