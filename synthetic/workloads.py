"""Workload table and seeded random draws.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(0,
spawn_key=key)))`` with ``key = (workload id, layer, tensor id, sub-index)``,
so any slice (one expert, one layer) can be regenerated on its own and the
result does not depend on the order in which tensors are requested.

bf16 values are produced by rounding an fp32 sample to the nearest bf16,
ties to even, with integer bit operations; they are returned as ``uint16``
bit patterns so that no library bf16 type is involved.

Shapes and value laws follow the five workloads of the NVFP4 MoE block
(hidden 2816, 128 experts, expert intermediate 704, top-8) plus a tiny one.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

SEED = 0

# tensor ids inside a spawn key
_X, _LOGITS, _BIAS, _W13, _W2, _CAL_X, _CAL_LOGITS, _OUTLIER_CH, _ZIPF, _BAD = range(1, 11)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id used in spawn keys
    T: int              # tokens
    H: int              # hidden size
    E: int              # experts
    I: int              # expert intermediate size
    k: int              # experts per token
    layers: int = 1
    router: str = "normal"          # normal | uniform | normal_bias | zipf
    outlier_frac: float = 0.0       # fraction of hidden channels scaled up
    outlier_gain: float = 1.0
    calib_tokens: int = 512
    weight_std: float = 0.02
    layer_wid: Optional[int] = None  # workload whose layer (weights, scales) is reused
    zipf_s: float = 1.1
    zipf_masked: int = 8            # lowest-ranked experts that never receive tokens

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def weight_wid(self) -> int:
        return self.layer_wid if self.layer_wid is not None else self.wid


WORKLOADS = {
    "tiny": Workload("tiny", 1, T=64, H=256, E=4, I=128, k=2, router="normal", calib_tokens=256),
    "quant": Workload("quant", 2, T=8192, H=2816, E=128, I=704, k=8, router="uniform",
                      outlier_frac=0.01, outlier_gain=50.0, calib_tokens=512),
    "decode": Workload("decode", 3, T=16, H=2816, E=128, I=704, k=8, router="normal",
                       calib_tokens=512),
    "prefill": Workload("prefill", 4, T=4096, H=2816, E=128, I=704, k=8, router="normal_bias",
                        outlier_frac=0.005, outlier_gain=30.0, calib_tokens=512, layer_wid=3),
    "stack": Workload("stack", 5, T=8192, H=2816, E=128, I=704, k=8, layers=30, router="zipf",
                      calib_tokens=512),
    # the boundary's largest expert count and top-k on a small hidden size: the
    # small-batch GEMM path at 96 tokens, the large one at 1024 (P = 32 E)
    "maxsize": Workload("maxsize", 6, T=1024, H=256, E=1024, I=128, k=32, router="normal",
                        calib_tokens=1024),
    # K-step counts that are not multiples of the register-ring depth in either
    # GEMM (w13: 5 steps of 128, w2: 5 steps of 64) and a skewed router
    "shapes": Workload("shapes", 7, T=200, H=640, E=8, I=320, k=3, router="normal_bias",
                       calib_tokens=512),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=tuple(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(shape, std: float, rng: np.random.Generator) -> np.ndarray:
    s = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        s *= np.float32(std)
    return f32_to_bf16_bits(s)


def _outlier_channels(w: Workload, layer: int) -> np.ndarray:
    n = int(round(w.outlier_frac * w.H))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w.wid, layer, _OUTLIER_CH).choice(w.H, size=n, replace=False))


def activations(w: Workload, layer: int = 0, tokens: Optional[int] = None) -> np.ndarray:
    """bf16 bits [T, H]: N(0,1), with the workload's outlier channels scaled up."""
    T = w.T if tokens is None else tokens
    s = _rng(w.wid, layer, _X).standard_normal(size=(T, w.H), dtype=np.float32)
    ch = _outlier_channels(w, layer)
    if ch.size:
        s[:, ch] *= np.float32(w.outlier_gain)
    return f32_to_bf16_bits(s)


def outlier_channels(w: Workload, layer: int = 0) -> np.ndarray:
    return _outlier_channels(w, layer)


def _zipf_logits(w: Workload, layer: int, T: int, key_tensor: int) -> np.ndarray:
    """Gumbel-perturbed log-Zipf logits: sampling k experts without replacement
    from p(rank) ~ rank^-s, with the ``zipf_masked`` lowest-ranked experts given a
    very negative (finite) logit so they never receive a token."""
    perm = _rng(w.wid, layer, _ZIPF).permutation(w.E)          # perm[rank] = expert
    ranks = np.empty(w.E, dtype=np.int64)
    ranks[perm] = np.arange(w.E)
    logp = -w.zipf_s * np.log(np.arange(1, w.E + 1, dtype=np.float64))
    base = logp[ranks].astype(np.float32)                      # [E]
    g = _rng(w.wid, layer, key_tensor).gumbel(size=(T, w.E)).astype(np.float32)
    logits = base[None, :] + g
    masked = perm[w.E - w.zipf_masked:]
    logits[:, masked] = np.float32(-1.0e30)
    return logits.astype(np.float32)


def router_logits(w: Workload, layer: int = 0, tokens: Optional[int] = None) -> np.ndarray:
    """fp32 router logits [T, E] following the workload's router law."""
    T = w.T if tokens is None else tokens
    if w.router == "zipf":
        return _zipf_logits(w, layer, T, _LOGITS)
    r = _rng(w.wid, layer, _LOGITS)
    if w.router == "uniform":
        return r.random(size=(T, w.E), dtype=np.float32)
    logits = r.standard_normal(size=(T, w.E), dtype=np.float32)
    if w.router == "normal_bias":
        bias = _rng(w.wid, layer, _BIAS).standard_normal(size=w.E, dtype=np.float32)
        logits = logits + bias[None, :]
    return logits


def expert_weights(w: Workload, layer: int = 0, experts=None, threads: Optional[int] = None):
    """bf16 bits of the gated expert weights, PyTorch [out, in] layout.

    Returns (w13 [n, 2I, H], w2 [n, H, I]) for the requested experts (all by
    default).  Rows [0, I) of w13 are the gate projection, rows [I, 2I) the up
    projection.  Each expert has its own stream, so experts can be drawn in
    parallel and independently.
    """
    ex = list(range(w.E)) if experts is None else list(experts)
    wid = w.weight_wid
    w13 = np.empty((len(ex), 2 * w.I, w.H), dtype=np.uint16)
    w2 = np.empty((len(ex), w.H, w.I), dtype=np.uint16)

    def one(i):
        e = ex[i]
        w13[i] = _normal_bf16((2 * w.I, w.H), w.weight_std, _rng(wid, layer, _W13, e))
        w2[i] = _normal_bf16((w.H, w.I), w.weight_std, _rng(wid, layer, _W2, e))

    n = threads or min(16, os.cpu_count() or 1)
    if n > 1 and len(ex) > 1:
        with ThreadPoolExecutor(n) as pool:
            list(pool.map(one, range(len(ex))))
    else:
        for i in range(len(ex)):
            one(i)
    return w13, w2


def calibration_batch(w: Workload, layer: int = 0):
    """Outlier-free calibration batch for the per-expert activation scales.

    Returns (x bf16 bits [Tc, H] ~ N(0,1), router logits fp32 [Tc, E]).  The
    router law is the workload's, except that skewed routers (bias, Zipf) are
    replaced by the unbiased N(0,1) router so that every expert slot receives
    calibration rows.
    """
    wid = w.weight_wid
    x = _normal_bf16((w.calib_tokens, w.H), 1.0, _rng(wid, layer, _CAL_X))
    r = _rng(wid, layer, _CAL_LOGITS)
    if w.router == "uniform":
        logits = r.random(size=(w.calib_tokens, w.E), dtype=np.float32)
    else:
        logits = r.standard_normal(size=(w.calib_tokens, w.E), dtype=np.float32)
    return x, logits


def bad_scale_slots(w: Workload, n_bad: int = 3):
    """Seeded corrupt expert slots for the load-time scale check.

    Returns a list of (projection, expert, kind) with projection in
    {"w13", "w2"} and kind in {"nan", "unwritten_garbage", "unwritten_neg"}:
    a NaN value, an unwritten slot whose stale bits look like a valid positive
    float, and an unwritten slot whose stale bits are -inf.
    """
    r = _rng(w.wid, 0, _BAD)
    experts = r.choice(w.E, size=n_bad, replace=False)
    projs = ["w13", "w2", "w13"]
    kinds = ["nan", "unwritten_garbage", "unwritten_neg"]
    return [(projs[i % 3], int(experts[i]), kinds[i % 3]) for i in range(n_bad)]
