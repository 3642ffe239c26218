"""MoE-level oracle: scale validation, router, permutation, fp64 GEMM
references, SiLU*mul, combine, calibration and the whole layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Page 3 ("Gemma 4 NVFP4 MoE 空输出"):
  * "ROOT CAUSE": the loader fills only the expert slots present in the
    checkpoint and nothing checks that every slot was written before format
    conversion takes reciprocals of w13_input_scale / w2_input_scale into
    a1_gscale / a2_gscale; stale bits become inf, NaN or arbitrary finite
    garbage.  ``validate_scales`` is that missing check.
  * "矩阵融合", MoE FFN paragraph and pipeline figure: rows are regrouped by
    routing so each expert's rows are contiguous (grouped GEMM), a1_gscale
    quantisation, grouped w13 GEMM, SiLU/mul, a2_gscale quantisation, grouped
    w2 GEMM, then token order is restored and rows are summed by routing
    weight.  Gated FFN paragraph: w13 = fused gate_up in [out, in] layout,
    activation(gate) x up.
  * "NVFP4", runtime-order figure: the GEMM output scaling folds in both FP32
    global scales (activation input_scale and weight_scale_2).
"""
from __future__ import annotations

import numpy as np

from .formats import NVFP4_RANGE, bf16_to_f32, f64_to_bf16
from .quant import dequant, quantize_bf16_rows, quantize_experts

# slot status codes (same meaning as the library's)
SLOT_OK, SLOT_UNWRITTEN, SLOT_NAN, SLOT_INF, SLOT_NONPOSITIVE, SLOT_RECIP_OVERFLOW = range(6)


# --- load-time check ----------------------------------------------------------

def validate_scales(input_scale, written=None):
    """Check every expert slot before any reciprocal is kept.

    A slot is rejected when it was not written by the loader, or its value is
    NaN, +-inf, <= 0 (including -0.0), or its fp32 reciprocal is not finite.
    Returns (ok, gscale fp32 [E] or None, status int32 [E]); gscale is only
    produced when every slot passes.
    """
    x = np.asarray(input_scale, dtype=np.float32)
    E = x.shape[0]
    status = np.zeros(E, dtype=np.int32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        for e in range(E):
            v = x[e]
            if written is not None and not written[e]:
                status[e] = SLOT_UNWRITTEN
            elif np.isnan(v):
                status[e] = SLOT_NAN
            elif np.isinf(v):
                status[e] = SLOT_INF
            elif not (v > 0):
                status[e] = SLOT_NONPOSITIVE
            elif not np.isfinite(np.float32(1.0) / v):
                status[e] = SLOT_RECIP_OVERFLOW
        if np.any(status != SLOT_OK):
            return False, None, status
        gscale = (np.float32(1.0) / x).astype(np.float32)
    return True, gscale, status


# --- router and permutation -------------------------------------------------

def route(logits: np.ndarray, k: int):
    """Top-k experts per token over fp32 logits: order by (logit descending,
    expert index ascending), keep the first k.  Routing weights are the
    softmax over the k selected logits (float64).
    Returns (ids int32 [T, k], weights float64 [T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")      # stable => ties by index
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1).astype(np.float64)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def permute(ids: np.ndarray, E: int):
    """Stable regrouping of the T*k (token, slot) pairs q = t*k + j by expert.
    Returns (expert_offsets int32 [E+1], src_pair int32 [P] (p -> q),
    inv int32 [P] (q -> p))."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    src_pair = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    inv = np.empty_like(src_pair)
    inv[src_pair] = np.arange(flat.size, dtype=np.int32)
    return offsets, src_pair, inv


def row_experts(offsets: np.ndarray) -> np.ndarray:
    E = offsets.size - 1
    return np.repeat(np.arange(E, dtype=np.int64), np.diff(offsets))


# --- GEMM references (fp64 over dequantised operands) -------------------------

def grouped_gemm_ref(a_codes, a_sf, offsets, w_codes, w_sf, alpha, rows=None):
    """C[p, n] = alpha[e] * sum_k deqA[p, k] * deqW[e][n, k] for the rows p of
    expert e (float64).  ``rows`` restricts the output to selected rows."""
    E = offsets.size - 1
    P = int(offsets[-1])
    N = w_codes.shape[1]
    sel = np.arange(P) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((sel.size, N), dtype=np.float64)
    rexp = row_experts(offsets)[sel] if P else np.zeros(0, dtype=np.int64)
    for e in range(E):
        m = np.nonzero(rexp == e)[0]
        if m.size == 0:
            continue
        A = dequant(a_codes[sel[m]], a_sf[sel[m]])
        W = dequant(w_codes[e], w_sf[e])
        out[m] = np.float64(alpha[e]) * (A @ W.T)
    return out


def grouped_gemm_w16_ref(a, offsets, w_codes, w_sf, alpha, rows=None):
    """Weight-only grouped GEMM (page 3, "Kernel Backend": the MARLIN backend
    runs W4A16 and consumes no activation input_scale): C[p, n] = alpha[e] *
    sum_k A[p, k] * deqW[e][n, k] for the rows p of expert e, with A the
    16-bit activations as real values (float64)."""
    a = np.asarray(a, dtype=np.float64)
    E = offsets.size - 1
    P = int(offsets[-1])
    N = w_codes.shape[1]
    sel = np.arange(P) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((sel.size, N), dtype=np.float64)
    rexp = row_experts(offsets)[sel] if P else np.zeros(0, dtype=np.int64)
    for e in range(E):
        m = np.nonzero(rexp == e)[0]
        if m.size == 0:
            continue
        W = dequant(w_codes[e], w_sf[e])
        out[m] = np.float64(alpha[e]) * (a[sel[m]] @ W.T)
    return out


def silu_mul(c1: np.ndarray, I: int) -> np.ndarray:
    """h = silu(gate) * up, gate = columns [0, I), up = columns [I, 2I);
    silu(z) = z / (1 + exp(-z))."""
    g = c1[:, :I]
    u = c1[:, I:2 * I]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def combine_ref(c2, w, inv, T, k, residual_f32=None):
    """out[t] = residual[t] + sum_j w[t, j] * C2[inv[t*k + j]] (float64)."""
    c2 = np.asarray(c2, dtype=np.float64)
    out = np.zeros((T, c2.shape[1]), dtype=np.float64)
    invm = np.asarray(inv).reshape(T, k)
    for j in range(k):
        out += np.asarray(w, dtype=np.float64)[:, j:j + 1] * c2[invm[:, j]]
    if residual_f32 is not None:
        out += np.asarray(residual_f32, dtype=np.float64)
    return out


# --- weights and calibration (harness side of the checkpoint) ----------------

def fl32_div_range(amax) -> np.ndarray:
    """fp32 global scale = fl32(amax / 2688) (headroom factor 1)."""
    return (np.asarray(amax, dtype=np.float32) / np.float32(NVFP4_RANGE)).astype(np.float32)


def quantize_weight(w_bits: np.ndarray):
    """Static NVFP4 quantisation of one expert weight [N, K] (bf16 bits):
    weight_scale_2 = fl32(amax / 2688); codes and E4M3 scales with
    SFScaleVal = fl32(1 / weight_scale_2).  Returns (codes, sf, scale2)."""
    amax = np.abs(bf16_to_f32(w_bits)).max()
    scale2 = fl32_div_range(amax)
    gs = np.float32(1.0) / scale2
    codes, sf = quantize_bf16_rows(w_bits, np.full(w_bits.shape[0], gs, dtype=np.float32))
    return codes, sf, np.float32(scale2)


def quantize_weights(w_bits: np.ndarray, threads: int = 8):
    """All experts [E, N, K] -> (codes [E,N,K/2], sf [E,N,K/16], scale2 [E])."""
    from concurrent.futures import ThreadPoolExecutor
    E, N, K = w_bits.shape
    codes = np.empty((E, N, K // 2), dtype=np.uint8)
    sf = np.empty((E, N, K // 16), dtype=np.uint8)
    s2 = np.empty(E, dtype=np.float32)

    def one(e):
        codes[e], sf[e], s2[e] = quantize_weight(w_bits[e])

    with ThreadPoolExecutor(max(1, threads)) as pool:
        list(pool.map(one, range(E)))
    return codes, sf, s2


def dequant_weight(codes, sf, scale2) -> np.ndarray:
    """Real-valued weight [N, K] = E2M1 * E4M3 * weight_scale_2 (float64)."""
    return dequant(codes, sf) * np.float64(scale2)


def calibrate_input_scale(x_cal_bits, logits_cal, k, E):
    """w13 activation scale only: fl32(amax|x| / 2688) over the calibration rows
    routed to each expert; experts without rows stay unwritten (NaN, written 0)."""
    ids, _ = route(logits_cal, k)
    x = bf16_to_f32(x_cal_bits)
    s13 = np.full(E, np.nan, dtype=np.float32)
    written = np.zeros(E, dtype=np.uint8)
    for e in range(E):
        t = np.nonzero((ids == e).any(axis=1))[0]
        if t.size:
            s13[e] = fl32_div_range(np.abs(x[t]).max())
            written[e] = 1
    return s13, written


def calibrate(x_cal_bits, logits_cal, k, w13c, w13s, w13s2, w2c, w2s, w2s2):
    """Per-expert activation global scales from a calibration batch.

    The batch is routed with the real router; for each expert, over the rows
    routed to it: w13_input_scale = fl32(amax|x| / 2688) and
    w2_input_scale = fl32(fl32(amax|h|) / 2688), where h = silu(gate)*up is
    computed in float64 from the dequantised weights without activation
    quantisation.  An expert that receives no calibration row is left
    unwritten (written = 0), as the exporter does on the page.
    Returns (w13_input_scale, w2_input_scale, written) with unwritten slots NaN.
    """
    E = w13c.shape[0]
    I = w2c.shape[2] * 2
    ids, _ = route(logits_cal, k)
    x = bf16_to_f32(x_cal_bits).astype(np.float64)
    s13 = np.full(E, np.nan, dtype=np.float32)
    s2 = np.full(E, np.nan, dtype=np.float32)
    written = np.zeros(E, dtype=np.uint8)
    for e in range(E):
        t = np.nonzero((ids == e).any(axis=1))[0]
        if t.size == 0:
            continue
        xe = x[t]
        s13[e] = fl32_div_range(np.float32(np.abs(xe).max()))
        W13 = dequant_weight(w13c[e], w13s[e], w13s2[e])
        h = silu_mul(xe @ W13.T, I)
        s2[e] = fl32_div_range(np.float32(np.abs(h).max()))
        written[e] = 1
    return s13, s2, written


class Layer:
    """One prepared MoE layer, as the checkpoint would hold it."""

    def __init__(self, w13c, w13s, w13s2, w2c, w2s, w2s2, s13, s2, written13, written2):
        self.w13c, self.w13s, self.w13s2 = w13c, w13s, w13s2
        self.w2c, self.w2s, self.w2s2 = w2c, w2s, w2s2
        self.w13_input_scale, self.w2_input_scale = s13, s2
        self.written13, self.written2 = written13, written2
        self.E = w13c.shape[0]
        self.I = w13c.shape[1] // 2
        self.H = w13c.shape[2] * 2

    @property
    def alpha1(self):
        return self.w13_input_scale.astype(np.float64) * self.w13s2.astype(np.float64)

    @property
    def alpha2(self):
        return self.w2_input_scale.astype(np.float64) * self.w2s2.astype(np.float64)


def prepare_layer(w13_bits, w2_bits, x_cal_bits, logits_cal, k, threads=8) -> Layer:
    w13c, w13s, w13s2 = quantize_weights(w13_bits, threads)
    w2c, w2s, w2s2 = quantize_weights(w2_bits, threads)
    s13, s2, wr = calibrate(x_cal_bits, logits_cal, k, w13c, w13s, w13s2, w2c, w2s, w2s2)
    return Layer(w13c, w13s, w13s2, w2c, w2s, w2s2, s13, s2, wr, wr.copy())


# --- the whole layer ----------------------------------------------------------

def layer_forward_w4a16(layer: Layer, x_bits, logits, k, residual_bits=None, h_from=None):
    """The weight-only (W4A16) forward of one MoE layer (page 3, "Kernel
    Backend" / "本案例：CUTLASS 与 Marlin": the MARLIN backend executes W4A16 and
    sets the activation scale to None).  Activations stay bf16; the expert
    weights are the same NVFP4 checkpoint; the GEMM scaling is the weight's
    weight_scale_2 alone.  The activation input scales are never read.

        C1 = w13_weight_scale_2[e] * x[token(p)] . deqW13[e]^T
        h  = bf16(silu(C1[:, :I]) * C1[:, I:])
        C2 = w2_weight_scale_2[e] * h . deqW2[e]^T
        out[t] = bf16(residual[t] + sum_j w[t, j] * C2[inv[t*k + j]])

    ``h_from`` replaces the oracle's own h (bf16 bits [P, I]) by a given one
    (the GEMM2 reference over given operands).  Returns a dict with ids, w,
    offsets, src_pair, inv, c1, h_bits, c2, out_f64, out_bf16."""
    T = x_bits.shape[0]
    E, I = layer.E, layer.I
    ids, w = route(logits, k)
    offsets, src_pair, inv = permute(ids, E)
    xp = bf16_to_f32(np.asarray(x_bits)[src_pair // k])
    c1 = grouped_gemm_w16_ref(xp, offsets, layer.w13c, layer.w13s, layer.w13s2)
    h_bits = f64_to_bf16(silu_mul(c1, I))
    hin = bf16_to_f32(h_bits if h_from is None else h_from)
    c2 = grouped_gemm_w16_ref(hin, offsets, layer.w2c, layer.w2s, layer.w2s2)
    res = None if residual_bits is None else bf16_to_f32(residual_bits)
    out = combine_ref(c2, w, inv, T, k, res)
    return dict(ids=ids, w=w, offsets=offsets, src_pair=src_pair, inv=inv, c1=c1,
                h_bits=h_bits, c2=c2, out_f64=out, out_bf16=f64_to_bf16(out))


def layer_forward(layer: Layer, x_bits, logits, k, residual_bits=None, a2_from=None):
    """Independent end-to-end forward of one MoE layer.

    Returns a dict with every intermediate: ids, w, offsets, src_pair, inv,
    a1 (codes, sf), c1 (fp64), h_bf16 (bits), a2 (codes, sf), c2 (fp64),
    out_f64 and out_bf16 (bits).  ``a2_from=(codes, sf)`` replaces the
    oracle's own A2 by a given one (the GEMM2 reference over given operands).
    """
    T = x_bits.shape[0]
    E, I = layer.E, layer.I
    ok1, a1_gscale, _ = validate_scales(layer.w13_input_scale, layer.written13)
    ok2, a2_gscale, _ = validate_scales(layer.w2_input_scale, layer.written2)
    if not (ok1 and ok2):
        raise ValueError("layer has invalid activation scales")
    ids, w = route(logits, k)
    offsets, src_pair, inv = permute(ids, E)
    rexp = row_experts(offsets)
    xp = np.asarray(x_bits)[src_pair // k]
    a1c, a1s = quantize_experts(xp, rexp, a1_gscale)
    c1 = grouped_gemm_ref(a1c, a1s, offsets, layer.w13c, layer.w13s, layer.alpha1)
    h = silu_mul(c1, I)
    h_bits = f64_to_bf16(h)
    if a2_from is None:
        a2c, a2s = quantize_experts(h_bits, rexp, a2_gscale)
    else:
        a2c, a2s = a2_from
    c2 = grouped_gemm_ref(a2c, a2s, offsets, layer.w2c, layer.w2s, layer.alpha2)
    res = None if residual_bits is None else bf16_to_f32(residual_bits)
    out = combine_ref(c2, w, inv, T, k, res)
    return dict(ids=ids, w=w, offsets=offsets, src_pair=src_pair, inv=inv,
                a1=(a1c, a1s), c1=c1, h_bits=h_bits, a2=(a2c, a2s), c2=c2,
                out_f64=out, out_bf16=f64_to_bf16(out), a1_gscale=a1_gscale,
                a2_gscale=a2_gscale)
