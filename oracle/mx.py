"""UE8M0 (MX-style) block-scale variant of the NVFP4 pipeline (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Page 3 ("NVFP4" section, quantiser excerpt) shows the per-expert quantiser as
a template whose last parameter, UE8M0_SF, switches the block-scale encoding
to UE8M0: an unsigned 8-bit power-of-two exponent.  The pages give nothing
beyond the name.  Reading taken here (plainest one consistent with the rest
of the page):

  * the block-scale value is formed exactly as in the E4M3 mode,
    s = fl32(gs * fl32(amax / 6)), with the same per-expert SFScaleVal gs;
  * it is encoded as the smallest power of two >= s (rounding up, so no
    element of the block exceeds the E2M1 maximum after normalisation),
    code = log2(scale) + 127, clamped to [1, 254] (scales 2^-126 .. 2^127:
    every scale is a normal fp32 number; 255 would be NaN);
  * a block covers 32 consecutive elements, the MX block size and the
    granularity at which a block scale enters a scaled matrix core product;
  * normalisation and element rounding are those of the E4M3 mode:
    inv = fl32(gs / scale) clamped to FLT_MAX, code_i = E2M1(fl32(x_i * inv)).

Dequantised value: E2M1(code) * 2^(sf - 127); the real value is that times
the FP32 global scale (input_scale for activations, weight_scale_2 for
weights), so the GEMM output scaling alpha = input_scale * weight_scale_2 is
unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import (E2M1_MAX, bf16_to_f32, e2m1_decode_vec, e2m1_encode, e2m1_encode_exact,
                      f64_to_bf16, pack_nibbles)
from .moe import (combine_ref, fl32_div_range, permute, route, row_experts, silu_mul,
                  validate_scales)

BLOCK = 32
CODE_MIN, CODE_MAX = 1, 254
FLT_MAX = np.float32(np.finfo(np.float32).max)
_SIX = np.float32(E2M1_MAX)


# --- UE8M0 scale codec ----------------------------------------------------------

def ue8m0_decode(code) -> np.ndarray:
    """code -> 2^(code - 127) as float64 (exact)."""
    return np.ldexp(1.0, np.asarray(code, dtype=np.int64) - 127)


def ue8m0_encode_exact(s) -> int:
    """Smallest power of two >= s, as a UE8M0 code clamped to [1, 254].
    s = 0 (or below 2^-126) gives 1; +inf, NaN or s > 2^127 give 254."""
    s = float(s)
    if not s < math.inf:            # inf, NaN
        return CODE_MAX
    if s <= 0.0:
        return CODE_MIN
    m, e = math.frexp(s)            # s = m * 2^e, 0.5 <= m < 1
    p = e - 1 if m == 0.5 else e    # exact power of two keeps its exponent
    return int(min(max(p + 127, CODE_MIN), CODE_MAX))


def ue8m0_encode(s) -> np.ndarray:
    """Vectorised ue8m0_encode_exact over fp32 values."""
    s = np.asarray(s, dtype=np.float64)
    bad = ~(s < np.inf)
    pos = np.where(bad | (s <= 0), 1.0, s)
    m, e = np.frexp(pos)
    p = np.where(m == 0.5, e - 1, e)
    code = np.clip(p + 127, CODE_MIN, CODE_MAX)
    code = np.where(s <= 0, CODE_MIN, code)
    code = np.where(bad, CODE_MAX, code)
    return code.astype(np.uint8)


# --- quantiser --------------------------------------------------------------------

def quant_block_exact(x32, gs=1.0):
    """One 32-element block, scalar, with the exact encoders.
    Returns (UE8M0 code, [32 nibble codes])."""
    assert len(x32) == BLOCK
    gs = np.float32(gs)
    xs = [np.float32(v) for v in x32]
    with np.errstate(over="ignore", invalid="ignore"):
        amax = max(abs(v) for v in xs)
        s = np.float32(gs * np.float32(amax / _SIX))
        sf = ue8m0_encode_exact(s)
        scale = np.float32(ue8m0_decode(sf))           # a normal fp32 power of two
        inv = np.float32(gs / scale)
        if inv > FLT_MAX:
            inv = FLT_MAX
        codes = [e2m1_encode_exact(np.float32(v * inv)) for v in xs]
    return sf, codes


def quantize_f32_rows(x: np.ndarray, gs_row: np.ndarray):
    """Rows of exact fp32 values [R, K] (K % 32 == 0), SFScaleVal per row ->
    (packed codes uint8 [R, K/2], UE8M0 codes uint8 [R, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    assert K % BLOCK == 0
    gs = np.asarray(gs_row, dtype=np.float32).reshape(R, 1)
    xb = x.reshape(R, K // BLOCK, BLOCK)
    with np.errstate(over="ignore", invalid="ignore"):
        amax = np.abs(xb).max(axis=-1)
        s = (gs * (amax / _SIX)).astype(np.float32)
        sf = ue8m0_encode(s)
        scale = ue8m0_decode(sf).astype(np.float32)
        inv = np.minimum(gs / scale, FLT_MAX).astype(np.float32)
        v = (xb * inv[..., None]).astype(np.float32)
    codes = e2m1_encode(v).reshape(R, K)
    return pack_nibbles(codes), sf


def quantize_bf16_rows(x_bits: np.ndarray, gs_row: np.ndarray, chunk: int = 4096):
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    codes = np.empty((R, K // 2), dtype=np.uint8)
    sf = np.empty((R, K // BLOCK), dtype=np.uint8)
    gs_row = np.asarray(gs_row, dtype=np.float32)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        codes[r0:r1], sf[r0:r1] = quantize_f32_rows(bf16_to_f32(x_bits[r0:r1]), gs_row[r0:r1])
    return codes, sf


def quantize_experts(x_bits: np.ndarray, row_expert: np.ndarray, gscale):
    """Row r uses SFScaleVal = gscale[row_expert[r]] (1.0 when gscale is None)."""
    R = x_bits.shape[0]
    if gscale is None:
        gs = np.ones(R, dtype=np.float32)
    else:
        gs = np.asarray(gscale, dtype=np.float32)[np.asarray(row_expert, dtype=np.int64)]
    return quantize_bf16_rows(x_bits, gs)


def dequant(packed: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """float64 [R, K] = E2M1(code) * 2^(sf - 127), exact."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, Kh = packed.shape
    K = 2 * Kh
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_decode_vec(codes).reshape(R, K // BLOCK, BLOCK)
    return (vals * ue8m0_decode(sf).reshape(R, K // BLOCK, 1)).reshape(R, K)


# --- weights, GEMM, layer -----------------------------------------------------------

def quantize_weight(w_bits: np.ndarray):
    """Static quantisation of one expert weight [N, K] in the UE8M0 mode, with
    the same per-expert weight_scale_2 = fl32(amax / 2688) and SFScaleVal
    fl32(1 / weight_scale_2) as the E4M3 mode.  Returns (codes, sf, scale2)."""
    amax = np.abs(bf16_to_f32(w_bits)).max()
    scale2 = fl32_div_range(amax)
    gs = np.float32(1.0) / scale2
    codes, sf = quantize_bf16_rows(w_bits, np.full(w_bits.shape[0], gs, dtype=np.float32))
    return codes, sf, np.float32(scale2)


def quantize_weights(w_bits: np.ndarray, threads: int = 8):
    """All experts [E, N, K] -> (codes [E,N,K/2], sf [E,N,K/32], scale2 [E])."""
    from concurrent.futures import ThreadPoolExecutor
    E, N, K = w_bits.shape
    codes = np.empty((E, N, K // 2), dtype=np.uint8)
    sf = np.empty((E, N, K // BLOCK), dtype=np.uint8)
    s2 = np.empty(E, dtype=np.float32)

    def one(e):
        codes[e], sf[e], s2[e] = quantize_weight(w_bits[e])

    with ThreadPoolExecutor(max(1, threads)) as pool:
        list(pool.map(one, range(E)))
    return codes, sf, s2


def grouped_gemm_ref(a_codes, a_sf, offsets, w_codes, w_sf, alpha, rows=None):
    """C[p, n] = alpha[e] * sum_k deqA[p, k] * deqW[e][n, k] for the rows of
    expert e, both operands in the UE8M0 format (float64)."""
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


def calibrate(x_cal_bits, logits_cal, k, w13c, w13s, w13s2, w2c, w2s, w2s2):
    """Activation global scales as in the E4M3 mode (fl32(amax / 2688) of x
    and of the unquantised-activation h per expert over the calibration rows
    routed to it), with the UE8M0 weights.  Unwritten experts stay NaN."""
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
        W13 = dequant(w13c[e], w13s[e]) * np.float64(w13s2[e])
        h = silu_mul(xe @ W13.T, I)
        s2[e] = fl32_div_range(np.float32(np.abs(h).max()))
        written[e] = 1
    return s13, s2, written


class LayerMX:
    """One MoE layer in the UE8M0 format (same fields as the E4M3 layer, with
    block scales [.., K/32])."""

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


def prepare_layer(w13_bits, w2_bits, x_cal_bits, logits_cal, k, threads=8) -> LayerMX:
    w13c, w13s, w13s2 = quantize_weights(w13_bits, threads)
    w2c, w2s, w2s2 = quantize_weights(w2_bits, threads)
    s13, s2, wr = calibrate(x_cal_bits, logits_cal, k, w13c, w13s, w13s2, w2c, w2s, w2s2)
    return LayerMX(w13c, w13s, w13s2, w2c, w2s, w2s2, s13, s2, wr, wr.copy())


def layer_forward(layer: LayerMX, x_bits, logits, k, residual_bits=None, a2_from=None):
    """The W4A4 layer of page 3 ("矩阵融合" pipeline figure) with every NVFP4
    quantisation step in the UE8M0 mode: route, permute, quantise x with
    a1_gscale, grouped w13 GEMM (alpha1), h = bf16(silu(gate) * up), quantise h
    with a2_gscale, grouped w2 GEMM (alpha2), combine.  ``a2_from`` replaces
    the oracle's A2 by a given (codes, sf) pair.  The activation scales must
    pass the load-time check, which also yields a*_gscale."""
    T = x_bits.shape[0]
    E, I = layer.E, layer.I
    ok1, g1, _ = validate_scales(layer.w13_input_scale, layer.written13)
    ok2, g2, _ = validate_scales(layer.w2_input_scale, layer.written2)
    if not (ok1 and ok2):
        raise ValueError("layer has invalid activation scales")
    ids, w = route(logits, k)
    offsets, src_pair, inv = permute(ids, E)
    rexp = row_experts(offsets)
    a1 = quantize_experts(np.asarray(x_bits)[src_pair // k], rexp, g1)
    c1 = grouped_gemm_ref(a1[0], a1[1], offsets, layer.w13c, layer.w13s, layer.alpha1)
    h_bits = f64_to_bf16(silu_mul(c1, I))
    a2 = quantize_experts(h_bits, rexp, g2) if a2_from is None else a2_from
    c2 = grouped_gemm_ref(a2[0], a2[1], offsets, layer.w2c, layer.w2s, layer.alpha2)
    res = None if residual_bits is None else bf16_to_f32(residual_bits)
    out = combine_ref(c2, w, inv, T, k, res)
    return dict(ids=ids, w=w, offsets=offsets, src_pair=src_pair, inv=inv, a1=a1, c1=c1,
                h_bits=h_bits, a2=a2, a1_gscale=g1, a2_gscale=g2, c2=c2, out_f64=out,
                out_bf16=f64_to_bf16(out))
