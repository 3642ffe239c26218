"""Helpers shared by the oracle pins (CPU only): a token-major restatement of
the W4A4 layer with its scalings written out, and a tiny layer whose two
projections have clearly different global scales."""
import math

import numpy as np

from oracle import formats as F
import synthetic as S


def token_major_w4a4(layer, x, logits, k, res, quant, dequant, swap_alpha=False,
                      a2_with_a1_scale=False):
    """The W4A4 layer per token, without permutation or grouping, written from
    the page's definitions ("NVFP4" runtime figure: SFScaleVal is the
    reciprocal of the expert's FP32 input_scale, and the GEMM output scaling
    folds in the activation input_scale and the weight_scale_2 of the same
    projection; "矩阵融合": w13 rows [0, I) gate, [I, 2I) up, then
    act(gate) x up, w2, and the routing-weight sum).  Routing comes from
    Python's ``sorted`` and ``math.exp``.  The two keyword switches plant the
    mistakes the pin must catch."""
    T, H = x.shape
    E, I = layer.E, layer.I
    s13 = layer.w13_input_scale.astype(np.float32)
    s2 = layer.w2_input_scale.astype(np.float32)
    out = S.bf16_bits_to_f32(res).astype(np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        sel = [float(logits[t, e]) for e in order]
        ex = [math.exp(v - sel[0]) for v in sel]
        for j, e in enumerate(order):
            wt = ex[j] / sum(ex)
            alpha13 = float(s13[e]) * float(layer.w13s2[e])        # w13_input_scale x w13 scale_2
            alpha2 = float(s2[e]) * float(layer.w2s2[e])           # w2_input_scale x w2 scale_2
            if swap_alpha:
                alpha13, alpha2 = alpha2, alpha13
            gs1 = np.float32(1.0) / s13[e]
            gs2 = gs1 if a2_with_a1_scale else np.float32(1.0) / s2[e]
            ac, asf = quant(x[t:t + 1], np.array([gs1], dtype=np.float32))
            c1 = alpha13 * (dequant(ac, asf)[0] @ dequant(layer.w13c[e], layer.w13s[e]).T)
            gate, up = c1[:I], c1[I:]
            hb = F.f64_to_bf16(gate / (1.0 + np.exp(-gate)) * up)
            a2c, a2s = quant(hb[None, :], np.array([gs2], dtype=np.float32))
            c2 = alpha2 * (dequant(a2c, a2s)[0] @ dequant(layer.w2c[e], layer.w2s[e]).T)
            out[t] += wt * c2
    return out


def tiny_layer_with_distinct_scales(prepare):
    """The tiny layer with its w2 weights multiplied by 2^3 (exact in bf16), so
    the two projections' weight_scale_2 differ by 8x and their activation
    input scales differ too: a swapped alpha or a wrong SFScaleVal changes the
    output by far more than rounding."""
    w = S.WORKLOADS["tiny"]
    w13, w2 = S.expert_weights(w)
    w2 = S.f32_to_bf16_bits(S.bf16_bits_to_f32(w2) * np.float32(8.0))
    xc, lc = S.calibration_batch(w)
    layer = prepare(w13, w2, xc, lc, w.k)
    assert np.all(layer.w2s2 >= 4 * layer.w13s2)
    assert np.all(np.abs(np.log2(layer.w2_input_scale / layer.w13_input_scale)) > 0.5)
    return w, layer


def identity_w13(E, I, H, gate_val, up_val, block=16, unit_code=0x38):
    """w13 codes/scales whose dequantised gate row i is gate_val * e_i and up
    row i is up_val * e_i: unit block scales (E4M3 1.0 = 0x38 per 16 elements,
    or UE8M0 1.0 = 127 per 32 with block=32, unit_code=127) and
    weight_scale_2 = 1."""
    codes = np.zeros((E, 2 * I, H), dtype=np.uint8)
    enc = {0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    for i in range(I):
        codes[:, i, i] = enc[gate_val]
        codes[:, I + i, i] = enc[up_val]
    packed = F.pack_nibbles(codes.reshape(E * 2 * I, H)).reshape(E, 2 * I, H // 2)
    sf = np.full((E, 2 * I, H // block), unit_code, dtype=np.uint8)
    return packed, sf, np.ones(E, dtype=np.float32)
