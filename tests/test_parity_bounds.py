"""CPU checks of the element-wise parity bounds the GPU tests apply
(tests/gpu_helpers.py): an fp32 evaluation of the same layer stages (fp32
products and sums in NumPy, then one bf16 rounding) stays inside every bound,
and an output one bf16 ulp away from the correctly rounded value does not.
This shows the bounds are neither violated by honest fp32 arithmetic nor
loose enough to accept a wrongly rounded element."""
import numpy as np
import pytest

import synthetic as S
from oracle import formats as OF
from oracle import moe as OM
from oracle import quant as OQ

from gpu_helpers import (U32, assert_correctly_rounded_bf16, bf16_half_ulp, combine_error_bound,
                         dot_error_bound, routing_weight_bound, silu_mul_error_bound,
                         weight_row_norms)


def test_half_ulp_from_the_bf16_exponent():
    v = np.array([1.0, 1.99, 2.0, 3.5, -0.75, 2.0 ** -126, 0.0])
    got = bf16_half_ulp(v)
    assert got.tolist() == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -9,
                            2.0 ** -134, 2.0 ** -134]
    # rounding to nearest bf16 never moves a value by more than that
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))
    r = OF.bf16_to_f32(OF.f64_to_bf16(x)).astype(np.float64)
    assert np.all(np.abs(r - x) <= bf16_half_ulp(x))
    # and a whole ulp step exceeds it
    assert np.all(2 * bf16_half_ulp(x) > bf16_half_ulp(x))


def _fp32_layer(layer, x_bits, logits, k, res_bits):
    """The layer's GEMMs, SiLU*mul and combine in fp32 arithmetic (NumPy
    float32 matmul and elementwise ops), with the oracle's own quantised
    operands: a stand-in for any fp32 implementation."""
    ref = OM.layer_forward(layer, x_bits, logits, k, res_bits)
    rexp = OM.row_experts(ref["offsets"])
    a1 = OQ.dequant(*ref["a1"]).astype(np.float32)
    c1 = np.zeros(ref["c1"].shape, dtype=np.float32)
    for e in range(layer.E):
        m = rexp == e
        W = OQ.dequant(layer.w13c[e], layer.w13s[e]).astype(np.float32)
        c1[m] = np.float32(layer.alpha1[e]) * (a1[m] @ W.T)
    g, u = c1[:, :layer.I], c1[:, layer.I:]
    h32 = (g * (np.float32(1) / (np.float32(1) + np.exp(-g))) * u).astype(np.float32)
    h_bits = OF.f64_to_bf16(h32.astype(np.float64))
    a2c, a2s = OQ.quantize_experts(h_bits, rexp, ref["a2_gscale"])
    a2 = OQ.dequant(a2c, a2s).astype(np.float32)
    c2 = np.zeros((a2.shape[0], layer.H), dtype=np.float32)
    for e in range(layer.E):
        m = rexp == e
        W = OQ.dequant(layer.w2c[e], layer.w2s[e]).astype(np.float32)
        c2[m] = np.float32(layer.alpha2[e]) * (a2[m] @ W.T)
    T = x_bits.shape[0]
    invm = ref["inv"].reshape(T, k)
    w32 = ref["w"].astype(np.float32)
    acc = np.zeros((T, layer.H), dtype=np.float32)
    for j in range(k):
        acc = acc + w32[:, j:j + 1] * c2[invm[:, j]]
    acc = acc + OF.bf16_to_f32(res_bits)
    return ref, rexp, c1, h_bits, (a2c, a2s), c2, w32, OF.f64_to_bf16(acc.astype(np.float64))


def test_fp32_evaluation_is_inside_every_bound():
    w = S.WORKLOADS["tiny"]
    w13, w2 = S.expert_weights(w)
    xc, lc = S.calibration_batch(w)
    layer = OM.prepare_layer(w13, w2, xc, lc, w.k)
    x = S.activations(w)
    logits = S.router_logits(w)
    rng = np.random.default_rng(9)
    res = S.f32_to_bf16_bits(rng.standard_normal(x.shape).astype(np.float32))
    ref, rexp, c1, h_bits, a2, c2, w32, out_bits = _fp32_layer(layer, x, logits, w.k, res)

    w_err = routing_weight_bound(logits, ref["ids"], ref["w"])
    assert np.all(np.abs(w32.astype(np.float64) - ref["w"]) <= w_err)
    a1_norm = np.linalg.norm(OQ.dequant(*ref["a1"]), axis=1)
    err_c1 = dot_error_bound(a1_norm, weight_row_norms(layer, "w13", OQ.dequant), layer.alpha1,
                             rexp, w.H)
    assert np.all(np.abs(c1 - ref["c1"]) <= err_c1)
    h_exact = OM.silu_mul(ref["c1"], w.I)
    err_h = silu_mul_error_bound(ref["c1"], err_c1, w.I)
    h = OF.bf16_to_f32(h_bits).astype(np.float64)
    assert_correctly_rounded_bf16(h, h_exact, err_h, "fp32 h")

    c2_ref = OM.grouped_gemm_ref(a2[0], a2[1], ref["offsets"], layer.w2c, layer.w2s, layer.alpha2)
    a2_norm = np.linalg.norm(OQ.dequant(*a2), axis=1)
    err_c2 = dot_error_bound(a2_norm, weight_row_norms(layer, "w2", OQ.dequant), layer.alpha2,
                             rexp, w.I)
    assert np.all(np.abs(c2 - c2_ref) <= err_c2)
    res_f = OF.bf16_to_f32(res)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], w.T, w.k, res_f)
    err_out = combine_error_bound(c2_ref, err_c2, ref["w"], w_err, ref["inv"], w.T, w.k, res_f)
    out = OF.bf16_to_f32(out_bits).astype(np.float64)
    assert_correctly_rounded_bf16(out, out_ref, err_out, "fp32 out")

    # the fp32 error terms are small next to half a bf16 ulp for most elements
    assert np.median(err_out / bf16_half_ulp(out_ref)) < 0.1
    assert np.median(err_h / bf16_half_ulp(h_exact)) < 0.25

    # one element moved by one bf16 ulp (away from the exact value) is caught
    for arr, exact, err, name in ((out, out_ref, err_out, "out"), (h, h_exact, err_h, "h")):
        bad = arr.copy()
        i = np.unravel_index(np.argmax(np.abs(exact) / (err + 1e-300)), arr.shape)
        step = 2 * bf16_half_ulp(bad[i])
        bad[i] += step if bad[i] >= exact[i] else -step
        with pytest.raises(AssertionError):
            assert_correctly_rounded_bf16(bad, exact, err, name)
    assert U32 == 2.0 ** -24
