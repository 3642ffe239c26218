"""Pins for the UE8M0 (MX-style) variant of the oracle (CPU only).

Pinned by: the UE8M0 codec at every power of two and its neighbours, the
minimality of the chosen scale checked by brute force over all 254 codes,
the scalar exact encoder, reduction to the (independently pinned) E4M3 mode
when the block-scale value is a power of two inside the E4M3 range, a triple
loop for the GEMM, and a token-major definition of the layer.
"""
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M
from oracle import mx as X
from oracle import quant as Q
import synthetic as S

from pin_helpers import identity_w13, token_major_w4a4, tiny_layer_with_distinct_scales


def _f32(v):
    return np.float32(v)


def test_ue8m0_codec_at_powers_of_two_and_neighbours():
    for code in range(1, 255):
        p = _f32(math.ldexp(1.0, code - 127))
        assert X.ue8m0_encode_exact(p) == code
        up = np.nextafter(p, _f32(np.inf), dtype=np.float32)
        dn = np.nextafter(p, _f32(0), dtype=np.float32)
        assert X.ue8m0_encode_exact(up) == min(code + 1, 254)
        if code > 1:
            assert X.ue8m0_encode_exact(dn) == code
        assert float(X.ue8m0_decode(code)) == math.ldexp(1.0, code - 127)
    # below the smallest normal, zero, huge, inf, NaN
    assert X.ue8m0_encode_exact(0.0) == 1
    assert X.ue8m0_encode_exact(_f32(1e-45)) == 1
    assert X.ue8m0_encode_exact(np.finfo(np.float32).max) == 254
    assert X.ue8m0_encode_exact(np.inf) == 254
    assert X.ue8m0_encode_exact(np.nan) == 254


def test_ue8m0_vector_encoder_matches_scalar_and_brute_force_minimality():
    rng = np.random.default_rng(3)
    s = np.concatenate([
        (rng.random(3000) * 2.0 ** rng.integers(-140, 128, 3000)).astype(np.float32),
        np.array([0, 1, 2, 3, 0.75, 448, 1e-39, np.inf, np.nan], dtype=np.float32)])
    vec = X.ue8m0_encode(s)
    powers = [math.ldexp(1.0, c - 127) for c in range(1, 255)]
    for v, c in zip(s, vec):
        assert c == X.ue8m0_encode_exact(v)
        if np.isfinite(v):
            # brute force: the first code whose power of two is >= s, else 254
            want = next((i + 1 for i, p in enumerate(powers) if p >= float(v)), 254)
            assert c == want, (v, c, want)


def test_block_never_saturates_unless_the_scale_clamps():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((200, 64)) * 10.0 ** rng.uniform(-20, 20, (200, 1))).astype(np.float32)
    gs = (10.0 ** rng.uniform(-3, 3, 200)).astype(np.float32)
    codes, sf = X.quantize_f32_rows(x, gs)
    assert np.all((sf > 1) & (sf < 254))
    scale = X.ue8m0_decode(sf).reshape(200, 2, 1)
    v = x.reshape(200, 2, 32).astype(np.float64) * gs.reshape(200, 1, 1) / scale
    assert np.abs(v).max() <= 6.0 * (1 + 2 ** -20)
    # and the scale is the smallest such power of two for each block: halving
    # it would push the largest element past 6 (up to the fp32 rounding of s)
    amax = np.abs(x.reshape(200, 2, 32)).max(axis=-1).astype(np.float64)
    assert np.all(amax * gs.reshape(200, 1) / (scale[..., 0] / 2) > 6.0 * (1 - 2 ** -20))


def test_scalar_exact_block_matches_vectorised():
    rng = np.random.default_rng(5)
    for t in range(200):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        if t % 7 == 0:
            x[rng.integers(0, 32, 4)] = 0.0
        gs = np.float32(10.0 ** rng.uniform(-2, 3))
        sf, codes = X.quant_block_exact(x, gs)
        vc, vs = X.quantize_f32_rows(x[None, :], np.array([gs], dtype=np.float32))
        assert vs[0, 0] == sf
        assert F.unpack_nibbles(vc)[0].tolist() == codes


def test_reduces_to_e4m3_mode_when_the_scale_is_a_power_of_two():
    # blocks whose two 16-halves share amax = 6 * 2^j (gs = 1): the block-scale
    # value is 2^j, exact in both encodings, so both modes normalise by the
    # same power of two and must produce identical element codes
    rng = np.random.default_rng(6)
    rows = []
    for j in range(-8, 8):
        x = rng.uniform(-1, 1, 32) * 6.0 * 2.0 ** j
        x[3], x[20] = 6.0 * 2.0 ** j, -6.0 * 2.0 ** j
        rows.append(x)
    x = np.array(rows, dtype=np.float32)
    ones = np.ones(len(rows), dtype=np.float32)
    c_mx, s_mx = X.quantize_f32_rows(x, ones)
    c_nv, s_nv = Q.quantize_f32_rows(x, ones)
    assert np.array_equal(c_mx, c_nv)
    assert np.array_equal(X.ue8m0_decode(s_mx), F.e4m3_decode_vec(s_nv[:, 0::2]))


def test_dequant_values():
    packed = np.array([[0x71, 0xF9] + [0] * 14], dtype=np.uint8)     # codes 1,7,9,15,0...
    sf = np.array([[127 + 3]], dtype=np.uint8)
    d = X.dequant(packed, sf)
    assert d[0, :4].tolist() == [0.5 * 8, 6.0 * 8, -0.5 * 8, -6.0 * 8]
    assert np.all(d[0, 4:] == 0)


def test_grouped_gemm_brute_force():
    rng = np.random.default_rng(7)
    E, N, K = 3, 4, 64
    offsets = np.array([0, 2, 2, 5], dtype=np.int32)
    ac = rng.integers(0, 256, (5, K // 2)).astype(np.uint8)
    asf = rng.integers(110, 140, (5, K // 32)).astype(np.uint8)
    wc = rng.integers(0, 256, (E, N, K // 2)).astype(np.uint8)
    ws = rng.integers(110, 140, (E, N, K // 32)).astype(np.uint8)
    alpha = np.array([0.5, 3.0, -1.25])
    got = X.grouped_gemm_ref(ac, asf, offsets, wc, ws, alpha)

    def val(codes, sf, r, kk):
        b = int(codes[r, kk // 2])
        c = b & 0xF if kk % 2 == 0 else b >> 4
        return F.e2m1_decode(c) * math.ldexp(1.0, int(sf[r, kk // 32]) - 127)

    for p in range(5):
        e = 0 if p < 2 else 2
        for n in range(N):
            acc = sum(val(ac, asf, p, kk) * val(wc[e], ws[e], n, kk) for kk in range(K))
            assert got[p, n] == pytest.approx(alpha[e] * acc, rel=1e-13, abs=1e-300)
    assert np.array_equal(X.grouped_gemm_ref(ac, asf, offsets, wc, ws, alpha, rows=[4, 0]),
                          got[[4, 0]])


def test_mx_layer_token_major_and_close_to_unquantised():
    w = S.WORKLOADS["tiny"]
    w13, w2 = S.expert_weights(w)
    xc, lc = S.calibration_batch(w)
    layer = X.prepare_layer(w13, w2, xc, lc, w.k)
    assert layer.w13s.shape == (w.E, 2 * w.I, w.H // 32)
    x = S.activations(w)
    logits = S.router_logits(w)
    r = X.layer_forward(layer, x, logits, w.k)
    ids, wts = M.route(logits, w.k)
    # token-major definition over the same quantised operands, with the
    # scalings written out (alpha = input_scale x weight_scale_2 of the same
    # projection, SFScaleVal = fl32(1 / input_scale)): pinned on a layer whose
    # w2 weights are 2^3 larger, so a swapped alpha or a wrong SFScaleVal
    # cannot pass
    w_d, layer_d = tiny_layer_with_distinct_scales(X.prepare_layer)
    rng = np.random.default_rng(34)
    res = S.f32_to_bf16_bits(rng.standard_normal((w.T, w.H)).astype(np.float32))
    r_d = X.layer_forward(layer_d, x, logits, w.k, residual_bits=res)
    ref_d = token_major_w4a4(layer_d, x, logits, w.k, res, X.quantize_bf16_rows, X.dequant)
    assert np.allclose(r_d["out_f64"], ref_d, rtol=1e-12, atol=1e-12)
    base = S.bf16_bits_to_f32(res).astype(np.float64)
    for kw in (dict(swap_alpha=True), dict(a2_with_a1_scale=True)):
        wrong = token_major_w4a4(layer_d, x, logits, w.k, res, X.quantize_bf16_rows, X.dequant,
                                 **kw)
        assert np.linalg.norm(wrong - ref_d) > 0.05 * np.linalg.norm(ref_d - base), kw
    # the MX layer tracks the unquantised fp64 layer (coarser than E4M3 scales)
    xf = S.bf16_bits_to_f32(x).astype(np.float64)
    exact = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            e = ids[t, j]
            W13 = X.dequant(layer.w13c[e], layer.w13s[e]) * np.float64(layer.w13s2[e])
            W2 = X.dequant(layer.w2c[e], layer.w2s[e]) * np.float64(layer.w2s2[e])
            h = M.silu_mul((xf[t] @ W13.T)[None, :], w.I)
            exact[t] += wts[t, j] * (h @ W2.T)[0]
    rel = np.linalg.norm(r["out_f64"] - exact) / np.linalg.norm(exact)
    assert rel < 0.3, rel
    # unwritten activation scales are refused here as in the E4M3 mode
    bad = X.LayerMX(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s, layer.w2s2,
                    layer.w13_input_scale, layer.w2_input_scale,
                    np.zeros(w.E, dtype=np.uint8), layer.written2)
    with pytest.raises(ValueError):
        X.layer_forward(bad, x, logits, w.k)


def test_mx_calibration_w2_scale_closed_form():
    """The UE8M0 layer's calibration: w2_input_scale[e] = fl32(fl32(max |h|) /
    2688) with h = silu(gate) * up of the rows routed to e; with gate = x and
    up = 2x (identity-like w13 at unit UE8M0 scales) max |h| has a closed
    form.  An expert without rows stays unwritten."""
    E, I, H, k = 3, 32, 64, 1
    w13c, w13s, w13s2 = identity_w13(E, I, H, 1.0, 2.0, block=32, unit_code=127)
    assert np.array_equal(X.dequant(w13c[0], w13s[0])[:I, :I], np.eye(I))
    w2c = np.zeros((E, H, I // 2), dtype=np.uint8)
    w2s = np.full((E, H, I // 32), 127, dtype=np.uint8)
    rng = np.random.default_rng(43)
    T = 10
    x = S.f32_to_bf16_bits((rng.standard_normal((T, H)) * 2).astype(np.float32))
    xv = S.bf16_bits_to_f32(x).astype(np.float64)
    logits = np.full((T, E), -5.0, dtype=np.float32)
    logits[np.arange(T), 2 * (np.arange(T) % 2)] = 5.0      # experts 0 and 2; 1 gets none
    s13, s2, written = X.calibrate(x, logits, k, w13c, w13s, w13s2, w2c, w2s,
                                   np.ones(E, dtype=np.float32))
    assert written.tolist() == [1, 0, 1] and np.isnan(s2[1]) and np.isnan(s13[1])
    for e in (0, 2):
        rows = xv[2 * (np.arange(T) % 2) == e]
        amax_h = max(abs(2.0 * v * v / (1.0 + math.exp(-v))) for v in rows[:, :I].reshape(-1))
        assert s2[e] == np.float32(np.float32(amax_h) / np.float32(2688.0))
        assert s13[e] == np.float32(np.float32(np.abs(rows).max()) / np.float32(2688.0))
