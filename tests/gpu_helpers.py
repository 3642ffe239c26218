"""Shared pieces of the GPU parity tests: oracle-prepared layers (cached per
process), device upload, and the per-row relative-L2 metric.

Expected values always come from ``oracle/`` on the seeded inputs of
``synthetic/``; the HIP path only produces the values under test.
"""
from __future__ import annotations

import functools
import time

import numpy as np

import synthetic as S
from oracle import formats as OF
from oracle import moe as OM
from oracle import mx as OX
from oracle import quant as OQ

# Per-row relative L2 bound for expert-GEMM outputs and the layer output,
# versus the fp64 reference over the same dequantised operands.
REL_L2_TOL = 2e-3


def rel_l2_rows(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return out


def bf16_f64(bits):
    return OF.bf16_to_f32(bits).astype(np.float64)


U32 = 2.0 ** -24          # unit roundoff of fp32 (round to nearest)


def bf16_half_ulp(v):
    """Half the spacing of bf16 numbers at |v|.  bf16 keeps 8 significant
    bits, so in the binade [2^e, 2^(e+1)) the spacing is 2^(e-7) and half of
    it 2^(e-8); below 2^-126 the spacing stays 2^-133."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def assert_correctly_rounded_bf16(got, exact, err32, label):
    """Every bf16 element is the nearest bf16 number to a value that lies
    within err32 of the exact (fp64) one, where err32 bounds the GPU's fp32
    error before its single rounding to bf16:
        |got - exact| <= half_ulp(|exact| + err32) + err32."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    err32 = np.asarray(err32, dtype=np.float64)
    bound = bf16_half_ulp(np.abs(exact) + err32) + err32
    err = np.abs(got - exact)
    bad = err > bound
    assert not bad.any(), (label, "elements beyond half a bf16 ulp + the fp32 error bound",
                           int(bad.sum()), float((err / np.maximum(bound, 1e-300)).max()))


def dot_error_bound(a_norm, w_norm, alpha, row_expert, K):
    """Bound on the fp32 error of the GPU's grouped-GEMM outputs
    C[p, n] = alpha[e] * sum_k A[p, k] W[e][n, k] (exact operands, fp32
    accumulation): |fl(C) - C| <= gamma * u * |alpha| * sum_k |A W| with
    gamma = K/16 + 64 (one rounding per accumulation step of a 16-deep matrix
    instruction, plus a budget of 64 for the instruction's internal sum and the
    product by alpha; a 64-deep instruction needs fewer steps), and
    sum_k |A W| <= ||A[p]|| ||W[e][n]|| (Cauchy-Schwarz).  a_norm [P],
    w_norm [E, N] -> [P, N]."""
    gamma = K / 16 + 64
    e = np.asarray(row_expert, dtype=np.int64)
    scale = gamma * U32 * np.abs(np.asarray(alpha, dtype=np.float64))[e] * a_norm
    return scale[:, None] * w_norm[e]


def weight_row_norms(layer, proj: str, dequant, experts=None):
    """||dequantised W[e][n]|| for every weight row n of the given experts
    (all by default), as an [E, N] array; rows of experts not asked for are
    NaN, so a bound built from them rejects everything.  Cached on the layer
    per expert."""
    codes, sf = (layer.w13c, layer.w13s) if proj == "w13" else (layer.w2c, layer.w2s)
    key = f"_norms_{proj}"
    if not hasattr(layer, key):
        setattr(layer, key, {})
    cache = getattr(layer, key)
    want = range(codes.shape[0]) if experts is None else [int(e) for e in experts]
    for e in want:
        if e not in cache:
            cache[e] = np.linalg.norm(dequant(codes[e], sf[e]), axis=1)
    out = np.full((codes.shape[0], codes.shape[1]), np.nan)
    for e, v in cache.items():
        out[e] = v
    return out


def routing_weight_bound(logits, ids, w_ref):
    """Bound on the GPU's fp32 softmax weights against the fp64 ones.  With
    d_j = l_j - l_max (rounded once in fp32), exp correct to an ulp, k - 1
    additions and one division, the relative error of weight j is at most
    (|d_j| + max_i |d_i| + k + 8) u."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64),
                             np.asarray(ids, dtype=np.int64), axis=1)
    d = np.abs(sel - sel[:, :1])
    k = sel.shape[1]
    return np.abs(w_ref) * U32 * (d + d.max(axis=1, keepdims=True) + k + 8)


def silu_mul_error_bound(c1_exact, err_c1, I):
    """Bound on the fp32 error of h = silu(gate) * up computed from fp32 C1
    values that are each within err_c1 of c1_exact: |dsilu/dg| <= 1.1
    carries the gate's error, |silu(g)| the up's, and the fp32 evaluation
    itself (exp of an argument rounded to fp32, a reciprocal and two
    products) adds (|g| + 16) u of |h|."""
    g, u = c1_exact[:, :I], c1_exact[:, I:2 * I]
    dg, du = err_c1[:, :I], err_c1[:, I:2 * I]
    with np.errstate(over="ignore"):
        s = g / (1.0 + np.exp(-g))
    return 1.1 * np.abs(u) * dg + np.abs(s) * du + (np.abs(g) + 16.0) * U32 * np.abs(s * u)


def combine_error_bound(c2_exact, err_c2, w_ref, w_err, inv, T, k, residual_f32=None):
    """Bound on the fp32 error of out[t] = residual[t] + sum_j w[t,j] C2[q]
    before its rounding to bf16: the C2 rows' own errors weighted, the
    routing weights' errors times |C2|, and k + 2 roundings of the running
    sum."""
    invm = np.asarray(inv).reshape(T, k)
    err = np.zeros((T, c2_exact.shape[1]))
    mag = np.zeros_like(err) if residual_f32 is None else np.abs(residual_f32).astype(np.float64)
    for j in range(k):
        rows = invm[:, j]
        a = np.abs(c2_exact[rows])
        err += np.abs(w_ref[:, j:j + 1]) * err_c2[rows] + w_err[:, j:j + 1] * a
        mag += np.abs(w_ref[:, j:j + 1]) * a
    return err + (k + 2) * U32 * mag


@functools.lru_cache(maxsize=4)
def oracle_layer(name: str, layer: int = 0) -> OM.Layer:
    """The oracle's NVFP4 layer (weights quantised and scales calibrated by
    the oracle) for a workload; decode and prefill share one layer."""
    w = S.WORKLOADS[name]
    key_name = "decode" if name == "prefill" else name
    return _prepare(key_name, layer)


@functools.lru_cache(maxsize=2)
def oracle_layer_mx(name: str, layer: int = 0) -> OX.LayerMX:
    """The oracle's layer in the UE8M0 mode (weights quantised and scales
    calibrated by the oracle); decode and prefill share one layer."""
    key_name = "decode" if name == "prefill" else name
    w = S.WORKLOADS[key_name]
    t0 = time.time()
    progress(f"oracle: drawing {key_name} layer {layer} weights (UE8M0 mode)")
    w13, w2 = S.expert_weights(w, layer=layer)
    xc, lc = S.calibration_batch(w, layer=layer)
    out = OX.prepare_layer(w13, w2, xc, lc, w.k, threads=16)
    progress(f"oracle: UE8M0 {key_name} layer {layer} ready in {time.time() - t0:.1f}s")
    return out


@functools.lru_cache(maxsize=4)
def _prepare(name: str, layer: int) -> OM.Layer:
    w = S.WORKLOADS[name]
    t0 = time.time()
    progress(f"oracle: drawing {name} layer {layer} weights")
    w13, w2 = S.expert_weights(w, layer=layer)
    xc, lc = S.calibration_batch(w, layer=layer)
    progress(f"oracle: quantising and calibrating {name} layer {layer}")
    out = OM.prepare_layer(w13, w2, xc, lc, w.k, threads=16)
    progress(f"oracle: {name} layer {layer} ready in {time.time() - t0:.1f}s")
    return out


def progress(msg):
    print(f"[progress] {msg}", flush=True)


def device_layer(layer: OM.Layer):
    from nvfp4_w4a4_expert_amd import moe as M
    return M.NVFP4MoELayer(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s,
                           layer.w2s2, layer.w13_input_scale, layer.w2_input_scale,
                           layer.written13, layer.written2, device="cuda")


def device_layer_mx(layer: OX.LayerMX):
    from nvfp4_w4a4_expert_amd import moe as M
    return M.NVFP4MXMoELayer(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s,
                             layer.w2s2, layer.w13_input_scale, layer.w2_input_scale,
                             layer.written13, layer.written2, device="cuda")


def device_layer_w4a16(layer: OM.Layer):
    """The weight-only layer: weights only, no activation scale passed."""
    from nvfp4_w4a4_expert_amd import moe as M
    return M.NVFP4W4A16MoELayer(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s,
                                layer.w2s2, device="cuda")


def run_forward(layer: OM.Layer, x_bits, logits, k, residual_bits=None, w4a16=False, mx=False):
    """GPU forward with every intermediate dumped; returns numpy arrays."""
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    dl = (device_layer_w4a16(layer) if w4a16 else device_layer_mx(layer) if mx
          else device_layer(layer))
    x = M.bf16_tensor(x_bits)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    res = None if residual_bits is None else M.bf16_tensor(residual_bits)
    out, d = dl.forward(x, lg, k, residual=res, debug=True)
    torch.cuda.synchronize()
    got = {name: t.cpu().numpy() for name, t in d.items()}
    got["h"] = got["h"].view(np.uint16)
    got["out"] = M.bf16_bits(out)
    return got


def check_layer_parity(layer: OM.Layer, x_bits, logits, k, residual_bits=None, label="",
                       mx=False):
    """Stage-by-stage parity of one GPU forward against the oracle (of the
    UE8M0 mode when mx, with an OX.LayerMX).

    Unique results are compared exactly (routing ids, permutation, A1 codes
    and scales).  Floating-point stages are compared per row within
    REL_L2_TOL against the fp64 reference over the same dequantised
    operands, and element by element: h and the output must be the bf16
    rounding of a value within the fp32 error bound of the exact one (half a
    bf16 ulp plus that bound); routing weights within the fp32 softmax
    bound.  A2 depends on h's rounding, so it is checked to be the oracle
    quantiser's image of the GPU's own h, and GEMM2 is referenced over that
    A2.  Returns a dict of summary metrics."""
    T = x_bits.shape[0]
    E, I, H = layer.E, layer.I, layer.H
    progress(f"{label}: GPU forward")
    got = run_forward(layer, x_bits, logits, k, residual_bits, mx=mx)
    progress(f"{label}: oracle forward")
    OQm = OX if mx else OQ
    ref = (OX if mx else OM).layer_forward(layer, x_bits, logits, k, residual_bits)
    progress(f"{label}: comparing")

    assert np.array_equal(got["topk_ids"], ref["ids"]), label + " routing ids"
    w_err = routing_weight_bound(logits, ref["ids"], ref["w"])
    assert np.all(np.abs(got["topk_weights"] - ref["w"]) <= w_err), (
        label, "routing weights", float((np.abs(got["topk_weights"] - ref["w"]) / w_err).max()))
    assert np.array_equal(got["expert_offsets"], ref["offsets"]), label + " offsets"
    assert np.array_equal(got["src_pair"], ref["src_pair"]), label + " src_pair"
    assert np.array_equal(got["inv_pair"], ref["inv"]), label + " inv_pair"
    # A1 rows are dumped in (token, slot) order q; the oracle's in grouped order
    assert np.array_equal(got["a1_codes"][ref["src_pair"]], ref["a1"][0]), label + " A1 codes"
    assert np.array_equal(got["a1_sf"][ref["src_pair"]], ref["a1"][1]), label + " A1 scales"

    rexp = OM.row_experts(ref["offsets"])
    c1 = rel_l2_rows(got["c1"], ref["c1"])
    assert c1.max() <= REL_L2_TOL, (label, "C1", c1.max())
    a1_norm = np.linalg.norm(OQm.dequant(*ref["a1"]), axis=1)
    err_c1 = dot_error_bound(a1_norm, weight_row_norms(layer, "w13", OQm.dequant), layer.alpha1,
                             rexp, H)
    assert np.all(np.abs(got["c1"] - ref["c1"]) <= err_c1), (label, "C1 elements")
    h_exact = OM.silu_mul(ref["c1"], I)
    h_gpu = bf16_f64(got["h"])
    assert_correctly_rounded_bf16(h_gpu, h_exact, silu_mul_error_bound(ref["c1"], err_c1, I),
                                  label + " h")
    hr = rel_l2_rows(h_gpu, h_exact)
    del err_c1

    a2c, a2s = OQm.quantize_experts(got["h"], rexp, ref["a2_gscale"])
    assert np.array_equal(got["a2_codes"], a2c), label + " A2 codes vs Q(h_gpu)"
    assert np.array_equal(got["a2_sf"], a2s), label + " A2 scales vs Q(h_gpu)"

    progress(f"{label}: oracle GEMM2 over the GPU's A2")
    c2_ref = (OX if mx else OM).grouped_gemm_ref(got["a2_codes"], got["a2_sf"], ref["offsets"],
                                                 layer.w2c, layer.w2s, layer.alpha2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())
    a2_norm = np.linalg.norm(OQm.dequant(got["a2_codes"], got["a2_sf"]), axis=1)
    err_c2 = dot_error_bound(a2_norm, weight_row_norms(layer, "w2", OQm.dequant), layer.alpha2,
                             rexp, I)
    assert np.all(np.abs(got["c2"] - c2_ref) <= err_c2), (label, "C2 elements")

    res = None if residual_bits is None else OF.bf16_to_f32(residual_bits)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], T, k, res)
    out_gpu = bf16_f64(got["out"])
    err_out = combine_error_bound(c2_ref, err_c2, ref["w"], w_err, ref["inv"], T, k, res)
    del err_c2
    assert_correctly_rounded_bf16(out_gpu, out_ref, err_out, label + " out")
    outr = rel_l2_rows(out_gpu, out_ref)
    out_vs_rounded = rel_l2_rows(out_gpu, bf16_f64(OF.f64_to_bf16(out_ref)))
    assert out_vs_rounded.max() <= REL_L2_TOL, (label, "out vs bf16(ref)", out_vs_rounded.max())

    # independent end-to-end (the oracle's own A2): informational, loose bound
    e2e = rel_l2_rows(bf16_f64(got["out"]), ref["out_f64"])
    a2_flips = int(np.count_nonzero(got["a2_codes"] != ref["a2"][0]))
    return dict(c1_max=float(c1.max()), h_max=float(hr.max()), c2_max=float(c2.max()),
                out_max=float(outr.max()), out_median=float(np.median(outr)),
                out_vs_rounded_max=float(out_vs_rounded.max()),
                e2e_max=float(e2e.max()), a2_byte_diffs_vs_own=a2_flips, got=got, ref=ref)


def check_layer_parity_w4a16(layer: OM.Layer, x_bits, logits, k, residual_bits=None, label=""):
    """Stage-by-stage parity of one weight-only (W4A16) GPU forward against
    the oracle's layer_forward_w4a16.  Routing and permutation exactly; C1
    per row within REL_L2_TOL (and element by element within the fp32
    accumulation bound) of the fp64 product of the bf16 x rows and the
    dequantised weights; h the bf16 rounding of a value within the fp32 bound
    of the fp64 SiLU*mul; C2 against the fp64 product over the GPU's own h
    (one bf16 rounding may differ from the oracle's); the output likewise
    from that C2's combine."""
    T = x_bits.shape[0]
    I, H = layer.I, layer.H
    progress(f"{label}: GPU W4A16 forward")
    got = run_forward(layer, x_bits, logits, k, residual_bits, w4a16=True)
    progress(f"{label}: oracle W4A16 forward")
    ref = OM.layer_forward_w4a16(layer, x_bits, logits, k, residual_bits)
    progress(f"{label}: comparing")

    assert np.array_equal(got["topk_ids"], ref["ids"]), label + " routing ids"
    w_err = routing_weight_bound(logits, ref["ids"], ref["w"])
    assert np.all(np.abs(got["topk_weights"] - ref["w"]) <= w_err), (label, "routing weights")
    assert np.array_equal(got["expert_offsets"], ref["offsets"]), label + " offsets"
    assert np.array_equal(got["src_pair"], ref["src_pair"]), label + " src_pair"
    assert np.array_equal(got["inv_pair"], ref["inv"]), label + " inv_pair"

    rexp = OM.row_experts(ref["offsets"])
    c1 = rel_l2_rows(got["c1"], ref["c1"])
    assert c1.max() <= REL_L2_TOL, (label, "C1", c1.max())
    x_norm = np.linalg.norm(bf16_f64(np.asarray(x_bits)[ref["src_pair"] // k]), axis=1)
    err_c1 = dot_error_bound(x_norm, weight_row_norms(layer, "w13", OQ.dequant), layer.w13s2,
                             rexp, H)
    assert np.all(np.abs(got["c1"] - ref["c1"]) <= err_c1), (label, "C1 elements")
    h_exact = OM.silu_mul(ref["c1"], I)
    h_gpu = bf16_f64(got["h"])
    assert_correctly_rounded_bf16(h_gpu, h_exact, silu_mul_error_bound(ref["c1"], err_c1, I),
                                  label + " h")
    hr = rel_l2_rows(h_gpu, h_exact)
    del err_c1

    progress(f"{label}: oracle W4A16 GEMM2 over the GPU's h")
    c2_ref = OM.grouped_gemm_w16_ref(OF.bf16_to_f32(got["h"]), ref["offsets"], layer.w2c,
                                     layer.w2s, layer.w2s2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())
    err_c2 = dot_error_bound(np.linalg.norm(h_gpu, axis=1),
                             weight_row_norms(layer, "w2", OQ.dequant), layer.w2s2, rexp, I)
    assert np.all(np.abs(got["c2"] - c2_ref) <= err_c2), (label, "C2 elements")

    res = None if residual_bits is None else OF.bf16_to_f32(residual_bits)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], T, k, res)
    out_gpu = bf16_f64(got["out"])
    err_out = combine_error_bound(c2_ref, err_c2, ref["w"], w_err, ref["inv"], T, k, res)
    del err_c2
    assert_correctly_rounded_bf16(out_gpu, out_ref, err_out, label + " out")
    outr = rel_l2_rows(out_gpu, out_ref)
    e2e = rel_l2_rows(out_gpu, ref["out_f64"])
    h_diffs = int(np.count_nonzero(got["h"] != ref["h_bits"]))
    return dict(c1_max=float(c1.max()), h_max=float(hr.max()), c2_max=float(c2.max()),
                out_max=float(outr.max()), out_median=float(np.median(outr)),
                e2e_max=float(e2e.max()), h_diffs_vs_own=h_diffs, got=got, ref=ref)


def gather_token_subset(dev, logits, k, E, tokens, label=""):
    """From one full-batch GPU forward's device tensors ``dev`` (the debug
    dumps and "out"): check the routing ids and the permutation of the whole
    batch exactly against the oracle's router and permutation, and the
    routing weights within the fp32 softmax bound; then gather, as host
    arrays, the rows that a subset of tokens produced, in the order of the
    subset's own permutation (which the oracle's layer on the subset alone
    forms).  Returns the gathered arrays for check_gathered_subset."""
    import torch
    tokens = np.asarray(tokens, dtype=np.int64)
    assert np.array_equal(tokens, np.unique(tokens)), "sorted distinct tokens"
    ids, w = OM.route(logits, k)
    assert np.array_equal(dev["topk_ids"].cpu().numpy(), ids), label + " routing ids"
    w_err = routing_weight_bound(logits, ids, w)
    assert np.all(np.abs(dev["topk_weights"].cpu().numpy() - w) <= w_err), (
        label, "routing weights")
    offsets, src_pair, inv = OM.permute(ids, E)
    assert np.array_equal(dev["expert_offsets"].cpu().numpy(), offsets), label + " offsets"
    assert np.array_equal(dev["src_pair"].cpu().numpy(), src_pair), label + " src_pair"
    assert np.array_equal(dev["inv_pair"].cpu().numpy(), inv), label + " inv_pair"
    sub_ids, _ = OM.route(np.asarray(logits)[tokens], k)
    _, sub_src, _ = OM.permute(sub_ids, E)
    qs = sub_src.astype(np.int64)
    q = tokens[qs // k] * k + qs % k                   # the pairs, in the subset's order
    rows = inv[q].astype(np.int64)                     # their grouped rows
    rows_d = torch.from_numpy(rows).to(dev["c1"].device)
    q_d = torch.from_numpy(q).to(dev["c1"].device)
    got = {name: dev[name].index_select(0, rows_d).cpu().numpy()
           for name in ("c1", "h", "a2_codes", "a2_sf", "c2")}
    # A1 rows are dumped in (token, slot) order
    got.update({name: dev[name].index_select(0, q_d).cpu().numpy()
                for name in ("a1_codes", "a1_sf")})
    got["h"] = got["h"].view(np.uint16)
    tok_d = torch.from_numpy(tokens).to(dev["c1"].device)
    got["out"] = dev["out"].view(torch.int16).index_select(0, tok_d).cpu().numpy().view(
        np.uint16)
    return got


def check_gathered_subset(layer: OM.Layer, x_sub, logits_sub, k, res_sub, got, label=""):
    """Stage-by-stage parity of the gathered rows of a subset of tokens
    (gather_token_subset) against the oracle's layer on those tokens alone;
    the MoE layer treats tokens independently, so that is the reference for
    those rows of the full batch.  A1 codes and scales exactly; C1 per row
    within REL_L2_TOL and element-wise within the fp32 accumulation bound; h
    correctly rounded; A2 the oracle quantiser's image of the GPU's h; C2 over
    the GPU's A2 as C1; the output correctly rounded from that C2's combine.
    CPU only.  Returns per-stage maxima."""
    E, I, H = layer.E, layer.I, layer.H
    nt = x_sub.shape[0]
    ref = OM.layer_forward(layer, x_sub, logits_sub, k, res_sub)
    assert np.array_equal(got["a1_codes"], ref["a1"][0]), label + " A1 codes"
    assert np.array_equal(got["a1_sf"], ref["a1"][1]), label + " A1 scales"
    rexp = OM.row_experts(ref["offsets"])
    hit = np.unique(rexp)
    c1 = rel_l2_rows(got["c1"], ref["c1"])
    assert c1.max() <= REL_L2_TOL, (label, "C1", c1.max())
    err_c1 = dot_error_bound(np.linalg.norm(OQ.dequant(*ref["a1"]), axis=1),
                             weight_row_norms(layer, "w13", OQ.dequant, hit), layer.alpha1,
                             rexp, H)
    assert np.all(np.abs(got["c1"] - ref["c1"]) <= err_c1), (label, "C1 elements")
    h_exact = OM.silu_mul(ref["c1"], I)
    assert_correctly_rounded_bf16(bf16_f64(got["h"]), h_exact,
                                  silu_mul_error_bound(ref["c1"], err_c1, I), label + " h")
    a2c, a2s = OQ.quantize_experts(got["h"], rexp, ref["a2_gscale"])
    assert np.array_equal(got["a2_codes"], a2c), label + " A2 codes vs Q(h_gpu)"
    assert np.array_equal(got["a2_sf"], a2s), label + " A2 scales vs Q(h_gpu)"
    c2_ref = OM.grouped_gemm_ref(got["a2_codes"], got["a2_sf"], ref["offsets"], layer.w2c,
                                 layer.w2s, layer.alpha2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())
    err_c2 = dot_error_bound(np.linalg.norm(OQ.dequant(got["a2_codes"], got["a2_sf"]), axis=1),
                             weight_row_norms(layer, "w2", OQ.dequant, hit), layer.alpha2,
                             rexp, I)
    assert np.all(np.abs(got["c2"] - c2_ref) <= err_c2), (label, "C2 elements")
    res_f = None if res_sub is None else OF.bf16_to_f32(res_sub)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], nt, k, res_f)
    w_err = routing_weight_bound(logits_sub, ref["ids"], ref["w"])
    err_out = combine_error_bound(c2_ref, err_c2, ref["w"], w_err, ref["inv"], nt, k, res_f)
    out_gpu = bf16_f64(got["out"])
    assert_correctly_rounded_bf16(out_gpu, out_ref, err_out, label + " out")
    return dict(c1_max=float(c1.max()), c2_max=float(c2.max()),
                out_max=float(rel_l2_rows(out_gpu, out_ref).max()), experts_hit=int(hit.size))
