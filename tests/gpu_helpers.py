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


def assert_correctly_rounded_bf16(got, exact, label):
    """Every bf16 element is within half an ulp of the exact value (|exact| *
    2^-8 bounds half an ulp, 1% slack for the fp32 computation before the
    rounding) plus an absolute floor of 2^-16 of the row's RMS that covers
    fp32 cancellation in sums whose result is much smaller than their terms."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    rms = np.sqrt(np.mean(exact * exact, axis=1, keepdims=True))
    bound = np.abs(exact) * 2.0 ** -8 * 1.01 + rms * 2.0 ** -16
    err = np.abs(got - exact)
    bad = err > bound
    assert not bad.any(), (label, "elements outside half a bf16 ulp", int(bad.sum()),
                           float((err / np.maximum(bound, 1e-300)).max()))


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
    operands.  A2 depends on h's rounding, so it is checked to be the oracle
    quantiser's image of the GPU's own h, and GEMM2 is referenced over that
    A2.  Returns a dict of summary metrics."""
    T = x_bits.shape[0]
    E, I = layer.E, layer.I
    progress(f"{label}: GPU forward")
    got = run_forward(layer, x_bits, logits, k, residual_bits, mx=mx)
    progress(f"{label}: oracle forward")
    OQm = OX if mx else OQ
    ref = (OX if mx else OM).layer_forward(layer, x_bits, logits, k, residual_bits)
    progress(f"{label}: comparing")

    assert np.array_equal(got["topk_ids"], ref["ids"]), label + " routing ids"
    wrel = np.abs(got["topk_weights"] - ref["w"]) / np.abs(ref["w"])
    assert wrel.max() < 2e-6, (label, "routing weights", wrel.max())
    assert np.array_equal(got["expert_offsets"], ref["offsets"]), label + " offsets"
    assert np.array_equal(got["src_pair"], ref["src_pair"]), label + " src_pair"
    assert np.array_equal(got["inv_pair"], ref["inv"]), label + " inv_pair"
    assert np.array_equal(got["a1_codes"], ref["a1"][0]), label + " A1 codes"
    assert np.array_equal(got["a1_sf"], ref["a1"][1]), label + " A1 scales"

    c1 = rel_l2_rows(got["c1"], ref["c1"])
    assert c1.max() <= REL_L2_TOL, (label, "C1", c1.max())
    # h is bf16: the GPU rounds its fp32 SiLU*mul once, so every element is
    # within half a bf16 ulp of the fp64 value, up to fp32 error (floor).
    h_exact = OM.silu_mul(ref["c1"], I)
    h_gpu = bf16_f64(got["h"])
    assert_correctly_rounded_bf16(h_gpu, h_exact, label + " h")
    hr = rel_l2_rows(h_gpu, h_exact)

    rexp = OM.row_experts(ref["offsets"])
    a2c, a2s = OQm.quantize_experts(got["h"], rexp, ref["a2_gscale"])
    assert np.array_equal(got["a2_codes"], a2c), label + " A2 codes vs Q(h_gpu)"
    assert np.array_equal(got["a2_sf"], a2s), label + " A2 scales vs Q(h_gpu)"

    progress(f"{label}: oracle GEMM2 over the GPU's A2")
    c2_ref = (OX if mx else OM).grouped_gemm_ref(got["a2_codes"], got["a2_sf"], ref["offsets"],
                                                 layer.w2c, layer.w2s, layer.alpha2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())

    res = None if residual_bits is None else OF.bf16_to_f32(residual_bits)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], T, k, res)
    out_gpu = bf16_f64(got["out"])
    assert_correctly_rounded_bf16(out_gpu, out_ref, label + " out")
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
    per row within REL_L2_TOL of the fp64 product of the bf16 x rows and the
    dequantised weights; h correctly rounded from the fp64 SiLU*mul; C2
    against the fp64 product over the GPU's own h (one bf16 rounding may
    differ from the oracle's); the output correctly rounded from that C2's
    combine."""
    T = x_bits.shape[0]
    I = layer.I
    progress(f"{label}: GPU W4A16 forward")
    got = run_forward(layer, x_bits, logits, k, residual_bits, w4a16=True)
    progress(f"{label}: oracle W4A16 forward")
    ref = OM.layer_forward_w4a16(layer, x_bits, logits, k, residual_bits)
    progress(f"{label}: comparing")

    assert np.array_equal(got["topk_ids"], ref["ids"]), label + " routing ids"
    wrel = np.abs(got["topk_weights"] - ref["w"]) / np.abs(ref["w"])
    assert wrel.max() < 2e-6, (label, "routing weights", wrel.max())
    assert np.array_equal(got["expert_offsets"], ref["offsets"]), label + " offsets"
    assert np.array_equal(got["src_pair"], ref["src_pair"]), label + " src_pair"
    assert np.array_equal(got["inv_pair"], ref["inv"]), label + " inv_pair"

    c1 = rel_l2_rows(got["c1"], ref["c1"])
    assert c1.max() <= REL_L2_TOL, (label, "C1", c1.max())
    h_exact = OM.silu_mul(ref["c1"], I)
    h_gpu = bf16_f64(got["h"])
    assert_correctly_rounded_bf16(h_gpu, h_exact, label + " h")
    hr = rel_l2_rows(h_gpu, h_exact)

    progress(f"{label}: oracle W4A16 GEMM2 over the GPU's h")
    c2_ref = OM.grouped_gemm_w16_ref(OF.bf16_to_f32(got["h"]), ref["offsets"], layer.w2c,
                                     layer.w2s, layer.w2s2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())

    res = None if residual_bits is None else OF.bf16_to_f32(residual_bits)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], T, k, res)
    out_gpu = bf16_f64(got["out"])
    assert_correctly_rounded_bf16(out_gpu, out_ref, label + " out")
    outr = rel_l2_rows(out_gpu, out_ref)
    e2e = rel_l2_rows(out_gpu, ref["out_f64"])
    h_diffs = int(np.count_nonzero(got["h"] != ref["h_bits"]))
    return dict(c1_max=float(c1.max()), h_max=float(hr.max()), c2_max=float(c2.max()),
                out_max=float(outr.max()), out_median=float(np.median(outr)),
                e2e_max=float(e2e.max()), h_diffs_vs_own=h_diffs, got=got, ref=ref)
