"""Shared pieces of the GPU parity tests: oracle-prepared layers (cached per
process), device upload, and the per-row relative-L2 metric.

Expected values always come from ``oracle/`` on the seeded inputs of
``synthetic/``; the HIP path only produces the values under test.
"""
from __future__ import annotations

import functools

import numpy as np

import synthetic as S
from oracle import formats as OF
from oracle import moe as OM
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


@functools.lru_cache(maxsize=4)
def oracle_layer(name: str, layer: int = 0) -> OM.Layer:
    """The oracle's NVFP4 layer (weights quantised and scales calibrated by
    the oracle) for a workload; decode and prefill share one layer."""
    w = S.WORKLOADS[name]
    key_name = "decode" if name == "prefill" else name
    return _prepare(key_name, layer)


@functools.lru_cache(maxsize=4)
def _prepare(name: str, layer: int) -> OM.Layer:
    w = S.WORKLOADS[name]
    w13, w2 = S.expert_weights(w, layer=layer)
    xc, lc = S.calibration_batch(w, layer=layer)
    return OM.prepare_layer(w13, w2, xc, lc, w.k, threads=16)


def device_layer(layer: OM.Layer):
    from nvfp4_w4a4_expert_amd import moe as M
    return M.NVFP4MoELayer(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s,
                           layer.w2s2, layer.w13_input_scale, layer.w2_input_scale,
                           layer.written13, layer.written2, device="cuda")


def run_forward(layer: OM.Layer, x_bits, logits, k, residual_bits=None):
    """GPU forward with every intermediate dumped; returns numpy arrays."""
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    dl = device_layer(layer)
    x = M.bf16_tensor(x_bits)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    res = None if residual_bits is None else M.bf16_tensor(residual_bits)
    out, d = dl.forward(x, lg, k, residual=res, debug=True)
    torch.cuda.synchronize()
    got = {name: t.cpu().numpy() for name, t in d.items()}
    got["h"] = got["h"].view(np.uint16)
    got["out"] = M.bf16_bits(out)
    return got


def check_layer_parity(layer: OM.Layer, x_bits, logits, k, residual_bits=None, label=""):
    """Stage-by-stage parity of one GPU forward against the oracle.

    Unique results are compared exactly (routing ids, permutation, A1 codes
    and scales).  Floating-point stages are compared per row within
    REL_L2_TOL against the fp64 reference over the same dequantised
    operands.  A2 depends on h's rounding, so it is checked to be the oracle
    quantiser's image of the GPU's own h, and GEMM2 is referenced over that
    A2.  Returns a dict of summary metrics."""
    T = x_bits.shape[0]
    E, I = layer.E, layer.I
    got = run_forward(layer, x_bits, logits, k, residual_bits)
    ref = OM.layer_forward(layer, x_bits, logits, k, residual_bits)

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
    # h is bf16 on both sides: the GPU rounds its fp32 SiLU*mul, the oracle
    # rounds its fp64 one; they differ only where the two land on either side
    # of a bf16 rounding boundary (one ulp).
    h_ref = bf16_f64(ref["h_bits"])
    hr = rel_l2_rows(bf16_f64(got["h"]), h_ref)
    assert hr.max() <= REL_L2_TOL, (label, "h", hr.max())
    h_ulp = np.abs(h_ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(bf16_f64(got["h"]) - h_ref) <= h_ulp), label + " h within 1 bf16 ulp"

    rexp = OM.row_experts(ref["offsets"])
    a2c, a2s = OQ.quantize_experts(got["h"], rexp, ref["a2_gscale"])
    assert np.array_equal(got["a2_codes"], a2c), label + " A2 codes vs Q(h_gpu)"
    assert np.array_equal(got["a2_sf"], a2s), label + " A2 scales vs Q(h_gpu)"

    c2_ref = OM.grouped_gemm_ref(got["a2_codes"], got["a2_sf"], ref["offsets"], layer.w2c,
                                 layer.w2s, layer.alpha2)
    c2 = rel_l2_rows(got["c2"], c2_ref)
    assert c2.max() <= REL_L2_TOL, (label, "C2", c2.max())

    res = None if residual_bits is None else OF.bf16_to_f32(residual_bits)
    out_ref = OM.combine_ref(c2_ref, ref["w"], ref["inv"], T, k, res)
    outr = rel_l2_rows(bf16_f64(got["out"]), out_ref)
    assert outr.max() <= REL_L2_TOL, (label, "out", outr.max())
    o_ulp = np.abs(out_ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(bf16_f64(got["out"]) - out_ref) <= o_ulp), label + " out within 1 bf16 ulp"

    # independent end-to-end (the oracle's own A2): informational, loose bound
    e2e = rel_l2_rows(bf16_f64(got["out"]), ref["out_f64"])
    a2_flips = int(np.count_nonzero(got["a2_codes"] != ref["a2"][0]))
    return dict(c1_max=float(c1.max()), h_max=float(hr.max()), c2_max=float(c2.max()),
                out_max=float(outr.max()), out_median=float(np.median(outr)),
                e2e_max=float(e2e.max()), a2_byte_diffs_vs_own=a2_flips, got=got, ref=ref)
