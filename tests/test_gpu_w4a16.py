"""GPU parity of the weight-only (W4A16) forward, nvfp4_moe_forward_w4a16:
the same NVFP4 expert weights against bf16 activations, no activation scale
(page 3, "Kernel Backend": the Marlin backend's W4A16 execution).  Stage by
stage against the oracle's layer_forward_w4a16 on the workloads' layers,
plus edge cases: ragged tails, experts without rows, k = 1 and k = E, a
checkpoint whose input scales fail the load-time check, weight sharing with
the W4A4 layer, determinism."""
import numpy as np
import pytest

import synthetic as S

from gpu_helpers import (check_layer_parity_w4a16, device_layer, device_layer_w4a16,
                         oracle_layer)

pytestmark = pytest.mark.gpu


def _report(label, m):
    print(f"[{label}] W4A16 rel-L2 per row: C1 max {m['c1_max']:.2e}  h max {m['h_max']:.2e}  "
          f"C2 max {m['c2_max']:.2e}  out max {m['out_max']:.2e} (median {m['out_median']:.2e})"
          f"  e2e max {m['e2e_max']:.2e}  h elements differing from oracle-own h "
          f"{m['h_diffs_vs_own']}", flush=True)


def test_w4a16_tiny_layer():
    w = S.WORKLOADS["tiny"]
    m = check_layer_parity_w4a16(oracle_layer("tiny"), S.activations(w), S.router_logits(w),
                                 w.k, label="w4a16 tiny")
    _report("w4a16 tiny", m)


def test_w4a16_ragged_residual_and_empty_expert():
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(15)
    T = 70
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    res = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    logits[:, 1] = -50.0
    m = check_layer_parity_w4a16(oracle_layer("tiny"), x, logits, w.k, residual_bits=res,
                                 label="w4a16 tiny-res")
    assert m["got"]["expert_offsets"][1] == m["got"]["expert_offsets"][2]
    _report("w4a16 tiny-res", m)


@pytest.mark.parametrize("T,k", [(1, 1), (3, 4), (130, 1), (257, 3)])
def test_w4a16_k_and_token_counts(T, k):
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(100 + T * 10 + k)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    check_layer_parity_w4a16(oracle_layer("tiny"), x, logits, k, label=f"w4a16 T={T} k={k}")


def test_w4a16_wide_activation_range():
    """bf16 activations far outside fp16's range (1e-15 .. 1e15 per token)
    run exactly: the weight-only path keeps activations bf16."""
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(17)
    T = 40
    mag = 10.0 ** rng.uniform(-15, 15, size=(T, 1))
    x = S.f32_to_bf16_bits((rng.standard_normal((T, w.H)) * mag).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    m = check_layer_parity_w4a16(oracle_layer("tiny"), x, logits, w.k, label="w4a16 range")
    _report("w4a16 range", m)


def test_w4a16_runs_a_checkpoint_whose_input_scales_fail_the_check():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    bad = layer.w13_input_scale.copy()
    bad[1] = np.nan
    with pytest.raises(M.BadScaleError):
        M.NVFP4MoELayer(layer.w13c, layer.w13s, layer.w13s2, layer.w2c, layer.w2s, layer.w2s2,
                        bad, layer.w2_input_scale, device="cuda")
    # the weight-only layer never takes the scales: its output is the oracle's
    m = check_layer_parity_w4a16(layer, S.activations(w), S.router_logits(w), w.k,
                                 label="w4a16 bad-scale ckpt")
    assert m["c1_max"] <= 2e-3
    torch.cuda.synchronize()


def test_w4a16_sharing_weights_and_determinism():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    a4 = device_layer(layer)
    shared = M.NVFP4W4A16MoELayer.sharing(a4)
    own = device_layer_w4a16(layer)
    x = M.bf16_tensor(S.activations(w))
    lg = torch.from_numpy(S.router_logits(w)).cuda()
    a = shared.forward(x, lg, w.k)
    b = own.forward(x, lg, w.k)
    c = own.forward(x, lg, w.k)
    res = M.bf16_tensor(S.activations(w))
    d = own.forward(x, lg, w.k, residual=res)
    own.forward(x, lg, w.k, residual=res, out=res)           # out aliases residual
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(b.view(torch.int16), c.view(torch.int16))
    assert torch.equal(d.view(torch.int16), res.view(torch.int16))
    assert shared.w13.data_ptr() == a4.w13.data_ptr()


@pytest.mark.timeout(900)
def test_w4a16_decode_layer():
    w = S.WORKLOADS["decode"]
    m = check_layer_parity_w4a16(oracle_layer("decode"), S.activations(w), S.router_logits(w),
                                 w.k, label="w4a16 decode")
    _report("w4a16 decode", m)


@pytest.mark.timeout(900)
def test_w4a16_prefill_layer():
    w = S.WORKLOADS["prefill"]
    m = check_layer_parity_w4a16(oracle_layer("prefill"), S.activations(w), S.router_logits(w),
                                 w.k, label="w4a16 prefill")
    _report("w4a16 prefill", m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [96, 1024])
def test_w4a16_max_experts_and_topk(T):
    w = S.WORKLOADS["maxsize"]
    m = check_layer_parity_w4a16(oracle_layer("maxsize"), S.activations(w, tokens=T),
                                 S.router_logits(w, tokens=T), w.k, label=f"w4a16 maxsize T={T}")
    _report(f"w4a16 maxsize T={T}", m)


def test_w4a16_ring_tails():
    w = S.WORKLOADS["shapes"]
    m = check_layer_parity_w4a16(oracle_layer("shapes"), S.activations(w), S.router_logits(w),
                                 w.k, label="w4a16 shapes")
    _report("w4a16 shapes", m)
