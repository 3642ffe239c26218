"""GPU parity of the UE8M0 (MX-style) mode against the oracle's UE8M0
variant: quantiser codes and power-of-two scales bit-exact (every finite bf16
pattern under scales that reach both clamps), weight quantisation bit-exact,
and the whole layer (nvfp4_moe_forward_mx, scaled FP4 matrix instructions)
stage by stage on the workloads' layers and edge cases."""
import numpy as np
import pytest

import synthetic as S
from oracle import formats as OF
from oracle import moe as OM
from oracle import mx as OX

from gpu_helpers import check_layer_parity, device_layer_mx, oracle_layer_mx, progress

pytestmark = pytest.mark.gpu

GS_SET = np.array([1.0, 1.0 / 3.0, 448.0 / 6.0, 2688.0, 1e-3, 3.0e38, 0.7071, 12345.678,
                   2.0 ** -20, 1.0 / 2688.0], dtype=np.float32)


def _gpu_quantize_mx(x_bits, K, topk, expert_idx, dst_row, gscale, num_dst_rows):
    """nvfp4_quantize_pairs_mx: token rows scattered to their destination rows."""
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    R = x_bits.shape[0]
    x = M.bf16_tensor(x_bits)
    dev = lambda a, t: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    E = 1 if gscale is None else len(gscale)
    codes = torch.full((num_dst_rows, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((num_dst_rows, K // 32), 0xCD, dtype=torch.uint8, device="cuda")
    L.quantize_pairs_mx(x, x_bits.shape[1], R, K, topk, dev(expert_idx, np.int32),
                        dev(dst_row, np.int32), E, dev(gscale, np.float32), codes, sf,
                        num_dst_rows)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def _gpu_quantize_mx_gather(x_bits, K, src_row, offsets, gscale, P):
    """nvfp4_quantize_experts_mx: grouped output rows gathered from x."""
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    dev = lambda a, t: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    codes = torch.full((P, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((P, K // 32), 0xCD, dtype=torch.uint8, device="cuda")
    L.quantize_experts_mx(M.bf16_tensor(x_bits), x_bits.shape[1], K, dev(src_row, np.int32),
                          x_bits.shape[0], P, dev(offsets, np.int32), len(offsets) - 1,
                          dev(gscale, np.float32), codes, sf)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def test_mx_quantizer_every_bf16_pattern_every_scale():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(OF.bf16_to_f32(bits))]
    rng = np.random.default_rng(1)
    arr = [bits, bits[rng.permutation(bits.size)]]
    x = np.concatenate([a[:a.size // 256 * 256].reshape(-1, 256) for a in arr])
    R = x.shape[0]
    expert = np.arange(R, dtype=np.int32) % GS_SET.size
    codes, sf = _gpu_quantize_mx(x, 256, 1, expert, None, GS_SET, R)
    oc, osf = OX.quantize_experts(x, expert, GS_SET)
    assert (osf == 1).any() and (osf == 254).any()         # both clamps exercised
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)
    order = np.argsort(expert, kind="stable")
    offsets = np.zeros(GS_SET.size + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(np.bincount(expert, minlength=GS_SET.size))
    codes, sf = _gpu_quantize_mx_gather(x, 256, order, offsets, GS_SET, R)
    oc, osf = OX.quantize_experts(x[order], expert[order], GS_SET)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)


def test_mx_quantizer_routed_rows_and_ragged_width():
    """topk 8 of 128 experts with the permutation's destination rows, a row
    width that is not a multiple of 64 blocks, zero rows and outliers."""
    rng = np.random.default_rng(2)
    T, K, E, k = 300, 32 * 37, 128, 8
    x = S.f32_to_bf16_bits((rng.standard_normal((T, K)) *
                            10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32))
    x[7] = 0
    x[:, 5] = S.f32_to_bf16_bits(np.full(T, 3.0e4, dtype=np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = OM.route(logits, k)
    offsets, src, inv = OM.permute(ids, E)
    gs = (10.0 ** rng.uniform(-2, 3, E)).astype(np.float32)
    codes, sf = _gpu_quantize_mx(x, K, k, ids, inv, gs, T * k)
    oc, osf = OX.quantize_experts(x[src // k], OM.row_experts(offsets), gs)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)
    codes, sf = _gpu_quantize_mx_gather(x, K, src // k, offsets, gs, T * k)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)


def test_mx_weight_quantisation_matches_oracle():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    w13, w2 = S.expert_weights(w)
    for wb in (w13, w2):
        c, s, s2 = M.quantize_expert_weights(M.bf16_tensor(wb), mx=True)
        torch.cuda.synchronize()
        oc, osf, os2 = OX.quantize_weights(wb)
        assert np.array_equal(s2.cpu().numpy(), os2)
        assert np.array_equal(s.cpu().numpy(), osf)
        assert np.array_equal(c.cpu().numpy(), oc)


def _report(label, m):
    print(f"[{label}] UE8M0 rel-L2 per row: C1 max {m['c1_max']:.2e}  C2 max {m['c2_max']:.2e}  "
          f"out max {m['out_max']:.2e} (median {m['out_median']:.2e})  e2e max "
          f"{m['e2e_max']:.2e}  A2 bytes differing from oracle-own A2 "
          f"{m['a2_byte_diffs_vs_own']}", flush=True)


def test_mx_tiny_layer():
    w = S.WORKLOADS["tiny"]
    m = check_layer_parity(oracle_layer_mx("tiny"), S.activations(w), S.router_logits(w), w.k,
                           label="mx tiny", mx=True)
    _report("mx tiny", m)


def test_mx_ragged_residual_and_empty_expert():
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(25)
    T = 70
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    res = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    logits[:, 3] = -50.0
    m = check_layer_parity(oracle_layer_mx("tiny"), x, logits, w.k, residual_bits=res,
                           label="mx tiny-res", mx=True)
    assert m["got"]["expert_offsets"][3] == m["got"]["expert_offsets"][4]
    _report("mx tiny-res", m)


@pytest.mark.parametrize("T,k", [(1, 1), (3, 4), (130, 1), (257, 3)])
def test_mx_k_and_token_counts(T, k):
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(300 + T * 10 + k)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    check_layer_parity(oracle_layer_mx("tiny"), x, logits, k, label=f"mx T={T} k={k}", mx=True)


def test_mx_determinism():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    dl = device_layer_mx(oracle_layer_mx("tiny"))
    x = M.bf16_tensor(S.activations(w))
    lg = torch.from_numpy(S.router_logits(w)).cuda()
    a = dl.forward(x, lg, w.k)
    b = dl.forward(x, lg, w.k)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("E,k,T", [(64, 1, 5), (256, 32, 9), (512, 4, 33), (1024, 8, 3)])
def test_mx_fused_routing_and_quantisation(E, k, T):
    """The UE8M0 mode's fused routing + A1 quantisation (one launch) at
    hidden 1024, the narrowest row it takes, with expert counts that select
    each router width and top-k other than 8 as well as 8: ids, weights,
    permutation, A1 codes and power-of-two scales exactly, the rest within
    the bounds."""
    w = S.Workload(f"mx-fused-E{E}-k{k}", 8, T=T, H=1024, E=E, I=64, k=k, router="normal",
                   calib_tokens=2048)
    w13, w2 = S.expert_weights(w)
    layer = OX.prepare_layer(w13, w2, *S.calibration_batch(w), k, threads=16)
    del w13, w2
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), k, label=w.name, mx=True)
    _report(w.name, m)


@pytest.mark.timeout(900)
def test_mx_decode_layer():
    w = S.WORKLOADS["decode"]
    m = check_layer_parity(oracle_layer_mx("decode"), S.activations(w), S.router_logits(w), w.k,
                           label="mx decode", mx=True)
    _report("mx decode", m)


@pytest.mark.timeout(900)
def test_mx_prefill_layer():
    w = S.WORKLOADS["prefill"]
    progress("mx prefill: start")
    m = check_layer_parity(oracle_layer_mx("prefill"), S.activations(w), S.router_logits(w),
                           w.k, label="mx prefill", mx=True)
    _report("mx prefill", m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [96, 1024])
def test_mx_max_experts_and_topk(T):
    w = S.WORKLOADS["maxsize"]
    m = check_layer_parity(oracle_layer_mx("maxsize"), S.activations(w, tokens=T),
                           S.router_logits(w, tokens=T), w.k, label=f"mx maxsize T={T}", mx=True)
    _report(f"mx maxsize T={T}", m)

