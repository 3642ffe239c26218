"""GPU parity of nvfp4_moe_forward, stage by stage, on the five workloads'
layers, plus edge cases (ragged tails, experts without rows, k = 1 and
k = E, residual aliasing, determinism)."""
import numpy as np
import pytest

import synthetic as S
from oracle import moe as OM

from gpu_helpers import check_layer_parity, oracle_layer, run_forward, device_layer

pytestmark = pytest.mark.gpu


def _report(label, m):
    print(f"[{label}] rel-L2 per row: C1 max {m['c1_max']:.2e}  h max {m['h_max']:.2e}  "
          f"C2 max {m['c2_max']:.2e}  out max {m['out_max']:.2e} (median {m['out_median']:.2e}; "
          f"vs bf16(ref) {m['out_vs_rounded_max']:.2e})  e2e max {m['e2e_max']:.2e}  "
          f"A2 bytes differing from oracle-own A2 {m['a2_byte_diffs_vs_own']}", flush=True)


def test_tiny_layer():
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), w.k, label="tiny")
    _report("tiny", m)


def test_tiny_with_residual_ragged_and_empty_expert():
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    rng = np.random.default_rng(5)
    T = 70                                             # not a multiple of any tile
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    res = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    logits[:, 2] = -50.0                               # expert 2 receives no rows
    m = check_layer_parity(layer, x, logits, w.k, residual_bits=res, label="tiny-res")
    assert m["got"]["expert_offsets"][2] == m["got"]["expert_offsets"][3]
    _report("tiny-res", m)


@pytest.mark.parametrize("T,k", [(1, 1), (1, 4), (5, 4), (130, 1), (257, 3)])
def test_tiny_k_and_token_counts(T, k):
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    rng = np.random.default_rng(T * 10 + k)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    check_layer_parity(layer, x, logits, k, label=f"tiny T={T} k={k}")


def test_zero_tokens_is_noop():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    layer = device_layer(oracle_layer("tiny"))
    out = torch.full((1, 256), 3, dtype=torch.int16, device="cuda")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, 4), dtype=torch.float32, device="cuda")
    from nvfp4_w4a4_expert_amd import _lib as L
    L.moe_forward(layer.weights(), x, lg, 0, 2, None, out, None, 0)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 3)


def test_determinism_and_residual_alias():
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    dl = device_layer(oracle_layer("tiny"))
    x = M.bf16_tensor(S.activations(w))
    lg = torch.from_numpy(S.router_logits(w)).cuda()
    a = dl.forward(x, lg, w.k)
    b = dl.forward(x, lg, w.k)
    res = M.bf16_tensor(S.activations(w))
    c = dl.forward(x, lg, w.k, residual=res)
    dl.forward(x, lg, w.k, residual=res, out=res)           # out aliases residual
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), res.view(torch.int16))


@pytest.mark.timeout(900)
def test_decode_layer():
    w = S.WORKLOADS["decode"]
    layer = oracle_layer("decode")
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), w.k, label="decode")
    _report("decode", m)


@pytest.mark.parametrize("T", [64, 65])
def test_permutation_fold_threshold(T):
    """The decode layer's shape at 64 tokens (512 pairs: the most the
    small-batch w13 GEMM regroups itself, its LDS copy of the ids full) and
    at 65 tokens (520 pairs: the permutation kernel runs again), both on the
    small-batch GEMMs: ids, offsets, src_pair and inv exactly, the rest
    within the bounds."""
    w = S.WORKLOADS["decode"]
    rng = np.random.default_rng(640 + T)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    assert T * w.k < 32 * w.E                           # small-batch kernels
    m = check_layer_parity(oracle_layer("decode"), x, logits, w.k, label=f"fold T={T}")
    _report(f"fold T={T}", m)


@pytest.mark.timeout(900)
def test_prefill_layer():
    w = S.WORKLOADS["prefill"]
    layer = oracle_layer("prefill")
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), w.k, label="prefill")
    counts = np.diff(m["ref"]["offsets"])
    assert counts.max() > 4 * counts.mean()            # non-uniform expert loads
    _report("prefill", m)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("layer_idx", [0])
def test_stack_layer(layer_idx):
    """One layer of the 30-layer stack (its own weights, scales and Zipf
    router) on a seeded N(0,1) input and residual of the stack's shape, every
    row checked (the whole chain, on a subset of rows per layer, is in
    test_gpu_stack.py)."""
    w = S.WORKLOADS["stack"]
    layer = oracle_layer("stack", layer_idx)
    x = S.activations(w, layer=layer_idx)
    logits = S.router_logits(w, layer=layer_idx)
    m = check_layer_parity(layer, x, logits, w.k, residual_bits=x, label=f"stack L{layer_idx}")
    assert np.count_nonzero(np.diff(m["ref"]["offsets"]) == 0) >= 1
    _report(f"stack L{layer_idx}", m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [96, 1024])
def test_max_experts_and_topk(T):
    """E = 1024 experts (the boundary's limit) and k = 32: the small-batch
    GEMM path at 96 tokens and the large one at 1024 tokens (P = 32 E)."""
    w = S.WORKLOADS["maxsize"]
    layer = oracle_layer("maxsize")
    x = S.activations(w, tokens=T)
    logits = S.router_logits(w, tokens=T)
    m = check_layer_parity(layer, x, logits, w.k, label=f"maxsize T={T}")
    _report(f"maxsize T={T}", m)


def test_ring_tails_and_skewed_router():
    """hidden 640 / intermediate 320: both GEMMs end on a partial group of
    register-ring steps; a biased router concentrates rows on a few experts."""
    w = S.WORKLOADS["shapes"]
    layer = oracle_layer("shapes")
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), w.k, label="shapes")
    _report("shapes", m)


@pytest.mark.parametrize("E,k,T", [(64, 1, 5), (256, 32, 9), (512, 4, 33), (1024, 8, 3)])
def test_fused_routing_and_quantisation(E, k, T):
    """hidden 1024 (H/16 = 64 lanes, the narrowest row the fused routing + A1
    quantisation launch takes), with expert counts that select each router
    width (64 to 1024 experts) and top-k other than 8 (the generic slot
    loop) as well as 8: ids, weights, permutation and A1 exactly, the rest
    within the bounds."""
    w = S.Workload(f"fused-E{E}-k{k}", 8, T=T, H=1024, E=E, I=64, k=k, router="normal",
                   calib_tokens=2048)
    w13, w2 = S.expert_weights(w)
    layer = OM.prepare_layer(w13, w2, *S.calibration_batch(w), k, threads=16)
    del w13, w2
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), k, label=w.name)
    _report(w.name, m)


def test_all_rows_on_two_experts():
    """Every token routed to experts 0 and 1: many m-tiles of one expert, six
    experts without rows."""
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    rng = np.random.default_rng(31)
    T = 300
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    logits = rng.standard_normal((T, w.E)).astype(np.float32) - 40.0
    logits[:, 0] += 80.0
    logits[:, 1] += 60.0
    m = check_layer_parity(layer, x, logits, 2, label="two experts")
    counts = np.diff(m["ref"]["offsets"])
    assert counts[0] == T and counts[1] == T and counts[2:].sum() == 0


def test_concurrent_forwards_from_two_host_threads():
    """Two host threads, each with its own stream (default priority),
    workspace and layer object, run forwards at the same time: every output
    equals the serial one bit for bit."""
    import threading
    import torch
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["tiny"]
    layer = oracle_layer("tiny")
    xs = [M.bf16_tensor(S.activations(w, layer=i)) for i in range(4)]
    lgs = [torch.from_numpy(S.router_logits(w, layer=i)).cuda() for i in range(4)]
    ref_layer = device_layer(layer)
    ref = [ref_layer.forward(xs[i], lgs[i], w.k).clone() for i in range(4)]
    torch.cuda.synchronize()
    results = {}
    errors = []

    def worker(tid):
        try:
            dl = device_layer(layer)
            stream = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(stream):
                for rep in range(10):
                    i = (tid + rep) % 4
                    outs.append((i, dl.forward(xs[i], lgs[i], w.k, stream=stream.cuda_stream)))
            stream.synchronize()
            results[tid] = outs
        except Exception as e:                      # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for tid in range(2):
        for i, out in results[tid]:
            assert torch.equal(out.view(torch.int16), ref[i].view(torch.int16))
