"""GPU parity of the router (top-k ids bit-exact, softmax weights within the
fp32 error bound of the fp64 softmax) and of the stable permutation (offsets, src_pair, inv bit-exact)
on every workload's router law, including tie-heavy logits and Zipf routing
that leaves experts without tokens."""
import numpy as np
import pytest

import synthetic as S
from oracle import moe as OM

from gpu_helpers import routing_weight_bound

pytestmark = pytest.mark.gpu


def _route_permute(logits, k):
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    T, E = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.route_topk(lg, T, E, k, ids, w)
    L.permute(ids, T, k, E, off, src, inv)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (ids, w, off, src, inv)]


def _check(logits, k):
    ids, w, off, src, inv = _route_permute(logits, k)
    rids, rw = OM.route(logits, k)
    roff, rsrc, rinv = OM.permute(rids, logits.shape[1])
    assert np.array_equal(ids, rids)
    err = np.abs(w - rw)
    bound = routing_weight_bound(logits, rids, rw)
    assert np.all(err <= bound), (err / bound).max()
    assert np.array_equal(off, roff)
    assert np.array_equal(src, rsrc)
    assert np.array_equal(inv, rinv)
    return roff


@pytest.mark.parametrize("name", ["tiny", "quant", "decode", "prefill"])
def test_workload_routers(name):
    w = S.WORKLOADS[name]
    _check(S.router_logits(w), w.k)


@pytest.mark.parametrize("layer", [0, 17, 29])
def test_zipf_stack_router_has_empty_experts(layer):
    w = S.WORKLOADS["stack"]
    off = _check(S.router_logits(w, layer=layer), w.k)
    assert np.count_nonzero(np.diff(off) == 0) >= 1


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (3, 4, 4), (100, 64, 8), (50, 200, 32),
                                   (9, 1000, 8), (33, 1024, 2), (257, 128, 8),
                                   (1000, 1024, 32), (4097, 4, 1), (6000, 7, 3)])
def test_shapes_and_ties(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # heavy ties
    _check(logits, k)
    _check(rng.standard_normal((T, E)).astype(np.float32), k)


def test_permute_many_blocks_skewed():
    """131072 pairs (several permutation blocks, the last one ragged), most of
    them on a few experts, others on none: offsets, src_pair, inv bit-exact."""
    rng = np.random.default_rng(77)
    T, E, k = 16385, 256, 8
    p = np.exp(-0.05 * np.arange(E))
    p[100:140] = 0.0
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    d_ids = torch.from_numpy(ids).cuda()
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.permute(d_ids, T, k, E, off, src, inv)
    torch.cuda.synchronize()
    roff, rsrc, rinv = OM.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(src.cpu().numpy(), rsrc)
    assert np.array_equal(inv.cpu().numpy(), rinv)


@pytest.mark.parametrize("E,k", [(128, 8), (200, 32), (1024, 4)])
def test_signed_zeros_and_extremes(E, k):
    """-0.0 and +0.0 tie (lower index first); subnormals, huge and negative
    logits order like the reals."""
    rng = np.random.default_rng(E + k)
    T = 97
    pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-38, -3.0e38, 3.0e38, 1.0, -1.0, 2.5],
                    dtype=np.float32)
    logits = pool[rng.integers(0, pool.size, size=(T, E))]
    _check(logits, k)
