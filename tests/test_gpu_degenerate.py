"""GPU parity of the layer's most degenerate routing: a single expert (E = 1,
k = 1), so every token goes to expert 0 with weight exactly 1.0, the
permutation is the identity and one expert owns every GEMM row.  5 tokens run
the small-batch GEMMs (the w13 GEMM regrouping the ids itself), 300 tokens
the large-batch ones (several full m-tiles and a partial one), in all three
operand modes."""
import numpy as np
import pytest

import synthetic as S
from oracle import moe as OM
from oracle import mx as OX

from gpu_helpers import check_layer_parity, check_layer_parity_w4a16

pytestmark = pytest.mark.gpu

H, I = 256, 128


def _layer(T, mx):
    w = S.Workload(f"single-expert-T{T}", 10, T=T, H=H, E=1, I=I, k=1, router="normal",
                   calib_tokens=256)
    w13, w2 = S.expert_weights(w)
    prep = OX.prepare_layer if mx else OM.prepare_layer
    return w, prep(w13, w2, *S.calibration_batch(w), 1, threads=16)


def _check_routing(m, T):
    got = m["got"]
    assert np.all(got["topk_ids"] == 0)
    assert np.all(got["topk_weights"] == 1.0)
    assert np.array_equal(got["expert_offsets"], [0, T])
    assert np.array_equal(got["src_pair"], np.arange(T))
    assert np.array_equal(got["inv_pair"], np.arange(T))


@pytest.mark.parametrize("T", [5, 300])
@pytest.mark.parametrize("mx", [False, True])
def test_single_expert_w4a4(T, mx):
    w, layer = _layer(T, mx)
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), 1, label=w.name,
                           mx=mx)
    _check_routing(m, T)


@pytest.mark.parametrize("T", [5, 300])
def test_single_expert_w4a16(T):
    w, layer = _layer(T, mx=False)
    check_layer_parity_w4a16(layer, S.activations(w), S.router_logits(w), 1,
                             label=w.name + " w4a16")
