"""GPU parity of the whole layer at an expert count that is not a power of
two (200 experts, top-6, hidden 1024, intermediate 192), in all three operand
modes: the fused routing + A1 quantisation kernel fills 200 of its 256
router slots, the permutation ranks 8-bit ids, and the GEMMs' per-expert
prefix covers 200 entries.  2200 tokens
(13200 pairs >= 32 x 200; 47 to 92 rows per expert) run the large-batch GEMMs
with one or two m-tiles per expert and partial last tiles; 40 tokens (240
pairs, 58 experts without rows) the small-batch ones, where the w13 GEMM
regroups the routed ids itself."""
import pytest

import synthetic as S
from oracle import moe as OM
from oracle import mx as OX

from gpu_helpers import check_layer_parity, check_layer_parity_w4a16

pytestmark = pytest.mark.gpu

E, K, H, I = 200, 6, 1024, 192
TOKENS = [2200, 40]


def _workload(T):
    return S.Workload(f"odd-E{E}-T{T}", 9, T=T, H=H, E=E, I=I, k=K, router="normal",
                      calib_tokens=2048)


def _layer(T, mx):
    w = _workload(T)
    w13, w2 = S.expert_weights(w)
    prep = OX.prepare_layer if mx else OM.prepare_layer
    return w, prep(w13, w2, *S.calibration_batch(w), K, threads=16)


def _report(label, m):
    print(f"[{label}] rel-L2 per row: C1 max {m['c1_max']:.2e}  C2 max {m['c2_max']:.2e}  "
          f"out max {m['out_max']:.2e}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", TOKENS)
def test_e4m3_layer(T):
    w, layer = _layer(T, mx=False)
    assert (T * K >= 32 * E) == (T == 2200)
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), K, label=w.name)
    _report(w.name, m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", TOKENS)
def test_ue8m0_layer(T):
    w, layer = _layer(T, mx=True)
    m = check_layer_parity(layer, S.activations(w), S.router_logits(w), K, label=w.name + " mx",
                           mx=True)
    _report(w.name + " mx", m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", TOKENS)
def test_w4a16_layer(T):
    w, layer = _layer(T, mx=False)
    check_layer_parity_w4a16(layer, S.activations(w), S.router_logits(w), K,
                             label=w.name + " w4a16")
