"""Parity at tile boundaries: experts with exact row counts around the 32-row
sub-tiles of the large-batch GEMM tiles (64-row w13 and 128-row w2 tiles in the
E4M3 mode; 96-row w13 tiles in the weight-only and UE8M0 modes), so every
partly filled tile shape (1, 2, 3 or 4 occupied sub-tiles) runs in each mode;
and, below 32 rows per expert on average, the small-batch kernels' 32-row
tiles with an expert one row past a tile.  Top-1 routing with one dominant
logit per token fixes each expert's count."""
import numpy as np
import pytest

import synthetic as S

from gpu_helpers import (check_layer_parity, check_layer_parity_w4a16, oracle_layer,
                         oracle_layer_mx)

pytestmark = pytest.mark.gpu

# rows per expert (tiny layer: 4 experts); the first two keep T * k >= 32 * E,
# so the large-batch kernels run, the last stays below it
COUNTS = {
    "odd": [97, 65, 33, 1],      # 96 + 1, 65 (3 sub-tiles of a 96-row tile), 33, 1
    "even": [96, 64, 32, 129],   # whole 96- and 32-row tiles; 128 + 1 for w2
    "small": [33, 32, 31, 1],    # 97 pairs < 32 * E: the small-batch kernels
}


def _inputs(counts, seed):
    w = S.WORKLOADS["tiny"]
    rng = np.random.default_rng(seed)
    experts = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(experts)
    T = experts.size
    logits = rng.standard_normal((T, w.E)).astype(np.float32)
    logits[np.arange(T), experts] = 20.0          # the token's only choice at top-1
    x = S.f32_to_bf16_bits(rng.standard_normal((T, w.H)).astype(np.float32))
    return x, logits


@pytest.mark.parametrize("case", sorted(COUNTS))
def test_tile_boundaries_e4m3(case):
    x, logits = _inputs(COUNTS[case], 41)
    m = check_layer_parity(oracle_layer("tiny"), x, logits, 1, label=f"tiles {case} e4m3")
    assert np.array_equal(np.diff(m["got"]["expert_offsets"]), COUNTS[case])


@pytest.mark.parametrize("case", sorted(COUNTS))
def test_tile_boundaries_ue8m0(case):
    x, logits = _inputs(COUNTS[case], 42)
    m = check_layer_parity(oracle_layer_mx("tiny"), x, logits, 1, label=f"tiles {case} ue8m0",
                           mx=True)
    assert np.array_equal(np.diff(m["got"]["expert_offsets"]), COUNTS[case])


@pytest.mark.parametrize("case", sorted(COUNTS))
def test_tile_boundaries_w4a16(case):
    x, logits = _inputs(COUNTS[case], 43)
    check_layer_parity_w4a16(oracle_layer("tiny"), x, logits, 1, label=f"tiles {case} w4a16")
