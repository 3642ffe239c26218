"""Pins for the oracle's per-16 block quantiser (CPU only).

The pages print no worked example of a quantised block, so the operation
order s = fl32(gs * fl32(amax/6)), inv = fl32(gs/sv) is a reading, and the
quantiser is pinned by properties a wrong implementation would break:
  * the 2688 = 6 x 448 saturation point (page constants);
  * exact round trip of blocks built as E2M1 x E4M3 / gs (closed form);
  * sign symmetry, monotonicity, power-of-two invariance (invariants);
  * the null-scale case behaving as SFScaleVal = 1.0 (page excerpt);
  * the scalar exact quantiser (rational nearest search) agreeing with the
    vectorised one over every bf16 pattern (brute force).
"""
import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from synthetic import f32_to_bf16_bits

POS_E4M3 = F.E4M3_VALUES[:0x7F]


def _vec_block(x16, gs):
    c, s = Q.quantize_f32_rows(np.asarray(x16, dtype=np.float32)[None, :],
                               np.array([gs], dtype=np.float32))
    return int(s[0, 0]), F.unpack_nibbles(c)[0].tolist()


def test_combined_range_saturation_point():
    # gs = 1, amax = 2688: s = 448 -> 0x7E and the largest element -> code 7 (6.0)
    x = np.zeros(16, dtype=np.float32)
    x[3] = 2688.0
    x[5] = -1344.0
    sf, codes = Q.quant_block_exact(x, 1.0)
    assert sf == 0x7E and codes[3] == 0x7 and codes[5] == 0xD   # -1344/448 = -3 -> 1101
    # any larger amax saturates both levels: same block scale, top code 7
    for big in [2689.0, 5000.0, 1e6]:
        y = x.copy()
        y[3] = big
        sf2, codes2 = Q.quant_block_exact(y, 1.0)
        assert sf2 == 0x7E and codes2[3] == 0x7
        assert _vec_block(y, 1.0) == (sf2, codes2)


@pytest.mark.parametrize("j", [-8, -3, 0, 2, 5])
def test_exact_roundtrip_of_representable_blocks(j):
    rng = np.random.default_rng(100 + j)
    gs = np.float32(2.0 ** j)
    for _ in range(200):
        sf = int(rng.integers(0x10, 0x70))           # normal range, no clamp
        sv = POS_E4M3[sf]
        mags = rng.integers(0, 8, size=16)
        mags[rng.integers(16)] = 7                    # amax = 6 * sv / gs
        signs = rng.integers(0, 2, size=16)
        codes = (signs << 3) | mags
        x = np.array([F.e2m1_decode(int(c)) for c in codes]) * sv / float(gs)
        got_sf, got = Q.quant_block_exact(x.astype(np.float32), gs)
        assert got_sf == sf
        want = [int(c) if (c & 7) else int(c) for c in codes]
        assert got == want
        assert _vec_block(x, gs) == (got_sf, got)
        deq = np.array([F.e2m1_decode(c) for c in got]) * F.e4m3_decode(got_sf) / float(gs)
        assert np.array_equal(deq, x)


def test_sign_symmetry_and_monotonicity():
    rng = np.random.default_rng(7)
    for _ in range(300):
        x = (rng.standard_normal(16) * np.exp(rng.uniform(-6, 6))).astype(np.float32)
        gs = np.float32(np.exp(rng.uniform(-5, 5)))
        sf, c = _vec_block(x, gs)
        sfn, cn = _vec_block(-x, gs)
        assert sf == sfn
        assert [a ^ 0x8 for a in c] == cn
        order = np.argsort(x)
        vals = [F.e2m1_decode(c[i]) for i in order]
        assert all(vals[i] <= vals[i + 1] for i in range(15))


def test_power_of_two_invariance():
    rng = np.random.default_rng(8)
    for _ in range(300):
        x = rng.standard_normal(16).astype(np.float32)
        gs = np.float32(rng.uniform(20, 200))
        base = _vec_block(x, gs)
        for j in [-4, -1, 1, 3]:
            y = (x * np.float32(2.0 ** j)).astype(np.float32)
            assert _vec_block(y, np.float32(gs * 2.0 ** -j)) == base


def test_zero_block_and_tiny_scale():
    sf, c = Q.quant_block_exact(np.zeros(16), 1.0)
    assert sf == 0 and c == [0] * 16
    sf, c = Q.quant_block_exact(-np.zeros(16), 1.0)
    assert sf == 0 and c == [8] * 16            # -0.0 keeps its sign code
    # amax small enough that the block scale rounds to E4M3 zero: all codes zero
    x = np.full(16, 1e-6, dtype=np.float32)
    x[0] = -1e-6
    sf, c = Q.quant_block_exact(x, 1.0)
    assert sf == 0 and c == [8] + [0] * 15
    assert _vec_block(x, 1.0) == (sf, c)


def test_null_scale_is_unit_scale():
    rng = np.random.default_rng(9)
    bits = f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32))
    a = Q.quantize_experts(bits, np.array([0, 1, 1, 0, 2]), None)
    b = Q.quantize_experts(bits, np.array([0, 1, 1, 0, 2]), np.ones(3, dtype=np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_per_expert_scale_lookup():
    # the same row quantised for two experts uses each expert's own SFScaleVal
    rng = np.random.default_rng(10)
    row = f32_to_bf16_bits(rng.standard_normal((1, 32)).astype(np.float32))
    bits = np.repeat(row, 2, axis=0)
    gsc = np.array([1.0, 300.0], dtype=np.float32)
    c, s = Q.quantize_experts(bits, np.array([0, 1]), gsc)
    c0, s0 = Q.quantize_bf16_rows(row, np.array([1.0], dtype=np.float32))
    c1, s1 = Q.quantize_bf16_rows(row, np.array([300.0], dtype=np.float32))
    assert np.array_equal(c[0], c0[0]) and np.array_equal(s[0], s0[0])
    assert np.array_equal(c[1], c1[0]) and np.array_equal(s[1], s1[0])
    assert not np.array_equal(s0, s1)


@pytest.mark.parametrize("gs", [1.0, 1.0 / 3.0, 448.0 / 6.0, 2688.0, 1e-3, 3.0e38])
def test_exact_vs_vectorised_all_bf16_patterns(gs):
    """Every finite bf16 pattern, arranged in blocks of 16 (several block
    arrangements so amax takes many values), scalar exact == vectorised."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_to_f32(bits)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(int(gs * 1000) % 2**31)
    vals = vals[rng.permutation(vals.size)]
    n = (vals.size // 16) * 16
    blocks = vals[:n].reshape(-1, 16)
    gsv = np.float32(gs)
    codes, sfs = Q.quantize_f32_rows(blocks, np.full(blocks.shape[0], gsv, dtype=np.float32))
    codes = F.unpack_nibbles(codes)
    # the exact quantiser is slow: check a deterministic subset of blocks
    for b in range(0, blocks.shape[0], 23):
        sf, c = Q.quant_block_exact(blocks[b], gsv)
        assert sf == int(sfs[b, 0]) and c == codes[b].tolist(), (b, gs)


def test_dequant_is_exact_in_bf16_and_fp16():
    """Every E2M1 x E4M3 product has at most 6 significant bits and lies in
    [2^-10, 2688], so it is exact in bf16 and in fp16 (closed form)."""
    for c in range(16):
        for sfc in range(0x7F):
            v = F.e2m1_decode(c) * F.e4m3_decode(sfc)
            if v == 0:
                continue
            assert 2.0 ** -10 <= abs(v) <= 2688.0
            assert float(np.float16(v)) == v
            b = f32_to_bf16_bits(np.array([v], dtype=np.float32))
            assert float(F.bf16_to_f32(b)[0]) == v


def test_dequant_closed_form():
    packed = np.array([[0x21, 0x7F] * 4], dtype=np.uint8)       # codes 1,2,15,7,...
    sf = np.array([[0x38]], dtype=np.uint8)                       # 1.0
    d = Q.dequant(packed, sf)
    assert d[0, :4].tolist() == [0.5, 1.0, -6.0, 6.0]


def test_f16_decode_matches_ieee_binary16():
    """The oracle's field-by-field fp16 decode equals numpy's IEEE binary16
    conversion on every pattern, and a few values fixed by the format."""
    from oracle import formats as OF
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = b.view(np.float16).astype(np.float32)
    got = OF.f16_to_f32(b)
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin].view(np.uint32), got[fin].view(np.uint32))
    assert np.array_equal(np.isinf(ref), np.isinf(got)) and np.array_equal(np.isnan(ref), np.isnan(got))
    assert OF.f16_to_f32(np.array([0x3C00, 0x0001, 0x7BFF, 0x8000], np.uint16)).tolist() == \
        [1.0, 2.0 ** -24, 65504.0, -0.0]


def test_f16_rows_quantise_like_bf16_rows_on_shared_values():
    """Values that are both fp16 and bf16 numbers quantise identically through
    either input path (the arithmetic after the exact conversion is shared)."""
    from oracle import formats as OF
    from oracle import quant as OQ
    rng = np.random.default_rng(11)
    # fp16 numbers whose significand fits in bf16's 8 bits, over fp16's range
    m = rng.integers(128, 256, size=(64, 128)).astype(np.float64)
    e = rng.integers(-14, 8, size=(64, 128)).astype(np.float64)   # normal fp16 range
    sgn = np.where(rng.random((64, 128)) < 0.5, -1.0, 1.0)
    vals = (sgn * m / 128.0 * np.exp2(e)).astype(np.float32)
    f16 = vals.astype(np.float16)
    assert np.array_equal(f16.astype(np.float32), vals)
    bf16 = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(OF.bf16_to_f32(bf16), vals)
    gs = np.exp(rng.uniform(-3, 3, 64)).astype(np.float32)
    c1, s1 = OQ.quantize_f16_rows(f16.view(np.uint16), gs)
    c2, s2 = OQ.quantize_bf16_rows(bf16, gs)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
