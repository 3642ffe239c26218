"""Pins for the oracle's E2M1 / E4M3 / bf16 codecs (CPU only).

What pins them, other than the oracle itself:
  * the page's printed E2M1 code table and its constants (tests/golden);
  * round-to-nearest-even and saturation as the page states them (golden);
  * the public OCP E4M3 definition at a few well-known points (1.0 = 0x38,
    smallest subnormal 2^-9, smallest normal 2^-6, 448 = 0x7E, 0x7F = NaN);
  * brute force: the exact rational nearest-value search against the
    vectorised midpoint encoder over every bf16 bit pattern.
"""
import math
import os

import numpy as np
import pytest

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_e2m1_table_matches_page():
    rows = list(_rows("e2m1_code_table.txt"))
    assert len(rows) == 16
    for code_s, val_s in rows:
        code = int(code_s, 2)
        v = float(val_s)
        got = F.e2m1_decode(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (code_s, got, v)


def test_constants_match_page():
    c = {k: float(v) for k, v in _rows("nvfp4_constants.txt")}
    assert F.E2M1_MAX == c["e2m1_max"]
    assert F.E4M3_MAX == c["e4m3_max"]
    assert F.NVFP4_RANGE == c["combined_range"] == c["e2m1_max"] * c["e4m3_max"]
    assert max(abs(v) for v in F.E2M1_TABLE) == c["e2m1_max"]
    assert np.nanmax(F.E4M3_VALUES) == c["e4m3_max"]


@pytest.mark.parametrize("enc", ["exact", "vec"])
def test_e2m1_rounding_pins(enc):
    for x_s, code_s in _rows("e2m1_rounding.txt"):
        x = float(x_s)
        want = int(code_s, 2)
        got = F.e2m1_encode_exact(x) if enc == "exact" else int(F.e2m1_encode(np.float32(x)))
        assert got == want, (x_s, got, want)


def test_e2m1_representable_values_roundtrip():
    for code in range(16):
        v = F.e2m1_decode(code)
        assert F.e2m1_encode_exact(v) == code
        assert int(F.e2m1_encode(np.float32(v))) == code


def test_e2m1_just_off_midpoints():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for i, m in enumerate(mids):
        below = np.nextafter(np.float32(m), np.float32(0))
        above = np.nextafter(np.float32(m), np.float32(np.inf))
        assert int(F.e2m1_encode(below)) == i          # lower neighbour
        assert int(F.e2m1_encode(above)) == i + 1      # upper neighbour
        assert F.e2m1_encode_exact(float(below)) == i
        assert F.e2m1_encode_exact(float(above)) == i + 1


def test_e2m1_exact_vs_vectorised_all_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    vals = F.bf16_to_f32(bits.astype(np.uint16))
    keep = ~np.isnan(vals)
    vals = vals[keep]
    vec = F.e2m1_encode(vals)
    # the exact encoder is slow; compare on every distinct magnitude class
    # (all values > 8 saturate, so sample those) and all values <= 8
    small = np.abs(vals) <= 8
    idx = np.nonzero(small)[0]
    big = np.nonzero(~small)[0][::97]
    for i in np.concatenate([idx, big]):
        assert F.e2m1_encode_exact(float(vals[i])) == int(vec[i]), vals[i]


def test_e4m3_definition_points():
    assert F.e4m3_decode(0x7E) == 448.0
    assert F.e4m3_decode(0x38) == 1.0
    assert F.e4m3_decode(0x01) == 2.0 ** -9
    assert F.e4m3_decode(0x08) == 2.0 ** -6
    assert F.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert math.isnan(F.e4m3_decode(0x7F)) and math.isnan(F.e4m3_decode(0xFF))
    assert F.e4m3_decode(0xB8) == -1.0
    pos = F.E4M3_VALUES[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[0] == 0.0 and pos.size == 127


def test_e4m3_roundtrip_and_ties():
    pos = F.E4M3_VALUES[:0x7F]
    for c in range(0x7F):
        assert F.e4m3_encode_exact(pos[c]) == c
        assert int(F.e4m3_encode(np.float32(pos[c]))) == c
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode_exact(mid) == want
        assert int(F.e4m3_encode(np.float32(mid))) == want


def test_e4m3_saturation():
    for s in [448.0, 449.0, 464.0, 479.0, 480.0, 1e9, float("inf")]:
        assert F.e4m3_encode_exact(s) == 0x7E
        assert int(F.e4m3_encode(np.float32(s))) == 0x7E
    # below the smallest subnormal's midpoint -> 0, at it -> tie to even (0)
    assert int(F.e4m3_encode(np.float32(2.0 ** -10))) == 0
    assert int(F.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 1


def test_e4m3_exact_vs_vectorised_all_bf16_nonneg():
    bits = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)   # +0 .. +inf
    vals = F.bf16_to_f32(bits)
    vec = F.e4m3_encode(vals)
    sel = np.nonzero(vals <= 500)[0]
    for i in sel[::3]:
        assert F.e4m3_encode_exact(float(vals[i])) == int(vec[i]), vals[i]
    assert np.all(vec[vals >= 448] == 0x7E)


def test_bf16_rounding():
    # exact bf16 values pass through; midpoints go to even; brute force nearest
    rng = np.random.default_rng(1)
    a = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    got = F.f64_to_bf16(a)
    for x, b in zip(a[:3000], got[:3000]):
        v = float(F.bf16_to_f32(np.uint16(b)))
        lo = F.bf16_to_f32(np.uint16(b - 1 if b & 0x7FFF else b))
        hi = F.bf16_to_f32(np.uint16(b + 1))
        assert abs(v - x) <= abs(float(lo) - x) and abs(v - x) <= abs(float(hi) - x)
    one = np.float64(1.0)
    ulp = 2.0 ** -7
    assert F.f64_to_bf16(one + ulp / 2) == F.f64_to_bf16(one)            # tie -> even (1.0)
    assert F.f64_to_bf16(one + 1.5 * ulp) == F.f64_to_bf16(one + 2 * ulp)  # tie -> even


def test_nibble_packing_order():
    codes = np.arange(16, dtype=np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(F.unpack_nibbles(packed), codes)
