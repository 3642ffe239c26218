"""Bit-level codecs for the NVFP4 element and scale formats (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

E2M1 (page 3, "NVFP4" section, code table): 1 sign bit, 2 exponent bits,
1 mantissa bit; sixteen codes, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, with a
separate negative-zero code 1000.  Largest finite magnitude 6.

E2M1 encode (same section, the conversion-instruction paragraph): round to
nearest with ties to even; values beyond the range saturate to the largest
finite value.  "Even" is the code whose mantissa bit is 0.

E4M3 block scale (same section, two-level scaling paragraph): FP8 with
largest finite value 448.  The pages only give 448; the rest of the format is
the public OCP 8-bit E4M3 definition: exponent bias 7, subnormals for exponent
field 0, the all-ones pattern S.1111.111 is NaN and there is no infinity, so
0x7E = 448 is the largest finite code.

Two implementations are given for each encoder: an exact one that searches
the finite value set with rational arithmetic (scalar, slow, the definition)
and a vectorised one over midpoints (fast, used at scale).  Tests check that
they agree.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# --- E2M1 -------------------------------------------------------------------

# Code -> value, transcribed from the page's 16-entry table.
E2M1_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0)
E2M1_MAX = 6.0          # largest finite E2M1 magnitude
E4M3_MAX = 448.0        # largest finite E4M3 value
NVFP4_RANGE = E2M1_MAX * E4M3_MAX   # 2688, the combined two-level range

_E2M1_MAG = np.array(E2M1_TABLE[:8], dtype=np.float64)
# midpoints between consecutive magnitudes; all exact in fp32
_E2M1_MID = ((_E2M1_MAG[:-1] + _E2M1_MAG[1:]) / 2).astype(np.float32)


def e2m1_decode(code: int) -> float:
    return E2M1_TABLE[code & 0xF]


def e2m1_encode_exact(v) -> int:
    """Encode one real value: nearest E2M1 magnitude (exact rational distance),
    ties to the even code, saturating above 6; the sign bit copies the sign of
    v (so negative values that round to 0 give the -0.0 code 1000)."""
    v = float(v)
    neg = np.signbit(v)
    a = abs(v)
    if a == float("inf") or a > E2M1_MAX:
        mag = 7
    else:
        fa = Fraction(a)
        best = None
        for c in range(8):
            d = abs(fa - Fraction(E2M1_TABLE[c]))
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        mag = best[1]
    return (8 if neg else 0) | mag


def e2m1_encode_mag(a: np.ndarray) -> np.ndarray:
    """Vectorised magnitude encode of non-negative fp32 values (inf allowed)."""
    a = np.asarray(a, dtype=np.float32)
    idx = np.searchsorted(_E2M1_MID, a, side="left")      # number of midpoints < a
    tie = np.zeros(a.shape, dtype=bool)
    inr = idx < _E2M1_MID.size
    tie[inr] = a[inr] == _E2M1_MID[idx[inr]]
    # at a tie the candidates are idx and idx+1: keep the even one
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return idx.astype(np.uint8)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    return (np.signbit(v).astype(np.uint8) << 3) | e2m1_encode_mag(np.abs(v))


def e2m1_decode_vec(codes: np.ndarray) -> np.ndarray:
    return np.array(E2M1_TABLE, dtype=np.float64)[np.asarray(codes) & 0xF]


# --- E4M3 -------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    """OCP E4M3: s eeee mmm, bias 7; e == 0 is subnormal; S.1111.111 is NaN."""
    code &= 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E in increasing value order
_E4M3_POS = E4M3_VALUES[:0x7F]
_E4M3_MID = ((_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2).astype(np.float32)


def e4m3_encode_exact(s) -> int:
    """Nearest non-negative finite E4M3 value to s >= 0 (exact), ties to the
    even code, saturating at 448 (code 0x7E)."""
    s = float(s)
    assert not (s < 0) and s == s
    if s == float("inf") or s >= E4M3_MAX:
        return 0x7E
    fs = Fraction(s)
    best = None
    for c in range(0x7F):
        d = abs(fs - Fraction(float(_E4M3_POS[c])))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    """Vectorised: non-negative fp32 (inf allowed) -> code 0x00..0x7E."""
    s = np.asarray(s, dtype=np.float32)
    idx = np.searchsorted(_E4M3_MID, s, side="left")
    tie = np.zeros(s.shape, dtype=bool)
    inr = idx < _E4M3_MID.size
    tie[inr] = s[inr] == _E4M3_MID[idx[inr]]
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return idx.astype(np.uint8)


def e4m3_decode_vec(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


# --- bf16 -------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns (bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of IEEE binary16 bit patterns, decoded field by field:
    (-1)^s * 2^(e-15) * (1 + m/1024) for 0 < e < 31, (-1)^s * 2^-14 * m/1024
    for e == 0, +-inf / NaN for e == 31."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        val = np.where(e == 0, m / 1024.0 * 2.0 ** -14, (1.0 + m / 1024.0) * np.exp2(e - 15.0))
        val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return (sign * val).astype(np.float32)


def f64_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round real values to the nearest bf16, ties to even, via exact float64
    comparison with the two neighbouring bf16 values.  Returns uint16 bits."""
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)                  # nearest fp32 (may already tie-break)
    # choose between the two bf16 neighbours of the fp32 value using the
    # float64 value itself, so no double rounding is introduced
    u = f.view(np.uint32)
    lo = u & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)
    vlo = lo.view(np.float32).astype(np.float64)
    vhi = hi.view(np.float32).astype(np.float64)
    dlo = np.abs(a - vlo)
    dhi = np.abs(vhi - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (((lo >> np.uint32(16)) & np.uint32(1)) == 1))
    out = np.where(pick_hi, hi, lo) >> np.uint32(16)
    return out.astype(np.uint16)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: element 2j in the low nibble,
    element 2j+1 in the high nibble (page 3: two E2M1 values per byte, the
    first operand of each pair conversion landing in the lower half)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
