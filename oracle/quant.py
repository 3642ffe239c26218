"""Per-expert NVFP4 activation quantiser (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Follows the runtime-order figure of page 3 ("NVFP4" section), step by step,
for one 16-element micro-block of a row routed to expert e:

  1. read the expert's FP32 input_scale; its reciprocal (taken at load time)
     is SFScaleVal = gs.  With no scale array the value is 1.0 (the page's
     ``SFScale == nullptr ? 1.0f : SFScale[expert_idx]`` excerpt);
  2. amax = max |x_i| over the 16 elements (exact);
  3. combine gs with the E2M1 maximum 6 into the block-scale value
     s = fl32(gs * fl32(amax / 6))              [reading: order of operations]
     and round it to an E4M3 code sf (nearest, ties to even, saturate at 448);
  4. normalise the 16 values by the rounded block scale sv = E4M3(sf):
     v_i = fl32(x_i * inv), inv = fl32(gs / sv) clamped to FLT_MAX, and
     inv = 0 when sv == 0                       [reading: normalisation form]
  5. round each v_i to E2M1 (nearest, ties to even, saturate at 6, sign kept);
  6. pack two codes per byte, even element in the low nibble.

fl32(.) is one IEEE-754 binary32 operation rounded to nearest even; NumPy
float32 ufuncs and scalar operations are exactly that.

The dequantised value of code c with block scale sf is E2M1(c) * E4M3(sf);
the real value it stands for is that times the FP32 global scale
(input_scale for activations, weight_scale_2 for weights).
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E2M1_MAX,
    bf16_to_f32,
    f16_to_f32,
    e2m1_decode_vec,
    e2m1_encode,
    e2m1_encode_exact,
    e4m3_decode,
    e4m3_decode_vec,
    e4m3_encode,
    e4m3_encode_exact,
    pack_nibbles,
)

BLOCK = 16
FLT_MAX = np.float32(np.finfo(np.float32).max)
_SIX = np.float32(E2M1_MAX)


def quant_block_exact(x16, gs=1.0):
    """One block, scalar, with the exact encoders.  x16: 16 fp32-representable
    values; gs: fp32 SFScaleVal.  Returns (sf code, [16 nibble codes])."""
    assert len(x16) == BLOCK
    gs = np.float32(gs)
    xs = [np.float32(v) for v in x16]
    with np.errstate(over="ignore", invalid="ignore"):
        amax = max(abs(v) for v in xs)
        s = np.float32(gs * np.float32(amax / _SIX))
        sf = e4m3_encode_exact(s)
        sv = np.float32(e4m3_decode(sf))
        if sv == 0:
            inv = np.float32(0.0)
        else:
            inv = np.float32(gs / sv)
            if inv > FLT_MAX:
                inv = FLT_MAX
        codes = [e2m1_encode_exact(np.float32(v * inv)) for v in xs]
    return sf, codes


def quantize_f32_rows(x: np.ndarray, gs_row: np.ndarray):
    """Vectorised quantiser over rows of exact fp32 values.

    x: float32 [R, K] (K % 16 == 0); gs_row: float32 [R] (SFScaleVal per row).
    Returns (packed codes uint8 [R, K/2], E4M3 scale codes uint8 [R, K/16]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    assert K % BLOCK == 0
    gs = np.asarray(gs_row, dtype=np.float32).reshape(R, 1)
    xb = x.reshape(R, K // BLOCK, BLOCK)
    with np.errstate(over="ignore", invalid="ignore"):
        amax = np.abs(xb).max(axis=-1)                       # [R, K/16], exact
        s = (gs * (amax / _SIX)).astype(np.float32)           # two fp32 ops
        sf = e4m3_encode(s)
        sv = e4m3_decode_vec(sf).astype(np.float32)           # exact
        inv = np.where(sv == 0, np.float32(0),
                       np.minimum(gs / np.where(sv == 0, np.float32(1), sv), FLT_MAX))
        inv = inv.astype(np.float32)
        v = (xb * inv[..., None]).astype(np.float32)
    codes = e2m1_encode(v).reshape(R, K)
    return pack_nibbles(codes), sf.astype(np.uint8)


def quantize_bf16_rows(x_bits: np.ndarray, gs_row: np.ndarray, chunk: int = 4096):
    """Quantise bf16 rows (uint16 bits [R, K]) with a per-row SFScaleVal."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    codes = np.empty((R, K // 2), dtype=np.uint8)
    sf = np.empty((R, K // BLOCK), dtype=np.uint8)
    gs_row = np.asarray(gs_row, dtype=np.float32)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        c, s = quantize_f32_rows(bf16_to_f32(x_bits[r0:r1]), gs_row[r0:r1])
        codes[r0:r1] = c
        sf[r0:r1] = s
    return codes, sf


def quantize_f16_rows(x_bits: np.ndarray, gs_row: np.ndarray, chunk: int = 4096):
    """Quantise fp16 rows (uint16 bits [R, K]) with a per-row SFScaleVal (page
    3, "NVFP4" runtime figure: the hidden state may be BF16 or FP16; each fp16
    value is exactly an fp32 value, so the fp32 quantiser applies unchanged)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    codes = np.empty((R, K // 2), dtype=np.uint8)
    sf = np.empty((R, K // BLOCK), dtype=np.uint8)
    gs_row = np.asarray(gs_row, dtype=np.float32)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        c, s = quantize_f32_rows(f16_to_f32(x_bits[r0:r1]), gs_row[r0:r1])
        codes[r0:r1] = c
        sf[r0:r1] = s
    return codes, sf


def quantize_experts(x_bits: np.ndarray, row_expert: np.ndarray, gscale, fp16: bool = False):
    """The MoE quantiser: row r uses SFScaleVal = gscale[row_expert[r]], or 1.0
    for every row when ``gscale`` is None.  Rows are bf16 bit patterns, or
    fp16 ones when ``fp16``."""
    R = x_bits.shape[0]
    if gscale is None:
        gs = np.ones(R, dtype=np.float32)
    else:
        gs = np.asarray(gscale, dtype=np.float32)[np.asarray(row_expert, dtype=np.int64)]
    return quantize_f16_rows(x_bits, gs) if fp16 else quantize_bf16_rows(x_bits, gs)


def dequant(packed: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """float64 [R, K] = E2M1(code) * E4M3(sf), exact."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, Kh = packed.shape
    K = 2 * Kh
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_decode_vec(codes).reshape(R, K // BLOCK, BLOCK)
    sc = e4m3_decode_vec(sf).reshape(R, K // BLOCK, 1)
    return (vals * sc).reshape(R, K)
