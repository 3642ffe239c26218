// Device-side NVFP4 helpers for gfx950: bf16 unpacking, OCP E4M3 scale
// encode/decode, E2M1 encode, and the 16-element block quantiser.
//
// Format facts (page 3, "Gemma 4 NVFP4 MoE 空输出", "NVFP4" section): an
// NVFP4 value is an E2M1 code (1 sign, 2 exponent, 1 mantissa bit; largest
// magnitude 6) times an E4M3 block scale shared by 16 consecutive elements
// (largest finite 448) times an FP32 global scale.  Encoding to E2M1 rounds
// to nearest with ties to even and saturates to the largest finite value.
// The activation quantiser (same section, runtime-order figure) takes the
// expert's SFScaleVal (the reciprocal of its FP32 input_scale), the block's
// absolute maximum and the E2M1 maximum 6 to form the block scale, rounds it
// to E4M3, normalises the 16 values by it and rounds them to E2M1.
//
// Every fp32 operation below is a single IEEE operation rounded to nearest
// even (no contraction, correctly rounded division, fp32 denormals kept), so
// the produced codes are a deterministic function of the inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kE2M1Max = 6.0f;
constexpr float kE4M3Max = 448.0f;
constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-negative fp32 (or +inf) -> E4M3 code 0x00..0x7E: nearest finite value,
// ties to the even code, saturating at 448 (0x7E; 0x7F is NaN in E4M3).
// Branch-free: both the subnormal and the normal candidate are formed and one
// is selected.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  // NaN, +inf and everything >= 448 saturate: fminf returns 448 for them
  const float c = fminf(s, kE4M3Max);
  const uint32_t u = __float_as_uint(c);
  const int e = (int)(u >> 23) - 127;              // exponent of c (-127 for 0 / fp32 denormals)
  // E4M3 subnormal range (c < 2^-6): multiples of 2^-9 (code == multiple,
  // 8 == 2^-6).  c * 512 is exact; rintf rounds to nearest even.
  const uint32_t sub = (uint32_t)__builtin_rintf(c * 512.0f);
  const uint32_t mant = u & 0x7FFFFFu;
  uint32_t code = ((uint32_t)(e + 7) << 3) | (mant >> 20);
  const uint32_t rem = mant & 0xFFFFFu;               // dropped 20 mantissa bits
  code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
  return e < -6 ? sub : code;                        // c <= 448 keeps code <= 0x7E
}

// E4M3 code (non-negative, finite) -> fp32 value, exact and branch-free.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float sub = (float)m * 0.001953125f;                    // m * 2^-9
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// The same two conversions with the gfx950 FP8 instructions (OCP E4M3):
// values above 448 are clamped first (the instruction alone would give
// NaN), then the conversion rounds to nearest even.  A device self-check pins
// both to the definitions above: the encode on every non-negative fp32 input
// and +inf, the decode on every non-negative code.
__device__ __forceinline__ uint32_t e4m3_encode_hw(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, kE4M3Max), 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_decode_hw(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// |v| -> E2M1 magnitude code, nearest with ties to the even code, saturating.
// Midpoints between the magnitudes {0,.5,1,1.5,2,3,4,6}: .25 .75 1.25 1.75
// 2.5 3.5 5; a midpoint goes to the neighbour whose code is even.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t u = __float_as_uint(v);
  return ((u >> 28) & 8u) | e2m1_mag(__uint_as_float(u & 0x7FFFFFFFu));
}

// Block scale for one (block, expert): from amax/6 (computed once per block)
// and the expert's SFScaleVal gs.  Returns the E4M3 code and the multiplier
// that normalises the block's elements.
struct BlockScale {
  uint32_t sf;
  float inv;
};

__device__ __forceinline__ BlockScale block_scale(float amax_over_6, float gs) {
#pragma clang fp contract(off)
  BlockScale r;
  const float s = gs * amax_over_6;
  r.sf = e4m3_encode_hw(s);
  const float sv = e4m3_decode_hw(r.sf);
  r.inv = (sv == 0.0f) ? 0.0f : fminf(gs / sv, kFltMax);
  return r;
}

// The UE8M0 (power-of-two) block scale of the MX-style mode (page 3, "NVFP4"
// section: the quantiser template's UE8M0_SF switch; a block is 32
// elements).  s = gs * amax/6 as in the E4M3 mode, encoded as the smallest
// power of two >= s: code = biased exponent of s, plus one unless s is an
// exact power of two, clamped to [1, 254] (s = 0 or an fp32 denormal gives 1;
// +inf, NaN or s above 2^127 give 254).  The normalising multiplier is
// fl32(gs / 2^(code - 127)), clamped to FLT_MAX, exactly as in the E4M3 mode.
__device__ __forceinline__ BlockScale block_scale_ue8m0(float amax_over_6, float gs) {
#pragma clang fp contract(off)
  BlockScale r;
  const float s = gs * amax_over_6;
  const uint32_t u = __float_as_uint(s);
  const uint32_t up = (u >> 23) + ((u & 0x7FFFFFu) != 0u ? 1u : 0u);
  r.sf = up < 1u ? 1u : (up > 254u ? 254u : up);
  const float sv = __uint_as_float(r.sf << 23);        // 2^(code - 127), a normal float
  r.inv = fminf(gs / sv, kFltMax);
  return r;
}

// Encode 8 consecutive elements, each multiplied by `inv` (one fp32 product,
// no contraction), into one 32-bit word of packed codes: element i goes to
// bits [4i, 4i+4).  The E2M1 rounding is done by the gfx950 conversion
// instruction with a unit scale; it rounds to nearest-even, saturates to 6 and
// keeps the sign of zero, identically to e2m1_code() on every non-NaN fp32
// input (checked exhaustively over all 2^32 patterns on the device).
__device__ __forceinline__ uint32_t encode8(const float* x, float inv) {
#pragma clang fp contract(off)
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * inv, x[1] * inv, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * inv, x[3] * inv, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * inv, x[5] * inv, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * inv, x[7] * inv, 1.0f, 3);
  return w;
}

// Reference encoder built from the comparisons above (kept for the device
// self-check that pins the conversion instruction to it).
__device__ __forceinline__ uint32_t encode8_compare(const float* x, float inv) {
#pragma clang fp contract(off)
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_code(x[i] * inv) << (4 * i);
  return w;
}

// max |x_i| over 16 values (exact).
__device__ __forceinline__ float absmax16(const float* x) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

// Unpack 8 bf16 held in a 16-byte vector into floats.
__device__ __forceinline__ void unpack_bf16x8(const u32x4& u, float* x) {
  x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
  x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
  x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
  x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}

// Unpack 8 fp16 held in a 16-byte vector into floats (exact conversions).
__device__ __forceinline__ void unpack_f16x8(const u32x4& u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

}  // namespace nvfp4
