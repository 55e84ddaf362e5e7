// mx_device.hpp -- gfx950 device primitives for the MXFP8 cast.
//
// Format facts (from "Add swiglu + MXFP8 fused CuTe DSL kernel", Summary,
// Numerics and tests, commit message): 32-element blocks, one E8M0 scale
// chosen by rounding the exponent up (RCEIL), E4M3 elements; a NaN/Inf amax
// invalidates the block (scale byte 255, data 0x7F).
//
// Every value that gets quantized here is a bf16 number (the fused
// activations are rounded to bf16 first, as eager bf16 does), so block amax
// is an integer max over bf16 magnitude bits and the scale byte follows
// from the exponent/mantissa fields of that bf16 amax.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef uint32_t u32;

struct alignas(16) V4 {
  u32 x, y, z, w;
};

// ---------------------------------------------------------------- bf16 pairs
// A u32 holds two bf16: element 0 in the low half, element 1 in the high half.
__device__ __forceinline__ float lo_f(u32 v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f(u32 v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(v, b2));
}

// Per-half unsigned max (v_pk_max_u16).
__device__ __forceinline__ u32 pk_max(u32 a, u32 b) {
  typedef unsigned short s2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(u32, __builtin_elementwise_max(__builtin_bit_cast(s2, a), __builtin_bit_cast(s2, b)));
}

// Largest bf16 magnitude (as bits, sign dropped) over n packed words.
// NaN has magnitude bits above 0x7F80 and Inf exactly 0x7F80, so a result
// >= 0x7F80 flags a non-finite block.
template <int n>
__device__ __forceinline__ u32 amax_bits(const u32 *v) {
  u32 m = v[0] & 0x7fff7fffu;
#pragma unroll
  for (int i = 1; i < n; i++) m = pk_max(m, v[i] & 0x7fff7fffu);
  return max(m & 0xffffu, m >> 16);
}

// ---------------------------------------------------------- cross-lane max
// DPP quad_perm lane swaps inside groups of four lanes.
__device__ __forceinline__ u32 max_xor1(u32 v) {
  return max(v, (u32)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
}
__device__ __forceinline__ u32 max_xor2(u32 v) {
  return max(v, (u32)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
}

// ---------------------------------------------------------------- E8M0 RCEIL
// Scale byte for a block whose amax is the bf16 magnitude a = (e, m):
// amax = (1 + m/128) 2^(e-127).  448 * 2^k = 1.75 * 2^(k+8), so the least
// k with amax <= 448 * 2^k is e-135 when m <= 0x60 (mantissa <= 1.75) and
// e-134 otherwise; byte = k + 127, floored at 0 (zero and subnormal amax and
// tiny normals all land on byte 0).  The largest finite bf16 gives 247; a
// non-finite amax (a >= 0x7f80) gives 255.
// In five instructions: a + 0x1f carries into the exponent field exactly
// when m > 0x60, so the byte is ((a + 0x1f) >> 7) - 8; a + 0x80 reaches bit
// 15 exactly when a >= 0x7f80, and adding that bit to a lifts the byte past
// 255, where the clamp to [0, 255] holds it.  Equal to the rule above for
// every a in [0, 0x7fff] (checked exhaustively).
__device__ __forceinline__ u32 e8m0_rceil(u32 a) {
  const int y = (int)(a + ((a + 0x80u) & 0x8000u)) + (0x1f - 0x400);
  return (u32)min(max(y >> 7, 0), 255);
}

// ---------------------------------------------------------------- E4M3 cast
// v_cvt_scalef32_pk_fp8_bf16 converts two packed bf16 values to E4M3 codes,
// dividing by 2^e where e is the exponent field of its fp32 scale operand
// read as an E8M0 byte (field 0 stands for 2^-127), rounding to nearest
// even.  Passing the bits (b << 23) therefore quantizes at scale byte b
// exactly: x * 2^(127-b) -> E4M3.  Checked on gfx950 against the definition
// for every bf16 value under scales 2^-127 .. 2^127.  Inputs above 464
// after scaling would give NaN instead of saturating, but under RCEIL every
// finite value of a block is at most 448 after scaling.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e8m0_as_scale(u32 b) { return __uint_as_float(b << 23); }

// Four bf16 values (two packed words) -> four codes, byte i = element i.
// Each convert replaces one 16-bit half of its destination and keeps the
// other; the two together replace both, so the destination may start as any
// value.  REUSE starts it as w0, whose register the first convert then takes
// over where the values are not needed afterwards (a zero start costs a
// move); elsewhere it starts at zero, which leaves the register allocator
// more freedom.
template <bool REUSE = false>
__device__ __forceinline__ u32 cvt4(u32 w0, u32 w1, float scale) {
  i16x2 r = REUSE ? __builtin_bit_cast(i16x2, w0) : i16x2{0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w1), scale, true);
  return __builtin_bit_cast(u32, r);
}

// Quantize eight values of a block (four packed words) with scale byte b;
// b == 255 marks an invalid (NaN/Inf) block, whose codes are all 0x7F.
template <bool REUSE = false>
__device__ __forceinline__ uint2 quant8(const u32 *v, u32 b) {
  const float s = e8m0_as_scale(b);
  uint2 q = make_uint2(cvt4<REUSE>(v[0], v[1], s), cvt4<REUSE>(v[2], v[3], s));
  if (b == 255u) q = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
  return q;
}

// ---------------------------------------------------------------- activation
// sigmoid(g) = 1 / (1 + e^-g) with the hardware exp2 and reciprocal.  Valid
// for g >= -80 (e^-g stays a normal fp32 and its reciprocal too); far
// negative gates go through the scaled forms below.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sigmoid_near(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
}

// The same sigmoid with one Newton step on the reciprocal: r' = r + r (1 - d r)
// for d = 1 + e^-g, two fma, which leaves the quotient within about half an
// ulp.  The hardware reciprocal alone is off by up to about one ulp, enough
// to round g sigmoid(g) to the other bf16 neighbour where the exact value
// lies about an ulp from a bf16 rounding midpoint (g = 5.9375 is the one
// finite bf16 gate where that happens).  Valid for g >= -80, as above.
__device__ __forceinline__ float sigmoid_refined(float g) {
  const float d = 1.0f + __builtin_amdgcn_exp2f(-g * kLog2e);
  const float r = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
}

// For g < -80: sigmoid(g) = e^g / (1 + e^g) and 1 + e^g == 1 in fp32, so
// sigmoid(g) == e^g, which is below 2^-115 and may be an fp32 subnormal.  It
// is formed as e^g * 2^64 (a normal number) and the 2^-64 is applied last,
// after the other factors, so the only subnormal rounding is the final one.
__device__ __forceinline__ float exp_g_times_2p64(float g) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(g, kLog2e, 64.0f));
}
constexpr float k2m64 = 5.421010862427522e-20f;  // 2^-64
constexpr float kFar = -80.0f;

__device__ __forceinline__ float round_bf16(float x) { return lo_f(pack_bf16(x, 0.0f)); }

}  // namespace mx
