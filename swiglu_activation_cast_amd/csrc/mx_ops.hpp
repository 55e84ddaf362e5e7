// mx_ops.hpp -- per-chunk value producers of the three casts.
//
// A chunk is eight consecutive columns of one row (one 16-byte load per
// input).  Each op turns its input chunks into the bf16 values that get
// quantized, packed two per word, entirely in registers:
//   OpQuant: x itself (the plain cast).
//   OpFwd:   h = bf16(bf16(silu(g)) * u)        -- two roundings, as eager bf16.
//   OpBwd:   dg, du of h = silu(g) * u for upstream gradient dh
//            (eager bf16 autograd): s = bf16(silu(g)), du = bf16(dh * s),
//            ds = bf16(dh * u), dg = bf16(ds * sig * (1 + g * (1 - sig))).
// Source: "Add swiglu + MXFP8 fused CuTe DSL kernel", Summary (activation
// never materialized), API ([gate | up] in, [dGate | dUp] out), Numerics
// and tests (equal to the eager activation followed by the quantizer).
#pragma once
#include "mx_device.hpp"

namespace mx {

struct OpQuant {
  static constexpr int IN = 1, OUT = 1;
  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) { out[0] = in[0]; }
};

// A gate below -80 needs the scaled sigmoid (see mx_device.hpp).  In bf16,
// g < -80 exactly when the 16-bit pattern, read unsigned, exceeds 0xC2A0
// (sign set, magnitude above 80); negative NaNs also land here, which is
// harmless because the careful path propagates NaN too.
__device__ __forceinline__ bool any_far(const u32 *g) {
  u32 m = pk_max(pk_max(g[0], g[1]), pk_max(g[2], g[3]));
  return max(m & 0xffffu, m >> 16) > 0xC2A0u;
}

// silu(g) in fp32.  `careful` handles gates below -80 through e^g * 2^64.
template <bool careful>
__device__ __forceinline__ float silu_f(float g) {
  float s = g * sigmoid_near(g);
  if (careful && g < kFar) s = (g * exp_g_times_2p64(g)) * k2m64;
  return s;
}

struct OpFwd {
  static constexpr int IN = 2, OUT = 1;  // in: gate, up

  template <bool careful>
  __device__ __forceinline__ static void eval(const u32 *g, const u32 *u, u32 *h) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      u32 sp = pack_bf16(silu_f<careful>(lo_f(g[k])), silu_f<careful>(hi_f(g[k])));
      h[k] = pack_bf16(lo_f(sp) * lo_f(u[k]), hi_f(sp) * hi_f(u[k]));
    }
  }

  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *g = &in[0].x, *u = &in[1].x;
    u32 *h = &out[0].x;
    eval<false>(g, u, h);
    // rare: redo the whole chunk from the packed inputs, so only packed
    // words are live across the branch
    if (__builtin_expect(any_far(g), 0)) eval<true>(g, u, h);
  }
};

struct OpBwd {
  static constexpr int IN = 3, OUT = 2;  // in: dh, gate, up; out: dgate, dup

  template <bool careful>
  __device__ __forceinline__ static void elem(float dhv, float gv, float uv, float &dg, float &du) {
    const float sig = sigmoid_near(gv);
    const float s = round_bf16(silu_f<careful>(gv));
    du = dhv * s;
    const float ds = round_bf16(dhv * uv);
    float r = (ds * sig) * (1.0f + gv * (1.0f - sig));
    // far-negative gate: sig == e^g, so dg = ds * e^g * (1 + g); 2^-64 last
    if (careful && gv < kFar) r = ((ds * (1.0f + gv)) * exp_g_times_2p64(gv)) * k2m64;
    dg = r;
  }

  template <bool careful>
  __device__ __forceinline__ static void eval(const u32 *dh, const u32 *g, const u32 *u, u32 *dg, u32 *du) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float g0, u0, g1, u1;
      elem<careful>(lo_f(dh[k]), lo_f(g[k]), lo_f(u[k]), g0, u0);
      elem<careful>(hi_f(dh[k]), hi_f(g[k]), hi_f(u[k]), g1, u1);
      dg[k] = pack_bf16(g0, g1);
      du[k] = pack_bf16(u0, u1);
    }
  }

  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *dh = &in[0].x, *g = &in[1].x, *u = &in[2].x;
    u32 *dg = &out[0].x, *du = &out[1].x;
    eval<false>(dh, g, u, dg, du);
    if (__builtin_expect(any_far(g), 0)) eval<true>(dh, g, u, dg, du);
  }
};

}  // namespace mx
