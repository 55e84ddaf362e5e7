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

struct OpFwd {
  static constexpr int IN = 2, OUT = 1;  // in: gate, up
  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *g = &in[0].x, *u = &in[1].x;
    u32 *h = &out[0].x;
    float s[8];
    bool far = false;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float g0 = lo_f(g[k]), g1 = hi_f(g[k]);
      s[2 * k] = g0 * sigmoid_near(g0);
      s[2 * k + 1] = g1 * sigmoid_near(g1);
      far |= (g0 < kFar) | (g1 < kFar);
    }
    if (__builtin_expect(far, 0)) {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        float gk = (k & 1) ? hi_f(g[k >> 1]) : lo_f(g[k >> 1]);
        if (gk < kFar) s[k] = (gk * exp_g_times_2p64(gk)) * k2m64;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      u32 sp = pack_bf16(s[2 * k], s[2 * k + 1]);
      h[k] = pack_bf16(lo_f(sp) * lo_f(u[k]), hi_f(sp) * hi_f(u[k]));
    }
  }
};

struct OpBwd {
  static constexpr int IN = 3, OUT = 2;  // in: dh, gate, up; out: dgate, dup
  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *dh = &in[0].x, *g = &in[1].x, *u = &in[2].x;
    u32 *dg = &out[0].x, *du = &out[1].x;
    float sig[8], s[8], gv[8];
    bool far = false;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      gv[k] = (k & 1) ? hi_f(g[k >> 1]) : lo_f(g[k >> 1]);
      sig[k] = sigmoid_near(gv[k]);
      s[k] = gv[k] * sig[k];
      far |= gv[k] < kFar;
    }
    float e[8];  // e^g * 2^64 for far-negative gates
    if (__builtin_expect(far, 0)) {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        e[k] = exp_g_times_2p64(gv[k]);
        if (gv[k] < kFar) s[k] = (gv[k] * e[k]) * k2m64;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float dh0 = lo_f(dh[k]), dh1 = hi_f(dh[k]);
      u32 sp = pack_bf16(s[2 * k], s[2 * k + 1]);
      du[k] = pack_bf16(dh0 * lo_f(sp), dh1 * hi_f(sp));
      u32 dsp = pack_bf16(dh0 * lo_f(u[k]), dh1 * hi_f(u[k]));
      float ds0 = lo_f(dsp), ds1 = hi_f(dsp);
      float a0 = sig[2 * k], a1 = sig[2 * k + 1];
      float r0 = (ds0 * a0) * (1.0f + gv[2 * k] * (1.0f - a0));
      float r1 = (ds1 * a1) * (1.0f + gv[2 * k + 1] * (1.0f - a1));
      dg[k] = pack_bf16(r0, r1);
    }
    if (__builtin_expect(far, 0)) {
      // sig == e^g here, so dg = ds * e^g * (1 + g); the 2^-64 goes last.
#pragma unroll
      for (int k = 0; k < 8; k++) {
        if (gv[k] < kFar) {
          float ds = (k & 1) ? hi_f(pack_bf16(0.0f, hi_f(dh[k >> 1]) * hi_f(u[k >> 1])))
                             : lo_f(pack_bf16(lo_f(dh[k >> 1]) * lo_f(u[k >> 1]), 0.0f));
          float r = ((ds * (1.0f + gv[k])) * e[k]) * k2m64;
          u32 w = dg[k >> 1];
          u32 rb = pack_bf16(r, r);
          dg[k >> 1] = (k & 1) ? ((w & 0x0000ffffu) | (rb & 0xffff0000u)) : ((w & 0xffff0000u) | (rb & 0x0000ffffu));
        }
      }
    }
  }
};

}  // namespace mx
