// mx_ops.hpp -- per-chunk value producers of the casts.
//
// A chunk is eight consecutive columns of one row (one 16-byte load per
// input).  Each op turns its input chunks into the bf16 values that get
// quantized, packed two per word, entirely in registers:
//   OpQuant:        x itself (the plain cast).
//   GatedFwd<Act>:  h = bf16(bf16(act(g)) * u)      -- two roundings, as eager bf16.
//   GatedBwd<Act>:  dg, du of h = act(g) * u for upstream gradient dh
//                   (eager bf16 autograd): a = bf16(act(g)), du = bf16(dh * a),
//                   da = bf16(dh * u), dg = bf16(da * act'(g)).
//   OpFwd / OpBwd:  the SwiGLU pair, act = silu.
// Source: "Add swiglu + MXFP8 fused CuTe DSL kernel", Summary (activation
// never materialized), API ([gate | up] in, [dGate | dUp] out; the activation
// is a compile-time policy of one kernel source), Numerics and tests (equal
// to the eager activation followed by the quantizer), Follow-ups (more gated
// activations).  The page names no activation besides SiLU; GELU (exact and
// tanh forms) and ReLU are taken here as the common gated-unit gates.
#pragma once
#include "mx_device.hpp"

namespace mx {

struct OpQuant {
  static constexpr int IN = 1, OUT = 1;
  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) { out[0] = in[0]; }
};

// True when some gate of the chunk, as a 16-bit pattern read unsigned,
// exceeds `far`: a negative gate beyond the activation's far threshold
// (negative NaNs land here too, harmlessly: the careful forms propagate NaN).
template <u32 far>
__device__ __forceinline__ bool any_far(const u32 *g) {
  if constexpr (far >= 0xFFFFu) {
    return false;
  } else {
    u32 m = pk_max(pk_max(g[0], g[1]), pk_max(g[2], g[3]));
    return max(m & 0xffffu, m >> 16) > far;
  }
}

// ------------------------------------------------------------ gate policies
// Each policy gives, in fp32 registers:
//   act<careful>(g)        the activation (rounded to bf16 by the caller);
//   dgate<careful>(da, g)  da * act'(g)   (rounded to bf16 by the caller);
//   kFarBits               the bf16 pattern above which a chunk takes the
//                          careful forms (gates so negative that the plain
//                          fp32 forms would flush a representable result);
//   kFolded                whether it also has backward forms that take the
//                          careful scaling per element, without a branch.
// The careful forms scale the vanishing exponential by 2^64 and apply 2^-64
// last, so the only subnormal rounding is the final one.

// silu(g) = g * sigmoid(g); silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
struct ActSilu {
  static constexpr u32 kFarBits = 0xC2A0u;  // g < -80
  static constexpr bool kFolded = false;  // no folded backward forms

  template <bool careful>
  __device__ __forceinline__ static float act(float g) {
    float s = g * sigmoid_refined(g);
    if (careful && g < kFar) s = (g * exp_g_times_2p64(g)) * k2m64;
    return s;
  }

  // the backward recomputes the activation as the forward does
  template <bool careful>
  __device__ __forceinline__ static float bwd_act(float g) { return act<careful>(g); }

  template <bool careful>
  __device__ __forceinline__ static float dgate(float da, float g) {
    const float sig = sigmoid_refined(g);
    float r = (da * sig) * (1.0f + g * (1.0f - sig));
    // far-negative gate: sig == e^g, so dg = da * e^g * (1 + g), the small
    // factors multiplied first: da (1 + g) would overflow for g near -2^127
    if (careful && g < kFar) r = (((1.0f + g) * exp_g_times_2p64(g)) * da) * k2m64;
    return r;
  }
};

// GELU, tanh form: 0.5 g (1 + tanh(c (g + 0.044715 g^3))), c = sqrt(2/pi),
// written as g * sigmoid(w) with w = 2c (g + 0.044715 g^3) (the same value:
// 0.5 (1 + tanh z) = sigmoid(2z)), which has no cancellation for g < 0.
// Derivative: sigmoid(w) + g sigmoid(w) (1 - sigmoid(w)) w'(g).
struct ActGeluTanh {
  static constexpr float kC1 = 1.5957691216057308f;   // 2 sqrt(2/pi)
  static constexpr float kC3 = 0.07135481627260025f;  // 2 sqrt(2/pi) * 0.044715
  static constexpr u32 kFarBits = 0xC118u;            // g < -9.5 (w < -80 needs g < -9.68)
  static constexpr bool kFolded = false;  // no folded backward forms

  __device__ __forceinline__ static float w(float g) { return g * (kC1 + kC3 * (g * g)); }
  __device__ __forceinline__ static float dw(float g) { return kC1 + 3.0f * kC3 * (g * g); }

  template <bool careful>
  __device__ __forceinline__ static float act(float g) {
    const float wv = w(g);
    float a = g * sigmoid_near(wv);
    if (careful && wv < kFar) a = (g * exp_g_times_2p64(wv)) * k2m64;
    return a;
  }

  // the backward recomputes the activation as the forward does
  template <bool careful>
  __device__ __forceinline__ static float bwd_act(float g) { return act<careful>(g); }

  template <bool careful>
  __device__ __forceinline__ static float dgate(float da, float g) {
    const float wv = w(g), sig = sigmoid_near(wv), d = dw(g);
    const float t = sig * (1.0f - sig);
    // where t is 0 the second term is 0 for finite g (g * t * d could read
    // 0 * inf once g^2 overflows) and NaN for infinite g
    const float term = (t == 0.0f) ? g * 0.0f : (g * t) * d;
    float r = da * (sig + term);
    if (careful && wv < kFar) {
      // sigmoid(w) == e^w and 1 - sigmoid(w) == 1: dg = da e^w (1 + g w')
      const float e = exp_g_times_2p64(wv);
      r = (e == 0.0f) ? da * (g * 0.0f) : (((1.0f + g * d) * e) * da) * k2m64;
    }
    return r;
  }
};

// GELU, exact form: g Phi(g), Phi(g) = erfc(-g / sqrt 2) / 2 (the normal
// cdf); derivative Phi(g) + g phi(g), phi(g) = e^(-g^2/2) / sqrt(2 pi).
//
// erfc(z) for z = |g| / sqrt 2 >= 0 is t e^(-z^2) Q(x) = t e^(-z^2 + P(x))
// with t = 2 / (2 + z) and x = 2t - 1: the change of variable of
// Schonfelder's Chebyshev expansions of the error function, which maps z in
// [0, inf) onto x in (-1, 1], where Q(x) = erfcx(z) (2 + z) / 2 and
// P(x) = ln Q(x) are smooth.  Both are evaluated in u = x - 1 = 2t - 2 as
// P = u R_P(u) and Q = 1 + u R_Q(u), so that erfc(0) = 1 exactly whatever the
// float32 rounding (tiny gates give the cdf 1/2 exactly, as the definition
// does).  R_P (degree 7, so P has degree 8) and R_Q (degree 6, Q degree 7)
// are the least-squares fits printed by gen_erfc_fit.py (fit errors 1.5e-6
// and 5.0e-6, relative in erfc), evaluated by Horner's rule.  -z^2 = -g^2 / 2 is
// exact for a bf16 g.  The forward forms e^(-z^2 + P) with one exponential;
// the backward forms e^(-z^2) once for both the cdf (times Q) and the
// Gaussian of the derivative.  Phi(g) is erfc(z) / 2 for g < 0 and
// 1 - erfc(z) / 2 otherwise.  For g < -8 the exponentials are formed times
// 2^64 (2^-64 applied last).
constexpr float kErfcP[8] = {0x1.41b1eep-1f, -0x1.3ad8b8p-4f, -0x1.a4d58ep-6f, -0x1.702f1ep-10f, -0x1.384eb8p-6f, -0x1.9bf628p-7f, -0x1.6f3c04p-9f, -0x1.8cb4e6p-13f};
constexpr float kErfcQ[7] = {0x1.41c448p-1f, 0x1.f5cf84p-4f, -0x1.745866p-6f, 0x1.1a637p-10f, 0x1.4bb7c2p-7f, 0x1.bbcf3ap-9f, 0x1.5f16c2p-12f};

struct ActGelu {
  static constexpr float kRsqrt2 = 0.7071067811865476f;
  static constexpr float kRsqrt2Pi = 0.3989422804014327f;  // 1 / sqrt(2 pi)
  static constexpr float kFarG = -8.0f;
  static constexpr u32 kFarBits = 0xC100u;  // g < -8

  // erfc(|g| / sqrt 2) / 2, times 2^64 when `scaled`
  template <bool scaled>
  __device__ __forceinline__ static float half_erfc(float g) {
    const float th = __builtin_amdgcn_rcpf(2.0f + __builtin_fabsf(g) * kRsqrt2);  // t / 2
    const float u = __builtin_fmaf(th, 4.0f, -2.0f);                              // x - 1
    float r = kErfcP[7];
#pragma unroll
    for (int i = 6; i >= 0; i--) r = __builtin_fmaf(r, u, kErfcP[i]);
    const float e = __builtin_fmaf(-0.5f * g, g, u * r);  // -z^2 + P(x)
    return th * __builtin_amdgcn_exp2f(scaled ? __builtin_fmaf(e, kLog2e, 64.0f) : e * kLog2e);
  }

  __device__ __forceinline__ static float cdf(float g) {
    const float q = half_erfc<false>(g);
    return g < 0.0f ? q : 1.0f - q;
  }

  // erfc(|g| / sqrt 2) / 2 from e = e^(-g^2/2) (times 2^64 if e is)
  __device__ __forceinline__ static float half_erfc_q(float g, float e) {
    const float th = __builtin_amdgcn_rcpf(2.0f + __builtin_fabsf(g) * kRsqrt2);  // t / 2
    const float u = __builtin_fmaf(th, 4.0f, -2.0f);                              // x - 1
    constexpr int nq = sizeof(kErfcQ) / sizeof(kErfcQ[0]);
    float r = kErfcQ[nq - 1];
#pragma unroll
    for (int i = nq - 2; i >= 0; i--) r = __builtin_fmaf(r, u, kErfcQ[i]);
    return (th * __builtin_fmaf(u, r, 1.0f)) * e;  // t/2 Q(x) e^(-z^2)
  }
  __device__ __forceinline__ static float cdf_q(float g, float e) {
    const float q = half_erfc_q(g, e);
    return g < 0.0f ? q : 1.0f - q;
  }

  // e^(-g^2/2), times 2^64 when `scaled`.  g^2 is exact for a bf16 g (a
  // normal number unless |g| < 2^-63) and -log2(e)/2 is exactly half of the
  // float log2(e), so g^2 times it rounds as -(g^2/2) times log2(e) does, in
  // one multiply fewer; where g^2 is subnormal the two arguments may differ
  // in the last bit, and the exponential is 1 either way.
  static constexpr float kNegHalfLog2e = -0.5f * kLog2e;
  template <bool scaled>
  __device__ __forceinline__ static float gauss(float g) {
    const float gg = g * g;
    return __builtin_amdgcn_exp2f(scaled ? __builtin_fmaf(gg, kNegHalfLog2e, 64.0f) : gg * kNegHalfLog2e);
  }

  template <bool careful>
  __device__ __forceinline__ static float act(float g) {
    float a = g * cdf(g);
    if (careful && g < kFarG) a = (g * half_erfc<true>(g)) * k2m64;
    return a;
  }

  // the activation as the backward recomputes it: from the same e^(-g^2/2)
  // as dgate below, so that the two share one exponential
  template <bool careful>
  __device__ __forceinline__ static float bwd_act(float g) {
    float a = g * cdf_q(g, gauss<false>(g));
    if (careful && g < kFarG) a = (g * half_erfc_q(g, gauss<true>(g))) * k2m64;
    return a;
  }

  template <bool careful>
  __device__ __forceinline__ static float dgate(float da, float g) {
    const float e = gauss<false>(g);
    float r = da * (cdf_q(g, e) + g * (kRsqrt2Pi * e));
    if (careful && g < kFarG) {
      const float es = gauss<true>(g);
      r = (da * (half_erfc_q(g, es) + g * (kRsqrt2Pi * es))) * k2m64;
    }
    return r;
  }

  // The same two values with the far-gate scaling taken in every element
  // instead of in a branch: the exponent gets 64 added and the result is
  // multiplied by 2^-64 where g < -8, 0 and 1 elsewhere.  fma(x, k, 0)
  // rounds as x k does (up to the sign of a zero, which the exponential
  // ignores) and a product with 1 is exact, so each element gets exactly
  // the value the forms above give it.  A few more instructions per
  // element, but no branch: the kernel needs far fewer registers.
  static constexpr bool kFolded = true;
  __device__ __forceinline__ static float far_bias(float g) { return g < kFarG ? 64.0f : 0.0f; }
  __device__ __forceinline__ static float far_scale(float g) { return g < kFarG ? k2m64 : 1.0f; }
  __device__ __forceinline__ static float gauss_b(float g, float bias) {  // e^(-g^2/2) 2^bias
    return __builtin_amdgcn_exp2f(__builtin_fmaf(g * g, kNegHalfLog2e, bias));
  }
  __device__ __forceinline__ static float bwd_act_folded(float g) {
    return (g * cdf_q(g, gauss_b(g, far_bias(g)))) * far_scale(g);
  }
  __device__ __forceinline__ static float dgate_folded(float da, float g) {
    const float e = gauss_b(g, far_bias(g));
    return (da * (cdf_q(g, e) + g * (kRsqrt2Pi * e))) * far_scale(g);
  }
};

// ReLU: g for g > 0, +0 otherwise (NaN stays NaN); derivative 0 for g <= 0
// and 1 otherwise, so a NaN gate passes the gradient through as eager's
// threshold backward does.
struct ActRelu {
  static constexpr u32 kFarBits = 0xFFFFu;  // no careful form needed
  static constexpr bool kFolded = false;  // no folded backward forms

  template <bool careful>
  __device__ __forceinline__ static float act(float g) {
    return g <= 0.0f ? 0.0f : g;
  }

  // the backward recomputes the activation as the forward does
  template <bool careful>
  __device__ __forceinline__ static float bwd_act(float g) { return act<careful>(g); }

  template <bool careful>
  __device__ __forceinline__ static float dgate(float da, float g) {
    return g <= 0.0f ? da * 0.0f : da;
  }
};

// ------------------------------------------------------------------ gated ops
template <class Act>
struct GatedFwd {
  static constexpr int IN = 2, OUT = 1;  // in: gate, up

  template <bool careful>
  __device__ __forceinline__ static void eval(const u32 *g, const u32 *u, u32 *h) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      u32 ap = pack_bf16(Act::template act<careful>(lo_f(g[k])), Act::template act<careful>(hi_f(g[k])));
      h[k] = pack_bf16(lo_f(ap) * lo_f(u[k]), hi_f(ap) * hi_f(u[k]));
    }
  }

  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *g = &in[0].x, *u = &in[1].x;
    u32 *h = &out[0].x;
    eval<false>(g, u, h);
    // rare: redo the whole chunk from the packed inputs, so only packed
    // words are live across the branch
    if (__builtin_expect(any_far<Act::kFarBits>(g), 0)) eval<true>(g, u, h);
  }
};

template <class Act>
struct GatedBwd {
  static constexpr int IN = 3, OUT = 2;  // in: dh, gate, up; out: dgate, dup

  // One packed word (two elements): a = bf16(act(g)), du = bf16(dh a),
  // da = bf16(dh u), dg = bf16(da act'(g)); each bf16 rounding takes both
  // elements of the pair in one convert.
  template <bool careful>
  __device__ __forceinline__ static void eval(const u32 *dh, const u32 *g, const u32 *u, u32 *dg, u32 *du) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const float g0 = lo_f(g[k]), g1 = hi_f(g[k]), h0 = lo_f(dh[k]), h1 = hi_f(dh[k]);
      const u32 ap = pack_bf16(Act::template bwd_act<careful>(g0), Act::template bwd_act<careful>(g1));
      du[k] = pack_bf16(h0 * lo_f(ap), h1 * hi_f(ap));
      const u32 dap = pack_bf16(h0 * lo_f(u[k]), h1 * hi_f(u[k]));
      dg[k] = pack_bf16(Act::template dgate<careful>(lo_f(dap), g0), Act::template dgate<careful>(hi_f(dap), g1));
    }
  }

  __device__ __forceinline__ static void apply(const V4 *in, V4 *out) {
    const u32 *dh = &in[0].x, *g = &in[1].x, *u = &in[2].x;
    u32 *dg = &out[0].x, *du = &out[1].x;
    eval<false>(dh, g, u, dg, du);
    if (__builtin_expect(any_far<Act::kFarBits>(g), 0)) eval<true>(dh, g, u, dg, du);
  }

  // apply() for launches held to a tighter register budget: policies with
  // folded forms (no rare branch) use them, the others take apply().
  __device__ __forceinline__ static void apply_lean(const V4 *in, V4 *out) {
    if constexpr (Act::kFolded) {
      const u32 *dh = &in[0].x, *g = &in[1].x, *u = &in[2].x;
      u32 *dg = &out[0].x, *du = &out[1].x;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float g0 = lo_f(g[k]), g1 = hi_f(g[k]), h0 = lo_f(dh[k]), h1 = hi_f(dh[k]);
        const u32 ap = pack_bf16(Act::bwd_act_folded(g0), Act::bwd_act_folded(g1));
        du[k] = pack_bf16(h0 * lo_f(ap), h1 * hi_f(ap));
        const u32 dap = pack_bf16(h0 * lo_f(u[k]), h1 * hi_f(u[k]));
        dg[k] = pack_bf16(Act::dgate_folded(lo_f(dap), g0), Act::dgate_folded(hi_f(dap), g1));
      }
    } else {
      apply(in, out);
    }
  }
};

// The SwiGLU pair under names of their own (kernel symbols stay short).
struct OpFwd : GatedFwd<ActSilu> {};
struct OpBwd : GatedBwd<ActSilu> {};

}  // namespace mx
