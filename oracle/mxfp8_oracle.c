/*
 * mxfp8_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU definition of what the fused SwiGLU +
 * MXFP8 cast computes.  It exists to check the HIP kernels: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no code, header, table or constant with the GPU library and never
 * includes anything from it.
 *
 * Sources (web pages, by title and section):
 *  [P1] "Add swiglu + MXFP8 fused CuTe DSL kernel"
 *       - Summary: one pass fuses swiglu with the RCEIL MXFP8 cast; gate/up
 *         read once; rowwise (1x32), colwise (32x1) or both scale layouts.
 *       - API: gated_input packs [gate | up]; backward takes grad_h and
 *         returns [dGate | dUp].
 *       - Numerics and tests: forward E4M3 data and E8M0 scales equal the
 *         eager activation followed by the standalone quantizers, including
 *         NaN/Inf, zero, subnormal-tiny and E4M3-boundary amax cases.
 *       - commit message: a NaN/Inf amax invalidates the block (scale byte
 *         255, all-NaN data); a byte-0 scale descales by 2^127.
 *  [P3] "[mxfp8 moe training] update 3d quant colwise scaling kernel to use
 *       single input/output TMA descriptors", Summary: the 3D (E,N,K)
 *       colwise quant writes each expert column-major.
 *  [P4] "[mxfp8 moe training] add compile support", Perf analysis: the 2D
 *       colwise ("dim1") cast output is column-major; the cast outputs feed
 *       a scaled grouped GEMM (the consumer, orc_mx_gemm below).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes of the repository):
 *  - RCEIL: the scale is the smallest power of two 2^k, k in [-127, 127],
 *    with amax <= 448 * 2^k, i.e. 2^ceil(log2(amax/448)) clamped to the E8M0
 *    range; E8M0 byte = k + 127.  amax == 0 gives byte 0.
 *  - E4M3 is OCP E4M3FN (bias 7, max 448, no infinities, 0x7F/0xFF NaN);
 *    the element cast rounds to nearest, ties to even, and saturates to
 *    +-448.  NaN data is written as 0x7F.
 *  - Any NaN or +-Inf element invalidates its block.
 *  - Eager forward rounds twice: s = bf16(silu(g)), h = bf16(s * u).
 *  - Eager backward (autograd of silu(g) * u in bf16): du = bf16(dh * s),
 *    ds = bf16(dh * u), dg = bf16(ds * sig * (1 + g * (1 - sig))).
 *  - Scales are plain row-major: rowwise [M, W/32], colwise [W, M/32].
 *    Colwise data is [W, M] row-major (the transpose of the [M, W] view).
 *  - 3D: blocks of 32 along N; expert e's data at q[e][k][n], scales at
 *    s[e][k][n/32].
 *  - More gated activations.  [P1] API makes the activation a compile-time
 *    policy, and [P1] Follow-ups plans more than SiLU without naming them.
 *    Taken here: GELU in its exact form x * Phi(x) and in the tanh form, and
 *    ReLU, each in place of silu with the same rounding sites:
 *    a = bf16(act(g)), h = bf16(a * u); du = bf16(dh * a),
 *    da = bf16(dh * u), dg = bf16(da * act'(g)).
 *  - The consumer GEMM is C = A B^T with both operands K-contiguous (as the
 *    rowwise output, or the colwise output of the transposed operand,
 *    stores them) and each element worth decode(code) * 2^(scale - 127).
 *
 * All real arithmetic here is IEEE double: a product of two bf16 values is
 * exact in double, and silu/sigmoid carry ~1e-16 relative error before the
 * single rounding to bf16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ROWWISE 1
#define ORC_COLWISE 2

/* ------------------------------------------------------------------ bf16 */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double orc_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to bf16: 8 significant bits, round to nearest with ties
 * to even, subnormal quantum 2^-133, overflow to +-Inf, NaN to 0x7FC0. */
uint16_t orc_bf16_round(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);              /* a = f * 2^e with f in [0.5, 1)           */
    int q = e - 8;             /* weight of the last kept bit (8 bits kept) */
    if (q < -133)
        q = -133;              /* below 2^-126 the spacing stays 2^-133     */
    double r = ldexp(a, -q);   /* exact: a power-of-two scaling             */
    double n = floor(r);
    double frac = r - n;       /* exact                                     */
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    double rounded = ldexp(n, q);
    double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127             */
    if (rounded > bf16_max)
        return sign | 0x7F80;
    float f = (float)rounded;  /* exact: 8 significant bits fit binary32   */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ E4M3 */

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
 * field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    if (e == 0xF && m == 0x7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9)            /* m/8 * 2^-6        */
                          : ldexp((double)(8 + m), e - 10); /* (1+m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Nearest E4M3 code to v: binary search over the 127 non-negative finite
 * codes (their values increase with the code), ties to the even code,
 * saturation to +-448 above the largest finite value, NaN -> 0x7F. */
uint8_t orc_e4m3_encode(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 126;      /* decode(lo) <= a < decode(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double below = a - orc_e4m3_decode((uint8_t)lo);
    double above = orc_e4m3_decode((uint8_t)hi) - a;
    int code;
    if (below < above)
        code = lo;
    else if (above < below)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------ E8M0 */

/* RCEIL: the smallest k in [-127, 127] with amax <= 448 * 2^k; byte k+127.
 * amax must be finite and >= 0. */
uint8_t orc_e8m0_rceil(double amax)
{
    for (int k = -127; k <= 127; k++)
        if (amax <= ldexp(448.0, k))
            return (uint8_t)(k + 127);
    return 254;
}

/* The real value an E8M0 byte stands for (255 is NaN). */
double orc_e8m0_decode(uint8_t b)
{
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------- one 32-element block */

/* Codes of n values at a given scale byte (x * 2^(127 - byte), then E4M3). */
void orc_quant_block_at(const double *y, int64_t n, int64_t ystride,
                        uint8_t scale, uint8_t *q, int64_t qstride)
{
    if (scale == 255) {
        for (int64_t i = 0; i < n; i++)
            q[i * qstride] = 0x7F;
        return;
    }
    double descale = ldexp(1.0, 127 - (int)scale);
    for (int64_t i = 0; i < n; i++)
        q[i * qstride] = orc_e4m3_encode(y[i * ystride] * descale);
}

/* Scale byte of a block: 255 if any element is NaN or +-Inf, else RCEIL of
 * the largest magnitude. */
uint8_t orc_block_scale(const double *y, int64_t n, int64_t ystride)
{
    double amax = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double v = y[i * ystride];
        if (!isfinite(v))
            return 255;
        if (fabs(v) > amax)
            amax = fabs(v);
    }
    return orc_e8m0_rceil(amax);
}

void orc_quant_block(const double *y, int64_t n, int64_t ystride,
                     uint8_t *q, int64_t qstride, uint8_t *s)
{
    *s = orc_block_scale(y, n, ystride);
    orc_quant_block_at(y, n, ystride, *s, q, qstride);
}

/* -------------------------------------------------------------- activation */

double orc_sigmoid(double x)
{
    if (isnan(x))
        return x;
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double t = exp(x);         /* no overflow for very negative x */
    return t / (1.0 + t);
}

double orc_silu(double x)
{
    return x * orc_sigmoid(x); /* -Inf * 0 = NaN, +Inf * 1 = +Inf */
}

/* Gate activations of the gated family (see the readings above). */
enum { ORC_ACT_SILU = 0, ORC_ACT_GELU_TANH = 1, ORC_ACT_GELU = 2, ORC_ACT_RELU = 3 };

#define ORC_PI 3.14159265358979323846

/* Standard normal cdf and density. */
static double norm_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }
static double norm_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * ORC_PI); }

/* GELU, tanh form: 0.5 x (1 + tanh(c (x + 0.044715 x^3))), c = sqrt(2/pi).
 * As 0.5 (1 + tanh(z)) = sigmoid(2 z), this is x * sigmoid(w(x)) with
 * w(x) = 2 c (x + 0.044715 x^3), a form without cancellation at negative x. */
static double gelu_tanh_w(double x) { return 2.0 * sqrt(2.0 / ORC_PI) * (x + 0.044715 * x * x * x); }
static double gelu_tanh_dw(double x) { return 2.0 * sqrt(2.0 / ORC_PI) * (1.0 + 3.0 * 0.044715 * x * x); }

/* act(x).  ReLU maps x <= 0 to +0 and keeps NaN. */
double orc_act(int act, double x)
{
    switch (act) {
    case ORC_ACT_SILU: return x * orc_sigmoid(x);
    case ORC_ACT_GELU_TANH: return x * orc_sigmoid(gelu_tanh_w(x));
    case ORC_ACT_GELU: return x * norm_cdf(x);
    case ORC_ACT_RELU: return (x <= 0.0) ? 0.0 : x;
    }
    return NAN;
}

/* act'(x), the textbook derivative of each.  ReLU's is 0 for x <= 0 and 1
 * otherwise (a NaN gate passes the gradient through, as the eager ReLU
 * backward does: it zeroes only where its output is <= 0). */
double orc_act_grad(int act, double x)
{
    switch (act) {
    case ORC_ACT_SILU: {
        double sig = orc_sigmoid(x);
        return sig * (1.0 + x * (1.0 - sig));
    }
    case ORC_ACT_GELU_TANH: {
        double sw = orc_sigmoid(gelu_tanh_w(x));
        return sw + x * sw * (1.0 - sw) * gelu_tanh_dw(x);
    }
    case ORC_ACT_GELU: return norm_cdf(x) + x * norm_pdf(x);
    case ORC_ACT_RELU: return (x <= 0.0) ? 0.0 : 1.0;
    }
    return NAN;
}

/* Forward value of one element as eager bf16 computes it: two roundings. */
static uint16_t fwd_value(int act, uint16_t g, uint16_t u)
{
    uint16_t a = orc_bf16_round(orc_act(act, orc_bf16_decode(g)));
    return orc_bf16_round(orc_bf16_decode(a) * orc_bf16_decode(u));
}

/* Backward values of one element (eager autograd of act(g) * u). */
static void bwd_value(int act, uint16_t dh, uint16_t g, uint16_t u, uint16_t *dg, uint16_t *du)
{
    double gv = orc_bf16_decode(g), uv = orc_bf16_decode(u), dhv = orc_bf16_decode(dh);
    uint16_t a = orc_bf16_round(orc_act(act, gv));
    *du = orc_bf16_round(dhv * orc_bf16_decode(a));
    uint16_t da = orc_bf16_round(dhv * uv);
    *dg = orc_bf16_round(orc_bf16_decode(da) * orc_act_grad(act, gv));
}

static int act_ok(int act) { return act >= ORC_ACT_SILU && act <= ORC_ACT_RELU; }

int orc_gated_fwd_values(int act, const uint16_t *g, const uint16_t *u, int64_t n, uint16_t *h)
{
    if (!act_ok(act))
        return -1;
    for (int64_t i = 0; i < n; i++)
        h[i] = fwd_value(act, g[i], u[i]);
    return 0;
}

int orc_gated_bwd_values(int act, const uint16_t *dh, const uint16_t *g, const uint16_t *u,
                         int64_t n, uint16_t *dg, uint16_t *du)
{
    if (!act_ok(act))
        return -1;
    for (int64_t i = 0; i < n; i++)
        bwd_value(act, dh[i], g[i], u[i], &dg[i], &du[i]);
    return 0;
}

void orc_swiglu_fwd_values(const uint16_t *g, const uint16_t *u, int64_t n, uint16_t *h)
{
    orc_gated_fwd_values(ORC_ACT_SILU, g, u, n, h);
}

void orc_swiglu_bwd_values(const uint16_t *dh, const uint16_t *g, const uint16_t *u,
                           int64_t n, uint16_t *dg, uint16_t *du)
{
    orc_gated_bwd_values(ORC_ACT_SILU, dh, g, u, n, dg, du);
}

/* ------------------------------------------------------------ matrix level */

typedef struct {
    uint8_t *q_row; int64_t ld_q_row; uint8_t *s_row; int64_t ld_s_row;
    uint8_t *q_col; int64_t ld_q_col; uint8_t *s_col; int64_t ld_s_col;
} orc_out;

/* Quantize a slab of R <= 32 rows (starting at row m0) of a [*, W] matrix
 * y held as doubles, row stride W.  Colwise needs a full 32-row slab. */
static void quant_slab(const double *y, int64_t R, int64_t W, int64_t m0,
                       int layout, const orc_out *o)
{
    if (layout & ORC_ROWWISE)
        for (int64_t r = 0; r < R; r++)
            for (int64_t c0 = 0; c0 < W; c0 += 32)
                orc_quant_block(y + r * W + c0, 32, 1,
                                o->q_row + (m0 + r) * o->ld_q_row + c0, 1,
                                o->s_row + (m0 + r) * o->ld_s_row + c0 / 32);
    if (layout & ORC_COLWISE)
        for (int64_t c = 0; c < W; c++)
            orc_quant_block(y + c, 32, W,
                            o->q_col + c * o->ld_q_col + m0, 1,
                            o->s_col + c * o->ld_s_col + m0 / 32);
}

enum { OP_QUANT = 0, OP_FWD = 1, OP_BWD = 2 };

/* Shared driver: builds the [M, W] values slab by slab, then quantizes. */
static int run(int op, int act, const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
               const uint16_t *c, int64_t ldc, int64_t M, int64_t N, int layout,
               const orc_out *o)
{
    if (M < 0 || N < 0 || layout < 1 || layout > 3 || !act_ok(act))
        return -1;
    if ((layout & ORC_COLWISE) && M % 32 != 0)
        return -1;
    if (op != OP_QUANT && N % 32 != 0)
        return -1;
    if (op == OP_QUANT && (layout & ORC_ROWWISE) && N % 32 != 0)
        return -1;
    int64_t W = (op == OP_BWD) ? 2 * N : N;
    double *y = (double *)malloc(sizeof(double) * 32 * (size_t)(W > 0 ? W : 1));
    if (!y)
        return -2;
    for (int64_t m0 = 0; m0 < M; m0 += 32) {
        int64_t R = (M - m0 < 32) ? M - m0 : 32;
        for (int64_t r = 0; r < R; r++) {
            int64_t m = m0 + r;
            double *yr = y + r * W;
            for (int64_t j = 0; j < N; j++) {
                if (op == OP_QUANT) {
                    yr[j] = orc_bf16_decode(a[m * lda + j]);
                } else if (op == OP_FWD) {
                    yr[j] = orc_bf16_decode(fwd_value(act, a[m * lda + j], b[m * ldb + j]));
                } else {
                    uint16_t dg, du;
                    bwd_value(act, a[m * lda + j], b[m * ldb + j], c[m * ldc + j], &dg, &du);
                    yr[j] = orc_bf16_decode(dg);
                    yr[N + j] = orc_bf16_decode(du);
                }
            }
        }
        quant_slab(y, R, W, m0, layout, o);
    }
    free(y);
    return 0;
}

int orc_quant_2d(const uint16_t *x, int64_t ld_x, int64_t M, int64_t K, int layout,
                 uint8_t *q_row, int64_t ld_q_row, uint8_t *s_row, int64_t ld_s_row,
                 uint8_t *q_col, int64_t ld_q_col, uint8_t *s_col, int64_t ld_s_col)
{
    orc_out o = {q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col};
    return run(OP_QUANT, ORC_ACT_SILU, x, ld_x, NULL, 0, NULL, 0, M, K, layout, &o);
}

int orc_gated_fwd(int act, const uint16_t *gate, int64_t ld_gate, const uint16_t *up, int64_t ld_up,
                  int64_t M, int64_t N, int layout,
                  uint8_t *q_row, int64_t ld_q_row, uint8_t *s_row, int64_t ld_s_row,
                  uint8_t *q_col, int64_t ld_q_col, uint8_t *s_col, int64_t ld_s_col)
{
    orc_out o = {q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col};
    return run(OP_FWD, act, gate, ld_gate, up, ld_up, NULL, 0, M, N, layout, &o);
}

int orc_gated_bwd(int act, const uint16_t *dh, int64_t ld_dh, const uint16_t *gate, int64_t ld_gate,
                  const uint16_t *up, int64_t ld_up, int64_t M, int64_t N, int layout,
                  uint8_t *q_row, int64_t ld_q_row, uint8_t *s_row, int64_t ld_s_row,
                  uint8_t *q_col, int64_t ld_q_col, uint8_t *s_col, int64_t ld_s_col)
{
    orc_out o = {q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col};
    return run(OP_BWD, act, dh, ld_dh, gate, ld_gate, up, ld_up, M, N, layout, &o);
}

int orc_swiglu_fwd(const uint16_t *gate, int64_t ld_gate, const uint16_t *up, int64_t ld_up,
                   int64_t M, int64_t N, int layout,
                   uint8_t *q_row, int64_t ld_q_row, uint8_t *s_row, int64_t ld_s_row,
                   uint8_t *q_col, int64_t ld_q_col, uint8_t *s_col, int64_t ld_s_col)
{
    return orc_gated_fwd(ORC_ACT_SILU, gate, ld_gate, up, ld_up, M, N, layout,
                         q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col);
}

int orc_swiglu_bwd(const uint16_t *dh, int64_t ld_dh, const uint16_t *gate, int64_t ld_gate,
                   const uint16_t *up, int64_t ld_up, int64_t M, int64_t N, int layout,
                   uint8_t *q_row, int64_t ld_q_row, uint8_t *s_row, int64_t ld_s_row,
                   uint8_t *q_col, int64_t ld_q_col, uint8_t *s_col, int64_t ld_s_col)
{
    return orc_gated_bwd(ORC_ACT_SILU, dh, ld_dh, gate, ld_gate, up, ld_up, M, N, layout,
                         q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col);
}

/* 3D per-expert colwise quant [P3, Summary]: expert e is the [N, K] matrix
 * w + e*stride_e (row stride ld_w); its 32x1 blocks run along N.  Output q
 * is column-major per expert, q[e*N*K + k*N + n]; scales s[e*K*(N/32) +
 * k*(N/32) + n/32]. */
int orc_quant_3d_colwise(const uint16_t *w, int64_t E, int64_t N, int64_t K,
                         int64_t stride_e, int64_t ld_w, uint8_t *q, uint8_t *s)
{
    if (E < 0 || N < 0 || K < 0 || N % 32 != 0)
        return -1;
    double *blk = (double *)malloc(sizeof(double) * 32);
    if (!blk)
        return -2;
    for (int64_t e = 0; e < E; e++)
        for (int64_t k = 0; k < K; k++)
            for (int64_t n0 = 0; n0 < N; n0 += 32) {
                for (int64_t i = 0; i < 32; i++)
                    blk[i] = orc_bf16_decode(w[e * stride_e + (n0 + i) * ld_w + k]);
                orc_quant_block(blk, 32, 1, q + e * N * K + k * N + n0, 1,
                                s + e * K * (N / 32) + k * (N / 32) + n0 / 32);
            }
    free(blk);
    return 0;
}

/* ------------------------------------------------------ MX GEMM (consumer) */

/* The consumer of the casts: C = A B^T with both operands MXFP8 and stored
 * with K contiguous, as the casts emit them (rowwise output of [M, K] and
 * of [N, K], or the colwise output, whose rows run along the blocked axis).
 * [P4, Perf analysis] feeds such operands to a scaled (grouped) GEMM;
 * [P1, Summary] casts for exactly that consumer.
 *   a  [M, K] E4M3 codes, row stride lda;  sa [M, K/32] E8M0, row stride ld_sa
 *   b  [N, K] E4M3 codes, row stride ldb;  sb [N, K/32] E8M0, row stride ld_sb
 * Every element stands for decode(code) * 2^(scale - 127) (NaN for the NaN
 * codes or scale byte 255); C[m][n] is the plain sum over k of products of
 * those values, in double (each product is exact), and cabs[m][n] the sum
 * of their magnitudes (the scale of the rounding error any summation order
 * can make).  K must be a multiple of 32. */
static void mx_row_values(const uint8_t *q, const uint8_t *s, int64_t K, double *out)
{
    for (int64_t k = 0; k < K; k++)
        out[k] = orc_e4m3_decode(q[k]) * orc_e8m0_decode(s[k / 32]);
}

int orc_mx_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa,
                const uint8_t *b, int64_t ldb, const uint8_t *sb, int64_t ld_sb,
                int64_t M, int64_t N, int64_t K, double *c, int64_t ldc, double *cabs, int64_t ld_cabs)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0)
        return -1;
    double *bv = (double *)malloc(sizeof(double) * (size_t)(N * K + K + 1));
    if (!bv)
        return -2;
    double *av = bv + N * K;
    for (int64_t n = 0; n < N; n++)
        mx_row_values(b + n * ldb, sb + n * ld_sb, K, bv + n * K);
    for (int64_t m = 0; m < M; m++) {
        mx_row_values(a + m * lda, sa + m * ld_sa, K, av);
        for (int64_t n = 0; n < N; n++) {
            const double *bn = bv + n * K;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                acc += av[k] * bn[k];
                mag += fabs(av[k] * bn[k]);
            }
            c[m * ldc + n] = acc;
            if (cabs)
                cabs[m * ld_cabs + n] = mag;
        }
    }
    free(bv);
    return 0;
}

/* Grouped (2D x 3D) form of the consumer, as a mixture-of-experts layer runs
 * it [P4, Perf analysis: M=16640, G=4, N=8192, K=5120 grouped GEMMs]: the
 * rows of A are split into G consecutive groups by the cumulative end
 * offsets offs[0..G-1] (group g is rows [offs[g-1], offs[g]), offs[-1] = 0),
 * and group g multiplies expert g's operand b + g*stride_b [N, K] (scales
 * sb + g*stride_sb [N, K/32]).  Offsets are clamped so that groups stay
 * ordered and inside [0, M]: end_g = min(max(offs[g], start_g), M).  Rows
 * at or past the last group's end are not written. */
int orc_mx_grouped_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa,
                        const uint8_t *b, int64_t ldb, int64_t stride_b, const uint8_t *sb, int64_t ld_sb,
                        int64_t stride_sb, const int32_t *offs, int64_t G, int64_t M, int64_t N, int64_t K,
                        double *c, int64_t ldc, double *cabs, int64_t ld_cabs)
{
    if (G < 0 || M < 0 || N < 0 || K < 0 || K % 32 != 0)
        return -1;
    int64_t start = 0;
    for (int64_t g = 0; g < G; g++) {
        int64_t end = offs[g];
        if (end < start)
            end = start;
        if (end > M)
            end = M;
        int rc = orc_mx_gemm(a + start * lda, lda, sa + start * ld_sa, ld_sa, b + g * stride_b, ldb,
                             sb + g * stride_sb, ld_sb, end - start, N, K, c + start * ldc, ldc,
                             cabs ? cabs + start * ld_cabs : NULL, ld_cabs);
        if (rc != 0)
            return rc;
        start = end;
    }
    return 0;
}

/* ------------------------------------------------- token groups (wgrad) */

/* Token groups along the blocked axis of a colwise cast ([P4, Perf
 * analysis]: the weight-gradient GEMMs of a mixture-of-experts layer
 * contract over each expert's tokens; [P4, Summary and review comments]:
 * per-group scale buffers are sized by an upper bound on their padding).
 * offs[0..G-1] are cumulative group ends.  Each end is rounded down to a
 * multiple of 32 (a scale block never straddles two groups), negative ends
 * count as 0, and the ends are made non-decreasing and at most T:
 *   end_g = min(max(round32(offs[g]), end_{g-1}), T),  end_{-1} = 0.
 * Group g is tokens [end_{g-1}, end_g); tokens from end_{G-1} to T form a
 * tail group G.  starts/ends receive G + 1 entries (the tail included). */
int orc_group_bounds(const int32_t *offs, int64_t G, int64_t T, int64_t *starts, int64_t *ends)
{
    if (G < 0 || T < 0)
        return -1;
    int64_t prev = 0;
    for (int64_t g = 0; g <= G; g++) {
        int64_t e;
        if (g == G) {
            e = T;
        } else {
            e = offs[g] <= 0 ? 0 : ((int64_t)offs[g] / 32) * 32;
            if (e < prev)
                e = prev;
            if (e > T)
                e = T;
        }
        starts[g] = prev;
        ends[g] = e;
        prev = e;
    }
    return 0;
}

/* Position, in a per-group padded scale row, of the first block of the group
 * that starts at token s: 16 * (g + floor(s / 512)).  It is a multiple of 16
 * (every group's scales start 16-byte aligned), group g + 1's region starts
 * after group g's last block, and no position reaches T/32 + 16 G. */
int64_t orc_group_scale_base(int64_t g, int64_t s)
{
    return 16 * (g + s / 512);
}

/* Per-group padded layout of colwise scales: the plain scale matrix s
 * [rows, T/32] (row stride ld_s) rewritten so that the blocks of each group
 * (the tail group included) start at orc_group_scale_base in every row of
 * out (row stride ld_out >= T/32 + 16 G).  Positions no block maps to are
 * left as they are.  T must be a multiple of 32. */
int orc_pad_group_scales(const uint8_t *s, int64_t rows, int64_t ld_s, int64_t T, const int32_t *offs, int64_t G,
                         uint8_t *out, int64_t ld_out)
{
    if (rows < 0 || T < 0 || T % 32 != 0 || G < 0 || ld_out < T / 32 + 16 * G)
        return -1;
    int64_t *st = (int64_t *)malloc(sizeof(int64_t) * 2 * (size_t)(G + 1));
    if (!st)
        return -2;
    int64_t *en = st + G + 1;
    orc_group_bounds(offs, G, T, st, en);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g <= G; g++) {
            int64_t base = orc_group_scale_base(g, st[g]);
            for (int64_t b = st[g] / 32; b < en[g] / 32; b++)
                out[r * ld_out + base + (b - st[g] / 32)] = s[r * ld_s + b];
        }
    free(st);
    return 0;
}

/* K-grouped form of the consumer (the weight gradient): the contraction
 * axis (tokens, T of them) is split into the groups above, and group g's
 * result is the plain C_g = A_g B_g^T over its own tokens, where A_g is
 * columns [start_g, end_g) of a [M, T] (and B_g of b [N, T]), with scales
 * read from the per-group padded layout (group g's first block at
 * orc_group_scale_base).  c holds G results [M, N], c + g * stride_c.  An
 * empty group gives zeros.  T must be a multiple of 32. */
int orc_mx_grouped_gemm_k(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa,
                          const uint8_t *b, int64_t ldb, const uint8_t *sb, int64_t ld_sb,
                          const int32_t *offs, int64_t G, int64_t M, int64_t N, int64_t T,
                          double *c, int64_t ldc, int64_t stride_c, double *cabs)
{
    if (G < 0 || M < 0 || N < 0 || T < 0 || T % 32 != 0)
        return -1;
    int64_t *st = (int64_t *)malloc(sizeof(int64_t) * 2 * (size_t)(G + 1));
    if (!st)
        return -2;
    int64_t *en = st + G + 1;
    orc_group_bounds(offs, G, T, st, en);
    int rc = 0;
    for (int64_t g = 0; g < G && rc == 0; g++) {
        int64_t base = orc_group_scale_base(g, st[g]);
        rc = orc_mx_gemm(a + st[g], lda, sa + base, ld_sa, b + st[g], ldb, sb + base, ld_sb, M, N,
                         en[g] - st[g], c + g * stride_c, ldc, cabs ? cabs + g * stride_c : NULL, ldc);
    }
    free(st);
    return rc;
}
