/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) fused SwiGLU + MXFP8 cast library
 * (libmxfp8.so).
 *
 * MXFP8 here: blocks of 32 consecutive elements (along a row for the rowwise
 * 1x32 layout, along a column for the colwise 32x1 layout) share one E8M0
 * scale byte b, standing for 2^(b-127).  b is chosen by RCEIL: the smallest
 * power of two 2^k (k in [-127, 127]) with amax <= 448 * 2^k, where amax is
 * the block's largest magnitude.  Each element x is stored as the FP8 E4M3
 * (OCP E4M3FN) code of x * 2^(127-b), rounded to nearest with ties to even
 * and saturated to +-448.  A block holding any NaN or +-Inf gets scale byte
 * 255 and data 0x7F in all 32 places; an all-zero block gets byte 0.
 * Source: "Add swiglu + MXFP8 fused CuTe DSL kernel" (Summary; Numerics and
 * tests; commit message).
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE pointers.  bf16 inputs are raw 16-bit
 *    patterns; outputs are bytes (E4M3 codes, E8M0 scales).
 *  - Dimensions and leading dimensions (ld_*) are int64 element counts
 *    (bytes for the 1-byte outputs).  Every matrix is row-major with unit
 *    column stride and the given row stride.
 *  - layout is MXFP8_ROWWISE, MXFP8_COLWISE or MXFP8_BOTH.  Rowwise outputs
 *    are q_row [M, W] and s_row [M, W/32]; colwise outputs are q_col [W, M]
 *    (the column-major form of the [M, W] result, one output row per input
 *    column) and s_col [W, M/32].  Pointers of a layout that is not asked
 *    for are ignored and may be NULL.
 *  - The caller owns and allocates every buffer.  The library never
 *    allocates, frees, synchronizes or reads device memory from the host.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  The call returns once the kernel is enqueued.
 *  - Every argument is checked before any HIP call; a failed check returns a
 *    status and enqueues nothing.  M == 0 or a zero width returns MXFP8_OK
 *    and enqueues nothing.
 *  - Alignment: input pointers and E4M3 output pointers 16-byte aligned,
 *    bf16 ld_* multiples of 8 elements, E4M3 ld_* multiples of 16 bytes.
 *    Scale pointers and scale ld_* have no alignment requirement.
 *  - Colwise and both-layout calls (and the 3D cast) need bf16 input ld_*
 *    below 2^24 elements and output ld_* below 2^25 bytes (so M below
 *    about 33 million rows); larger strides return MXFP8_ERR_OVERFLOW.
 *  - Outputs must not alias inputs or each other (not checked).
 *  - Calls are thread-safe; the library keeps no mutable global state.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxfp8_status {
    MXFP8_OK = 0,
    MXFP8_ERR_NULL = 1,     /* a pointer the layout needs is NULL                 */
    MXFP8_ERR_SHAPE = 2,    /* negative dim, or a blocked dim not a multiple of 32 */
    MXFP8_ERR_STRIDE = 3,   /* ld smaller than the row, or not a vector multiple   */
    MXFP8_ERR_ALIGN = 4,    /* input or E4M3 output pointer not 16-byte aligned    */
    MXFP8_ERR_LAYOUT = 5,   /* layout flags not in {1, 2, 3}                       */
    MXFP8_ERR_OVERFLOW = 6, /* an extent overflows int64, or the grid is too large */
    MXFP8_ERR_LAUNCH = 7,   /* the HIP runtime refused the launch                  */
    MXFP8_ERR_ACT = 8       /* activation code not one of MXFP8_ACT_*              */
} mxfp8_status;

enum { MXFP8_ROWWISE = 1, MXFP8_COLWISE = 2, MXFP8_BOTH = 3 };

/* Gate activations of the gated family h = act(gate) * up (see
 * mxfp8_gated_fwd). */
enum { MXFP8_ACT_SILU = 0, MXFP8_ACT_GELU_TANH = 1, MXFP8_ACT_GELU = 2, MXFP8_ACT_RELU = 3 };

/*
 * Fused forward: h = silu(gate) * up, cast to MXFP8; h is never written.
 * "Add swiglu + MXFP8 fused CuTe DSL kernel", Summary and API: gate and up
 * are the two halves of the [M, 2N] fused w13 projection ([gate | up]), read
 * once.  Pass gate = w13, up = w13 + N, ld_gate = ld_up = 2N for that
 * layout, or two separate [M, N] tensors.
 *   gate, up : bf16 [M, N], row strides ld_gate, ld_up.
 *   W = N.  Requires N % 32 == 0; colwise also M % 32 == 0.
 * Values: h = bf16(bf16(silu(g)) * u) computed in fp32 (two bf16
 * roundings, as eager bf16 does); codes may differ from an exact evaluation
 * by one E4M3 step where fp32 rounding moves h across a bf16 boundary.
 */
mxfp8_status mxfp8_swiglu_fwd(const void *gate, int64_t ld_gate,
                              const void *up, int64_t ld_up,
                              int64_t M, int64_t N, int layout,
                              void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                              void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                              void *stream);

/*
 * Fused backward of h = silu(gate) * up for upstream gradient dh.
 * "Add swiglu + MXFP8 fused CuTe DSL kernel", API: returns [dGate | dUp]
 * concatenated along the width, so W = 2N: rowwise q_row [M, 2N] holds dGate
 * in columns [0, N) and dUp in [N, 2N); colwise q_col [2N, M] holds dGate in
 * rows [0, N) and dUp in rows [N, 2N).
 *   dh, gate, up : bf16 [M, N], row strides ld_dh, ld_gate, ld_up.
 *   Requires N % 32 == 0; colwise also M % 32 == 0.
 * Values (eager bf16 autograd): s = bf16(silu(g)), du = bf16(dh * s),
 * ds = bf16(dh * up), dg = bf16(ds * sig(g) * (1 + g * (1 - sig(g)))).
 */
mxfp8_status mxfp8_swiglu_bwd(const void *dh, int64_t ld_dh,
                              const void *gate, int64_t ld_gate,
                              const void *up, int64_t ld_up,
                              int64_t M, int64_t N, int layout,
                              void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                              void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                              void *stream);

/*
 * The fused casts for other gated activations: h = act(gate) * up, with act
 * chosen by `act` (MXFP8_ACT_*).  "Add swiglu + MXFP8 fused CuTe DSL
 * kernel", API (the activation is a compile-time policy of one kernel
 * source) and Follow-ups (more gated activations planned; none named).
 * Taken here:
 *   MXFP8_ACT_SILU       silu(g) = g sigmoid(g)  (same as mxfp8_swiglu_*)
 *   MXFP8_ACT_GELU_TANH  0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))
 *   MXFP8_ACT_GELU       g Phi(g), Phi the standard normal cdf
 *   MXFP8_ACT_RELU       max(g, 0) (+0 for g <= 0, NaN kept)
 * Arguments, layouts, outputs and the [dGate | dUp] order are exactly those
 * of mxfp8_swiglu_fwd / mxfp8_swiglu_bwd.  Values follow the same eager
 * bf16 rounding sites with act in place of silu: a = bf16(act(g)),
 * h = bf16(a * up); du = bf16(dh * a), da = bf16(dh * up),
 * dg = bf16(da * act'(g)), act' the textbook derivative (ReLU's is 0 for
 * g <= 0, 1 otherwise).  Computed in fp32; codes may differ from an exact
 * evaluation by one E4M3 step.  An unknown `act` returns MXFP8_ERR_ACT
 * before any other check.
 */
mxfp8_status mxfp8_gated_fwd(int act, const void *gate, int64_t ld_gate,
                             const void *up, int64_t ld_up,
                             int64_t M, int64_t N, int layout,
                             void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                             void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                             void *stream);
mxfp8_status mxfp8_gated_bwd(int act, const void *dh, int64_t ld_dh,
                             const void *gate, int64_t ld_gate,
                             const void *up, int64_t ld_up,
                             int64_t M, int64_t N, int layout,
                             void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                             void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                             void *stream);

/*
 * Plain MXFP8 cast of a bf16 matrix x [M, K] (row stride ld_x): the
 * standalone quantizer the fused kernels are bit-compatible with ("Add
 * swiglu + MXFP8 fused CuTe DSL kernel", Summary), and the 2D colwise
 * ("dim1") cast ("[mxfp8 moe training] add compile support", Perf analysis).
 *   W = K.  Rowwise requires K % 32 == 0; colwise requires M % 32 == 0 and
 *   K % 8 == 0.  Results are exact (bit-identical to the definition).
 */
mxfp8_status mxfp8_quant_2d(const void *x, int64_t ld_x, int64_t M, int64_t K, int layout,
                            void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                            void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                            void *stream);

/*
 * 3D per-expert colwise cast of expert weights w (E, N, K), bf16: expert e
 * is the [N, K] matrix at w + e * stride_e with row stride ld_w (packed:
 * stride_e = N * K, ld_w = K).  Blocks of 32 run along N.  Output is
 * column-major per expert: q (E, K, N) packed, element (e, n, k) at
 * q[e*K*N + k*N + n]; scales s (E, K, N/32) packed, at s[e*K*(N/32) +
 * k*(N/32) + n/32].  One launch covers all experts.
 * "[mxfp8 moe training] update 3d quant colwise scaling kernel to use single
 * input/output TMA descriptors", Summary.
 *   Requires N % 32 == 0, K % 8 == 0, stride_e >= N * ld_w.  Exact results.
 */
mxfp8_status mxfp8_quant_3d_colwise(const void *w, int64_t E, int64_t N, int64_t K,
                                    int64_t stride_e, int64_t ld_w,
                                    void *q, void *s, void *stream);

/*
 * The activation alone, written as bf16 instead of being cast: the first
 * kernel of the unfused two-kernel pipeline (activation, then
 * mxfp8_quant_2d) that the fused calls replace.  "Add swiglu + MXFP8 fused
 * CuTe DSL kernel", Performance: the baseline arm is a fused activation
 * kernel followed by the standalone quantizer.  The values are the ones the
 * fused calls quantize, so mxfp8_quant_2d of this output equals the fused
 * result bit for bit.
 *   gate, up, dh : bf16 [M, N] as in the fused calls; N % 8 == 0.
 *   h            : bf16 [M, N], row stride ld_h (multiple of 8, >= N).
 *   dgdu         : bf16 [M, 2N] = [dGate | dUp], row stride ld_dgdu (>= 2N).
 * Same pointer, alignment and status conventions as above.
 */
mxfp8_status mxfp8_swiglu_fwd_bf16(const void *gate, int64_t ld_gate, const void *up, int64_t ld_up,
                                   int64_t M, int64_t N, void *h, int64_t ld_h, void *stream);
mxfp8_status mxfp8_swiglu_bwd_bf16(const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate,
                                   const void *up, int64_t ld_up, int64_t M, int64_t N,
                                   void *dgdu, int64_t ld_dgdu, void *stream);

/*
 * The consumer of the casts: C = A B^T on MXFP8 operands, with gfx950's
 * block-scaled matrix cores.  "[mxfp8 moe training] add compile support",
 * Perf analysis: the cast outputs feed a scaled (grouped) GEMM.
 *   a  : E4M3 [M, K], row stride lda (bytes, multiple of 16, >= K)
 *   sa : E8M0 [M, K/32], row stride ld_sa (>= K/32), plain row-major
 *   b  : E4M3 [N, K], row stride ldb (multiple of 16, >= K)
 *   sb : E8M0 [N, K/32], row stride ld_sb (>= K/32)
 *   c  : fp32 [M, N], row stride ldc (elements, >= N), 4-byte aligned
 * Both operands keep K contiguous: the rowwise output of an [M, K] matrix,
 * or the colwise output of a [K, N] matrix (q_col [N, K] with s_col), used
 * as is.  Element (m, k) of A is worth decode(a) * 2^(sa - 127); C[m][n] is
 * the sum over k of the products.  Each product is exact; within each
 * 64-element K step the matrix core aligns the products to the largest and
 * truncates each 13 bits below that one's leading bit, then adds the step's
 * sum into an fp32 accumulator.  So C is within sum_steps 64 * 2^-13 *
 * (largest |product| of the step) + (K/64) * 2^-24 * sum |products| of the
 * exact value.  K must be a multiple of 32 (whole blocks); M, N any.  a and
 * b 16-byte aligned.  Scales may sit at any byte offset; scale rows that
 * start 16-byte aligned (sa, sb, ld_sa, ld_sb, and stride_sb in the grouped
 * form, all multiples of 16, as the casts' outputs are when K is a multiple
 * of 512) are fetched 16 bytes at a time straight into shared memory,
 * others as 4-byte words through registers (a little slower), and the
 * blocks of a last group of fewer than 16 byte by byte.
 * A NaN code or a scale byte of 255 makes the sums it enters NaN.
 */
mxfp8_status mxfp8_gemm(const void *a, int64_t lda, const void *sa, int64_t ld_sa,
                        const void *b, int64_t ldb, const void *sb, int64_t ld_sb,
                        int64_t M, int64_t N, int64_t K, float *c, int64_t ldc, void *stream);

/*
 * Grouped (2D x 3D) form of mxfp8_gemm, as a mixture-of-experts layer runs
 * it: "[mxfp8 moe training] add compile support", Perf analysis (grouped
 * GEMMs at M=16640, G=4, N=8192, K=5120) and Summary (size buffers by an
 * upper bound instead of reading the last offset back to the host).
 *   a, sa     : as in mxfp8_gemm, [M, K] and [M, K/32]
 *   b, sb     : G experts; expert g is b + g * stride_b [N, K] (row stride
 *               ldb) with scales sb + g * stride_sb [N, K/32] (ld_sb);
 *               stride_b a multiple of 16 and >= (N-1)*ldb + K
 *   offsets   : DEVICE int32 [G], cumulative end rows: group g is rows
 *               [offsets[g-1], offsets[g]) of A and C (offsets[-1] = 0)
 *   c         : fp32 [M, N]; rows of group g get A_g B_g^T
 * The offsets are read on the GPU only; the launch covers M/256 + G row
 * tiles, an upper bound.  They are clamped into ordered groups inside
 * [0, M] (end_g = min(max(offsets[g], end_{g-1}), M)), so malformed
 * offsets cannot cause out-of-range accesses; rows past the last group's
 * end are not written.  1 <= G <= 1024; G == 0 returns MXFP8_OK and
 * launches nothing.  Same numerics as mxfp8_gemm.
 */
mxfp8_status mxfp8_grouped_gemm(const void *a, int64_t lda, const void *sa, int64_t ld_sa,
                                const void *b, int64_t ldb, int64_t stride_b,
                                const void *sb, int64_t ld_sb, int64_t stride_sb,
                                const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K,
                                float *c, int64_t ldc, void *stream);

/*
 * Token groups and the per-group padded colwise scale layout (the weight-
 * gradient side of a mixture-of-experts step).  "[mxfp8 moe training] add
 * compile support", Perf analysis (the colwise casts feed grouped GEMMs
 * that contract over each expert's tokens) and Summary with its review
 * comments (per-group scale buffers sized by an upper bound on their
 * padding, with the offsets left on the device).
 *
 * The M rows (tokens) of a cast are split into groups by group_ends, a
 * DEVICE int32 array of n_groups cumulative ends, read on the GPU only.  Each
 * end is rounded down to a multiple of 32 (a scale block never straddles two
 * groups; real group sizes should be multiples of 32), negative ends count
 * as 0, and the ends are made non-decreasing and at most M:
 *   end_g = min(max(round32(group_ends[g]), end_{g-1}), M),  end_{-1} = 0.
 * Group g is rows [end_{g-1}, end_g); rows from end_{n-1} to M form a tail
 * group n.  In every colwise scale row, the scale of the 32-row block that
 * starts at row t of group g (which starts at row s) is stored at position
 *   16 * (g + floor(s / 512)) + (t - s) / 32,
 * so every group's scales start 16-byte aligned, groups never overlap, and
 * every position is below M/32 + 16 * n_groups: ld_s_col must be at least
 * that.  Positions no block maps to are not written.  With one group
 * ending at M the layout is the plain one.  Any group_ends values give
 * in-range positions.
 *
 * The grouped casts are the casts above with that colwise scale layout;
 * everything else (codes, rowwise outputs, checks) is unchanged.  Extra
 * checks: 1 <= n_groups <= 1024 (else MXFP8_ERR_SHAPE), group_ends non-NULL
 * (MXFP8_ERR_NULL) and 4-byte aligned (MXFP8_ERR_ALIGN), M < 2^31 - 256
 * (MXFP8_ERR_OVERFLOW).
 */
mxfp8_status mxfp8_gated_fwd_grouped(int act, const void *gate, int64_t ld_gate,
                                     const void *up, int64_t ld_up, int64_t M, int64_t N, int layout,
                                     void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                                     void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                                     const int32_t *group_ends, int64_t n_groups, void *stream);
mxfp8_status mxfp8_gated_bwd_grouped(int act, const void *dh, int64_t ld_dh,
                                     const void *gate, int64_t ld_gate, const void *up, int64_t ld_up,
                                     int64_t M, int64_t N, int layout,
                                     void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                                     void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                                     const int32_t *group_ends, int64_t n_groups, void *stream);
mxfp8_status mxfp8_quant_2d_grouped(const void *x, int64_t ld_x, int64_t M, int64_t K, int layout,
                                    void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                                    void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                                    const int32_t *group_ends, int64_t n_groups, void *stream);

/*
 * K-grouped form of mxfp8_gemm: the weight gradient, which contracts over
 * each group's tokens ("[mxfp8 moe training] add compile support", Perf
 * analysis).  a [M, T] and b [N, T] hold E4M3 codes with the T tokens along
 * the rows (the colwise outputs of two [T, *] matrices); their scales sa
 * [M, ld_sa] and sb [N, ld_sb] are in the per-group padded layout above
 * (the grouped casts' colwise scales), for the same group_ends.  For each of
 * the G groups (bounds as above, with T in place of M; the tail group is
 * not used):
 *   C_g = A[:, start_g:end_g] B[:, start_g:end_g]^T,  fp32 [M, N],
 * written at c + g * stride_c (row stride ldc).  An empty group gives zeros.
 *   Requires T % 32 == 0, lda, ldb >= T and multiples of 16, ld_sa, ld_sb >=
 *   T/32 + 16 G, stride_c >= (M-1)*ldc + N, 1 <= G <= 1024 (G == 0 returns
 *   MXFP8_OK and launches nothing).  group_ends is read on the GPU only.
 * Same numerics as mxfp8_gemm; with every ld_sa, ld_sb a multiple of 16 the
 * scales of every group are fetched 16 bytes at a time.
 */
mxfp8_status mxfp8_grouped_gemm_k(const void *a, int64_t lda, const void *sa, int64_t ld_sa,
                                  const void *b, int64_t ldb, const void *sb, int64_t ld_sb,
                                  const int32_t *group_ends, int64_t G, int64_t M, int64_t N, int64_t T,
                                  float *c, int64_t ldc, int64_t stride_c, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *mxfp8_status_str(mxfp8_status status);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
