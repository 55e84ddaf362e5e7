// mxfp8.hip -- C ABI of libmxfp8.so: argument checks and kernel launches.
//
// Every entry point validates its arguments on the host before touching
// the HIP runtime, picks one kernel instantiation, sizes its grid and
// enqueues it on the caller's stream.  Nothing is allocated, synchronized
// or read back.  API shape: "Add swiglu + MXFP8 fused CuTe DSL kernel",
// API (forward/backward with rowwise/colwise switches, fixed-arity
// outputs; one kernel source per activation) and Numerics and tests
// (launcher guards on sizes and pointer alignment, each error path reachable
// without a device).
#include <hip/hip_runtime.h>
#include <algorithm>
#include <limits.h>
#include <stdint.h>

#include "mx_gemm.hpp"
#include "mx_kernels.hpp"
#include "mxfp8.h"

namespace {

using mx::Args;

constexpr int kRowUnroll = 4;

enum class Kind { Quant, Fwd, Bwd };

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_add_overflow(a, b, r); }

// Largest offset touched in a [rows, cols] matrix with row stride ld, plus
// one, must fit int64 (with room for a batch offset added on top).
bool extent_ok(int64_t rows, int64_t cols, int64_t ld) {
  if (rows == 0 || cols == 0) return true;
  int64_t r;
  return mul_ok(rows - 1, ld, &r) && add_ok(r, cols, &r) && r < (INT64_MAX >> 2);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool act_ok(int act) { return act >= MXFP8_ACT_SILU && act <= MXFP8_ACT_RELU; }

// The colwise kernel addresses each tile from a wave-uniform base with
// 32-bit per-lane offsets that reach (tile rows - 1) input / q_row / s_row
// strides and (tile columns - 1) q_col / s_col strides: keep them below
// 2^32 bytes.
constexpr int64_t kMaxLdIn = (int64_t(1) << 31) / mx::kTM;                                   // bf16 elements
constexpr int64_t kMaxLdOut = (int64_t(1) << 32) / (mx::kTM > mx::kTC ? mx::kTM : mx::kTC);  // bytes

// Tile order of the colwise kernel: bands of row tiles, row tiles fastest
// inside a band.  A colwise-only launch runs bands of 128 row tiles, so the
// tiles in flight extend each q_col output row in long contiguous runs; a
// both-layout launch also writes rowwise lines, which favour more column
// tiles in flight, and runs best with bands of 32 (both measured at
// 131072 x 8192 on MI355X).  Both-layout launches of at most 128 row tiles
// (each XCD's range then holds at most 16 row tiles of every column) run
// 1-1.5 points faster with bands of 8 (4096 and 16384 rows, N = 7168);
// from 256 row tiles on, bands of 32 win by 6-10 points.
#ifndef MX_BAND_COL
#define MX_BAND_COL 128
#endif
#ifndef MX_BAND_BOTH
#define MX_BAND_BOTH 32
#endif
constexpr int32_t kBandCol = MX_BAND_COL, kBandBoth = MX_BAND_BOTH, kBandBothSmall = 8;
constexpr int64_t kSmallBandRowTiles = 128;

bool tile_offsets_ok(const int64_t *ld_in, int n_in, int64_t ld_q_row, int64_t ld_s_row, int64_t ld_q_col,
                     int64_t ld_s_col) {
  for (int j = 0; j < n_in; j++)
    if (ld_in[j] >= kMaxLdIn) return false;
  return ld_q_row < kMaxLdOut && ld_s_row < kMaxLdOut && ld_q_col < kMaxLdOut && ld_s_col < kMaxLdOut;
}

// Checks shared by the 2-D entry points.  W = out_mult * N is the output
// width.  `blocked_cols` says whether the rowwise 32-blocks run along N.
mxfp8_status check_2d(Kind kind, const void *const *in, const int64_t *ld_in, int n_in, int64_t M,
                      int64_t N, int layout, const void *q_row, int64_t ld_q_row, const void *s_row,
                      int64_t ld_s_row, const void *q_col, int64_t ld_q_col, const void *s_col,
                      int64_t ld_s_col, int64_t n_groups = 0) {
  if (layout < MXFP8_ROWWISE || layout > MXFP8_BOTH) return MXFP8_ERR_LAYOUT;
  if (M < 0 || N < 0) return MXFP8_ERR_SHAPE;
  const bool rows = layout & MXFP8_ROWWISE, cols = layout & MXFP8_COLWISE;
  if (kind != Kind::Quant && N % 32 != 0) return MXFP8_ERR_SHAPE;
  if (kind == Kind::Quant && rows && N % 32 != 0) return MXFP8_ERR_SHAPE;
  if (kind == Kind::Quant && N % 8 != 0) return MXFP8_ERR_SHAPE;
  if (cols && M % 32 != 0) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  const int64_t W = (kind == Kind::Bwd ? 2 : 1) * N;
  for (int j = 0; j < n_in; j++)
    if (!in[j]) return MXFP8_ERR_NULL;
  if (rows && (!q_row || !s_row)) return MXFP8_ERR_NULL;
  if (cols && (!q_col || !s_col)) return MXFP8_ERR_NULL;
  for (int j = 0; j < n_in; j++)
    if (ld_in[j] < N || ld_in[j] % 8 != 0) return MXFP8_ERR_STRIDE;
  if (rows && (ld_q_row < W || ld_q_row % 16 != 0 || ld_s_row < W / 32)) return MXFP8_ERR_STRIDE;
  // colwise scale rows: M/32 blocks, or with token groups the per-group
  // padded layout, whose positions stay below M/32 + 16 groups
  const int64_t s_col_w = M / 32 + 16 * n_groups;
  if (cols && (ld_q_col < M || ld_q_col % 16 != 0 || ld_s_col < s_col_w)) return MXFP8_ERR_STRIDE;
  for (int j = 0; j < n_in; j++)
    if (!aligned16(in[j])) return MXFP8_ERR_ALIGN;
  if (rows && !aligned16(q_row)) return MXFP8_ERR_ALIGN;
  if (cols && !aligned16(q_col)) return MXFP8_ERR_ALIGN;
  for (int j = 0; j < n_in; j++)
    if (!extent_ok(M, N, ld_in[j])) return MXFP8_ERR_OVERFLOW;
  if (rows && (!extent_ok(M, W, ld_q_row) || !extent_ok(M, W / 32, ld_s_row))) return MXFP8_ERR_OVERFLOW;
  if (cols && (!extent_ok(W, M, ld_q_col) || !extent_ok(W, s_col_w, ld_s_col))) return MXFP8_ERR_OVERFLOW;
  if (cols && !tile_offsets_ok(ld_in, n_in, rows ? ld_q_row : 0, rows ? ld_s_row : 0, ld_q_col, ld_s_col))
    return MXFP8_ERR_OVERFLOW;
  return MXFP8_OK;
}

mxfp8_status launch(const void *kernel, int64_t blocks, int threads, const Args &a, void *stream,
                    unsigned dyn_lds = 0) {
  // Grid x is limited to 2^32 - 1 work-items; keep well inside it.
  if (blocks <= 0 || blocks > (int64_t)INT32_MAX / threads) return MXFP8_ERR_OVERFLOW;
  Args copy = a;
  void *kargs[] = {&copy};
  hipError_t err =
      hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3(threads), kargs, dyn_lds, (hipStream_t)stream);
  return err == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

// Occupancy cap of a colwise-only launch.  The tiled kernel's own LDS lets
// four workgroups share a CU (two for the backward, whose tile holds both
// output halves).  On the largest grids fewer tiles in flight per XCD stream
// faster (MI355X, colwise-only): the 2D casts at 131072 x 8192 run 2-3% faster
// at two workgroups per CU, the 3D cast of 16 or 64 experts of 8192 x 5120 1%
// faster at three; smaller grids lose from it.  The cap is applied by
// requesting dynamic LDS that the kernel does not touch: with 160 KiB of LDS
// per CU, more than 160 KiB / (cap + 1) per workgroup leaves room for `cap`.
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int64_t kCapTiles2d = 32768, kCapTiles3d = 40960;  // grid sizes where the caps were measured to pay
// Both-layout launches of the fused forward (gate and up in, one output
// half) fit four workgroups per CU; three stream faster on grids of at
// least 4096 tiles (131072 x 8192: +0.7 points, 16384 x 7168: +1.2), while
// 4096 x 2048 (512 tiles) loses a point and the plain cast gains nothing.
constexpr int64_t kCapTilesFwdBoth = 4096;

unsigned lds_pad_for_cap(int cap, size_t static_lds) {
  if (cap <= 0) return 0;
  const int64_t pad = kLdsPerCu / (cap + 1) + 1 - (int64_t)static_lds;
  return pad <= 0 ? 0u : (unsigned)((pad + 1023) / 1024 * 1024);
}

// Launch of the colwise / both-layout kernel over `batches` stacked [M, N]
// problems (batches > 1 only for the 3D cast); `cap` is the workgroups per
// CU (0: as many as fit).
template <class Op, bool GROUPS = false>
mxfp8_status launch_colwise(Args a, bool rows, int64_t batches, void *stream, int cap = 0) {
  const int64_t n_rt = (a.M + mx::kTM - 1) / mx::kTM, n_ct = (a.N + mx::kTC - 1) / mx::kTC;
  if (n_rt > INT32_MAX || n_ct > INT32_MAX) return MXFP8_ERR_OVERFLOW;
  a.n_rt = (int32_t)n_rt;
  a.n_ct = (int32_t)n_ct;
  int64_t blocks, per;
  if (!mul_ok(n_rt, n_ct, &per) || per > UINT32_MAX || !mul_ok(per, batches, &blocks)) return MXFP8_ERR_OVERFLOW;
  const void *k =
      rows ? (const void *)&mx::k_tiled<Op, true, GROUPS> : (const void *)&mx::k_tiled<Op, false, GROUPS>;
  // band <= n_rt keeps band * n_ct (computed in 32 bits in the kernel) <= per
  const int64_t band = !rows ? kBandCol : n_rt <= kSmallBandRowTiles ? kBandBothSmall : kBandBoth;
  a.band = (int32_t)std::min<int64_t>(band, n_rt);
  const unsigned pad =
      lds_pad_for_cap(cap, rows ? mx::tiled_lds_bytes<Op, true, GROUPS>() : mx::tiled_lds_bytes<Op, false, GROUPS>());
  return launch(k, blocks, mx::kNT, a, stream, pad);
}

// Checks of the bf16 value entry points: inputs as for the fused calls,
// one bf16 output [M, W] with row stride ld_out.
mxfp8_status check_values(const void *const *in, const int64_t *ld_in, int n_in, int64_t M, int64_t N,
                          const void *out, int64_t ld_out, int64_t W) {
  if (M < 0 || N < 0 || N % 8 != 0) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  for (int j = 0; j < n_in; j++)
    if (!in[j]) return MXFP8_ERR_NULL;
  if (!out) return MXFP8_ERR_NULL;
  for (int j = 0; j < n_in; j++)
    if (ld_in[j] < N || ld_in[j] % 8 != 0) return MXFP8_ERR_STRIDE;
  if (ld_out < W || ld_out % 8 != 0) return MXFP8_ERR_STRIDE;
  for (int j = 0; j < n_in; j++)
    if (!aligned16(in[j])) return MXFP8_ERR_ALIGN;
  if (!aligned16(out)) return MXFP8_ERR_ALIGN;
  for (int j = 0; j < n_in; j++)
    if (!extent_ok(M, N, ld_in[j])) return MXFP8_ERR_OVERFLOW;
  if (!extent_ok(M, W, ld_out)) return MXFP8_ERR_OVERFLOW;
  return MXFP8_OK;
}

template <class Op>
mxfp8_status launch_values(const Args &a, void *dst, int64_t ld_dst, void *stream) {
  const int64_t blocks = (a.M + mx::kRowWaves - 1) / mx::kRowWaves;
  if (blocks <= 0 || blocks > (int64_t)INT32_MAX / 256) return MXFP8_ERR_OVERFLOW;
  Args copy = a;
  uint16_t *d = static_cast<uint16_t *>(dst);
  void *kargs[] = {&copy, &d, &ld_dst};
  hipError_t err = hipLaunchKernel((const void *)&mx::k_values<Op, kRowUnroll>, dim3((unsigned)blocks), dim3(256),
                                   kargs, 0, (hipStream_t)stream);
  return err == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

template <class Op>
mxfp8_status dispatch_2d(const Args &a, int layout, void *stream) {
  if (layout == MXFP8_ROWWISE) {
    const int64_t blocks = (a.M + mx::kRowWaves - 1) / mx::kRowWaves;
    return launch((const void *)&mx::k_rowwise<Op, kRowUnroll>, blocks, 256, a, stream);
  }
  const int64_t tiles = ((a.M + mx::kTM - 1) / mx::kTM) * ((a.N + mx::kTC - 1) / mx::kTC);
  const bool both = layout == MXFP8_BOTH;
  const bool fused_fwd = Op::IN == 2 && Op::OUT == 1;
  const int cap = !both ? (tiles >= kCapTiles2d ? 2 : 0) : (fused_fwd && tiles >= kCapTilesFwdBoth ? 3 : 0);
  if (a.n_grp > 0) return launch_colwise<Op, true>(a, both, 1, stream, cap);
  return launch_colwise<Op>(a, both, 1, stream, cap);
}

// Checks of the token-group arguments of the grouped casts: 1..kMaxGroups
// cumulative ends in device memory (4-byte aligned); token indices are
// 32-bit in the kernel.
mxfp8_status check_groups(const int32_t *group_ends, int64_t n_groups, int64_t M) {
  if (n_groups < 1 || n_groups > mx::kMaxGroups) return MXFP8_ERR_SHAPE;
  if (!group_ends) return MXFP8_ERR_NULL;
  if (((uintptr_t)group_ends & 3u) != 0) return MXFP8_ERR_ALIGN;
  if (M > INT32_MAX - 256) return MXFP8_ERR_OVERFLOW;
  return MXFP8_OK;
}

Args make_args(const void *const *in, const int64_t *ld_in, int n_in, int64_t M, int64_t N, void *q_row,
               int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col, void *s_col,
               int64_t ld_s_col) {
  Args a{};
  for (int j = 0; j < n_in; j++) {
    a.in[j] = static_cast<const uint16_t *>(in[j]);
    a.ld_in[j] = ld_in[j];
  }
  a.M = M;
  a.N = N;
  a.q_row = static_cast<uint8_t *>(q_row);
  a.ld_q_row = ld_q_row;
  a.s_row = static_cast<uint8_t *>(s_row);
  a.ld_s_row = ld_s_row;
  a.q_col = static_cast<uint8_t *>(q_col);
  a.ld_q_col = ld_q_col;
  a.s_col = static_cast<uint8_t *>(s_col);
  a.ld_s_col = ld_s_col;
  return a;
}


mxfp8_status gated_fwd_impl(int act, const void *gate, int64_t ld_gate, const void *up, int64_t ld_up, int64_t M,
                            int64_t N, int layout, void *q_row, int64_t ld_q_row, void *s_row, int64_t ld_s_row,
                            void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col, const int32_t *grp,
                            int64_t n_grp, void *stream) {
  if (!act_ok(act)) return MXFP8_ERR_ACT;
  const void *in[2] = {gate, up};
  const int64_t ld[2] = {ld_gate, ld_up};
  mxfp8_status st = check_2d(Kind::Fwd, in, ld, 2, M, N, layout, q_row, ld_q_row, s_row, ld_s_row, q_col,
                             ld_q_col, s_col, ld_s_col, n_grp);
  if (st != MXFP8_OK || M == 0 || N == 0) return st;
  Args a = make_args(in, ld, 2, M, N, q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col);
  a.grp = grp;
  a.n_grp = (int32_t)n_grp;
  switch (act) {
    case MXFP8_ACT_SILU: return dispatch_2d<mx::OpFwd>(a, layout, stream);
    case MXFP8_ACT_GELU_TANH: return dispatch_2d<mx::GatedFwd<mx::ActGeluTanh>>(a, layout, stream);
    case MXFP8_ACT_GELU: return dispatch_2d<mx::GatedFwd<mx::ActGelu>>(a, layout, stream);
    default: return dispatch_2d<mx::GatedFwd<mx::ActRelu>>(a, layout, stream);
  }
}

mxfp8_status gated_bwd_impl(int act, const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate,
                            const void *up, int64_t ld_up, int64_t M, int64_t N, int layout, void *q_row,
                            int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                            void *s_col, int64_t ld_s_col, const int32_t *grp, int64_t n_grp, void *stream) {
  if (!act_ok(act)) return MXFP8_ERR_ACT;
  const void *in[3] = {dh, gate, up};
  const int64_t ld[3] = {ld_dh, ld_gate, ld_up};
  mxfp8_status st = check_2d(Kind::Bwd, in, ld, 3, M, N, layout, q_row, ld_q_row, s_row, ld_s_row, q_col,
                             ld_q_col, s_col, ld_s_col, n_grp);
  if (st != MXFP8_OK || M == 0 || N == 0) return st;
  Args a = make_args(in, ld, 3, M, N, q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col);
  a.grp = grp;
  a.n_grp = (int32_t)n_grp;
  switch (act) {
    case MXFP8_ACT_SILU: return dispatch_2d<mx::OpBwd>(a, layout, stream);
    case MXFP8_ACT_GELU_TANH: return dispatch_2d<mx::GatedBwd<mx::ActGeluTanh>>(a, layout, stream);
    case MXFP8_ACT_GELU: return dispatch_2d<mx::GatedBwd<mx::ActGelu>>(a, layout, stream);
    default: return dispatch_2d<mx::GatedBwd<mx::ActRelu>>(a, layout, stream);
  }
}

mxfp8_status quant_2d_impl(const void *x, int64_t ld_x, int64_t M, int64_t K, int layout, void *q_row,
                           int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                           void *s_col, int64_t ld_s_col, const int32_t *grp, int64_t n_grp, void *stream) {
  const void *in[1] = {x};
  const int64_t ld[1] = {ld_x};
  mxfp8_status st = check_2d(Kind::Quant, in, ld, 1, M, K, layout, q_row, ld_q_row, s_row, ld_s_row, q_col,
                             ld_q_col, s_col, ld_s_col, n_grp);
  if (st != MXFP8_OK || M == 0 || K == 0) return st;
  Args a = make_args(in, ld, 1, M, K, q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col);
  a.grp = grp;
  a.n_grp = (int32_t)n_grp;
  return dispatch_2d<mx::OpQuant>(a, layout, stream);
}

}  // namespace

extern "C" {

mxfp8_status mxfp8_gated_fwd(int act, const void *gate, int64_t ld_gate, const void *up, int64_t ld_up,
                             int64_t M, int64_t N, int layout, void *q_row, int64_t ld_q_row, void *s_row,
                             int64_t ld_s_row, void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                             void *stream) {
  return gated_fwd_impl(act, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row, ld_s_row, q_col,
                        ld_q_col, s_col, ld_s_col, nullptr, 0, stream);
}

mxfp8_status mxfp8_gated_bwd(int act, const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate,
                             const void *up, int64_t ld_up, int64_t M, int64_t N, int layout, void *q_row,
                             int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                             void *s_col, int64_t ld_s_col, void *stream) {
  return gated_bwd_impl(act, dh, ld_dh, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row, ld_s_row,
                        q_col, ld_q_col, s_col, ld_s_col, nullptr, 0, stream);
}

mxfp8_status mxfp8_gated_fwd_grouped(int act, const void *gate, int64_t ld_gate, const void *up, int64_t ld_up,
                                     int64_t M, int64_t N, int layout, void *q_row, int64_t ld_q_row, void *s_row,
                                     int64_t ld_s_row, void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                                     const int32_t *group_ends, int64_t n_groups, void *stream) {
  if (!act_ok(act)) return MXFP8_ERR_ACT;
  mxfp8_status st = check_groups(group_ends, n_groups, M);
  if (st != MXFP8_OK) return st;
  return gated_fwd_impl(act, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row, ld_s_row, q_col,
                        ld_q_col, s_col, ld_s_col, group_ends, n_groups, stream);
}

mxfp8_status mxfp8_gated_bwd_grouped(int act, const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate,
                                     const void *up, int64_t ld_up, int64_t M, int64_t N, int layout, void *q_row,
                                     int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                                     void *s_col, int64_t ld_s_col, const int32_t *group_ends, int64_t n_groups,
                                     void *stream) {
  if (!act_ok(act)) return MXFP8_ERR_ACT;
  mxfp8_status st = check_groups(group_ends, n_groups, M);
  if (st != MXFP8_OK) return st;
  return gated_bwd_impl(act, dh, ld_dh, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row, ld_s_row,
                        q_col, ld_q_col, s_col, ld_s_col, group_ends, n_groups, stream);
}

mxfp8_status mxfp8_swiglu_fwd(const void *gate, int64_t ld_gate, const void *up, int64_t ld_up, int64_t M,
                              int64_t N, int layout, void *q_row, int64_t ld_q_row, void *s_row,
                              int64_t ld_s_row, void *q_col, int64_t ld_q_col, void *s_col, int64_t ld_s_col,
                              void *stream) {
  return mxfp8_gated_fwd(MXFP8_ACT_SILU, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row, ld_s_row,
                         q_col, ld_q_col, s_col, ld_s_col, stream);
}

mxfp8_status mxfp8_swiglu_bwd(const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate, const void *up,
                              int64_t ld_up, int64_t M, int64_t N, int layout, void *q_row, int64_t ld_q_row,
                              void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col, void *s_col,
                              int64_t ld_s_col, void *stream) {
  return mxfp8_gated_bwd(MXFP8_ACT_SILU, dh, ld_dh, gate, ld_gate, up, ld_up, M, N, layout, q_row, ld_q_row, s_row,
                         ld_s_row, q_col, ld_q_col, s_col, ld_s_col, stream);
}

mxfp8_status mxfp8_quant_2d(const void *x, int64_t ld_x, int64_t M, int64_t K, int layout, void *q_row,
                            int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                            void *s_col, int64_t ld_s_col, void *stream) {
  return quant_2d_impl(x, ld_x, M, K, layout, q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col,
                       nullptr, 0, stream);
}

mxfp8_status mxfp8_quant_2d_grouped(const void *x, int64_t ld_x, int64_t M, int64_t K, int layout, void *q_row,
                                    int64_t ld_q_row, void *s_row, int64_t ld_s_row, void *q_col, int64_t ld_q_col,
                                    void *s_col, int64_t ld_s_col, const int32_t *group_ends, int64_t n_groups,
                                    void *stream) {
  mxfp8_status st = check_groups(group_ends, n_groups, M);
  if (st != MXFP8_OK) return st;
  return quant_2d_impl(x, ld_x, M, K, layout, q_row, ld_q_row, s_row, ld_s_row, q_col, ld_q_col, s_col, ld_s_col,
                       group_ends, n_groups, stream);
}

mxfp8_status mxfp8_quant_3d_colwise(const void *w, int64_t E, int64_t N, int64_t K, int64_t stride_e,
                                    int64_t ld_w, void *q, void *s, void *stream) {
  if (E < 0 || N < 0 || K < 0) return MXFP8_ERR_SHAPE;
  if (N % 32 != 0 || K % 8 != 0) return MXFP8_ERR_SHAPE;
  if (E == 0 || N == 0 || K == 0) return MXFP8_OK;
  if (!w || !q || !s) return MXFP8_ERR_NULL;
  if (ld_w < K || ld_w % 8 != 0) return MXFP8_ERR_STRIDE;
  int64_t slab;
  if (!mul_ok(N, ld_w, &slab)) return MXFP8_ERR_OVERFLOW;
  if (E > 1 && (stride_e < slab || stride_e % 8 != 0)) return MXFP8_ERR_STRIDE;
  if (!aligned16(w) || !aligned16(q)) return MXFP8_ERR_ALIGN;
  const int64_t ld_one[1] = {ld_w};
  if (!tile_offsets_ok(ld_one, 1, 0, 0, N, N / 32)) return MXFP8_ERR_OVERFLOW;
  int64_t in_ext, out_ext;
  if (!mul_ok(E - 1, stride_e, &in_ext) || !add_ok(in_ext, slab, &in_ext) || in_ext >= (INT64_MAX >> 2))
    return MXFP8_ERR_OVERFLOW;
  if (!mul_ok(E, N, &out_ext) || !mul_ok(out_ext, K, &out_ext) || out_ext >= (INT64_MAX >> 2))
    return MXFP8_ERR_OVERFLOW;
  const void *in[1] = {w};
  const int64_t ld[1] = {ld_w};
  // Expert e is a [N, K] matrix whose 32-blocks run down its N rows: the
  // colwise cast with rows = N, columns = K, output rows of length N.
  Args a = make_args(in, ld, 1, N, K, nullptr, 0, nullptr, 0, q, N, s, N / 32);
  a.bstride_in = stride_e;
  a.bstride_q = K * N;
  a.bstride_s = K * (N / 32);
  const int64_t tiles = E * ((N + mx::kTM - 1) / mx::kTM) * ((K + mx::kTC - 1) / mx::kTC);
  return launch_colwise<mx::OpQuant>(a, false, E, stream, tiles >= kCapTiles3d ? 3 : 0);
}

mxfp8_status mxfp8_swiglu_fwd_bf16(const void *gate, int64_t ld_gate, const void *up, int64_t ld_up, int64_t M,
                                   int64_t N, void *h, int64_t ld_h, void *stream) {
  const void *in[2] = {gate, up};
  const int64_t ld[2] = {ld_gate, ld_up};
  mxfp8_status st = check_values(in, ld, 2, M, N, h, ld_h, N);
  if (st != MXFP8_OK || M == 0 || N == 0) return st;
  Args a = make_args(in, ld, 2, M, N, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0);
  return launch_values<mx::OpFwd>(a, h, ld_h, stream);
}

mxfp8_status mxfp8_swiglu_bwd_bf16(const void *dh, int64_t ld_dh, const void *gate, int64_t ld_gate, const void *up,
                                   int64_t ld_up, int64_t M, int64_t N, void *dgdu, int64_t ld_dgdu,
                                   void *stream) {
  const void *in[3] = {dh, gate, up};
  const int64_t ld[3] = {ld_dh, ld_gate, ld_up};
  mxfp8_status st = check_values(in, ld, 3, M, N, dgdu, ld_dgdu, 2 * N);
  if (st != MXFP8_OK || M == 0 || N == 0) return st;
  Args a = make_args(in, ld, 3, M, N, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0);
  return launch_values<mx::OpBwd>(a, dgdu, ld_dgdu, stream);
}

}  // extern "C"

namespace {

// Checks and launch shared by the three GEMM forms.  G == 0 is the plain
// form (offsets unused, one expert); kGemmGroupM groups the rows of A (B per
// group at b + g * stride_b); kGemmGroupK groups the contraction axis (C per
// group at c + g * stride_c, scales in the per-group padded layout).
mxfp8_status gemm_launch(int mode, const void *a, int64_t lda, const void *sa, int64_t ld_sa, const void *b,
                         int64_t ldb, int64_t stride_b, const void *sb, int64_t ld_sb, int64_t stride_sb,
                         const int32_t *offs, int64_t G, int64_t M, int64_t N, int64_t K, float *c, int64_t ldc,
                         int64_t stride_c, void *stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || G < 0 || G > mx::kMaxGroups) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (!a || !sa || !b || !sb || !c || (G > 0 && !offs)) return MXFP8_ERR_NULL;
  // scale columns the operands reach: K/32, or with token groups the
  // per-group padded layout, whose positions stay below K/32 + 16 G
  const int64_t s_w = K / 32 + (mode == mx::kGemmGroupK ? 16 * G : 0);
  if (lda < K || ldb < K || lda % 16 != 0 || ldb % 16 != 0 || ld_sa < s_w || ld_sb < s_w || ldc < N)
    return MXFP8_ERR_STRIDE;
  if (mode == mx::kGemmGroupM) {
    int64_t span_b, span_sb;
    if (!mul_ok(N - 1, ldb, &span_b) || !add_ok(span_b, K, &span_b) || !mul_ok(N - 1, ld_sb, &span_sb) ||
        !add_ok(span_sb, K / 32, &span_sb))
      return MXFP8_ERR_OVERFLOW;
    if (stride_b < span_b || stride_b % 16 != 0 || stride_sb < span_sb) return MXFP8_ERR_STRIDE;
  }
  if (mode == mx::kGemmGroupK) {
    int64_t span_c;
    if (!mul_ok(M - 1, ldc, &span_c) || !add_ok(span_c, N, &span_c)) return MXFP8_ERR_OVERFLOW;
    if (stride_c < span_c) return MXFP8_ERR_STRIDE;
  }
  if (!aligned16(a) || !aligned16(b) || ((uintptr_t)c & 3u) != 0 || ((uintptr_t)offs & 3u) != 0)
    return MXFP8_ERR_ALIGN;
  if (!extent_ok(M, K, lda) || !extent_ok(N, K, ldb) || !extent_ok(M, s_w, ld_sa) || !extent_ok(N, s_w, ld_sb) ||
      !extent_ok(M, N, ldc))
    return MXFP8_ERR_OVERFLOW;
  if (G > 0) {
    int64_t e;
    if (mode == mx::kGemmGroupM &&
        (!mul_ok(G - 1, stride_b, &e) || e >= (INT64_MAX >> 2) || !mul_ok(G - 1, stride_sb, &e) ||
         e >= (INT64_MAX >> 2)))
      return MXFP8_ERR_OVERFLOW;
    if (mode == mx::kGemmGroupK && (!mul_ok(G - 1, stride_c, &e) || e >= (INT64_MAX >> 2)))
      return MXFP8_ERR_OVERFLOW;
  }
  // tile-relative offsets are 32-bit: 256 rows of either operand must span less than 2^32 bytes
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23) || ld_sa >= (int64_t(1) << 23) ||
      ld_sb >= (int64_t(1) << 23))
    return MXFP8_ERR_OVERFLOW;
  // M-grouped: an upper bound of row tiles, each group adding at most one
  // partial tile, so the host never reads the device-side offsets.
  const int64_t tiles_m = (M + mx::kBM - 1) / mx::kBM + (mode == mx::kGemmGroupM ? G : 0);
  const int64_t tiles_n = (N + mx::kBN - 1) / mx::kBN;
  int64_t blocks;
  if (!mul_ok(tiles_m, tiles_n, &blocks) || (mode == mx::kGemmGroupK && !mul_ok(blocks, G, &blocks)) ||
      blocks > (int64_t)INT32_MAX / mx::kGemmThreads)
    return MXFP8_ERR_OVERFLOW;
  // The kernel runs a last round of T tiles as 2 T half tiles when T is at
  // most half the CUs, as 4 T quarter tiles when at most a quarter
  // (k_mx_gemm): the grid holds those work items, in the M-grouped form an
  // upper bound (tiles + the larger of 3 (CUs / 4) and CUs / 2 extra items).
  // The CU count is the current device's; it only decides the split, not
  // any result.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  if (cus > 1) {
    if (mode == mx::kGemmGroupM) {
      blocks += std::max<int64_t>(3 * (cus / 4), cus / 2);
    } else {
      const int64_t tail = blocks % cus;
      if (tail > 0 && tail <= cus / 4) blocks += 3 * tail;
      else if (tail > 0 && tail <= cus / 2) blocks += tail;
    }
  }
  if (blocks > (int64_t)INT32_MAX / mx::kGemmThreads) return MXFP8_ERR_OVERFLOW;
  mx::GemmArgs g{};
  g.a = static_cast<const uint8_t *>(a);
  g.sa = static_cast<const uint8_t *>(sa);
  g.b = static_cast<const uint8_t *>(b);
  g.sb = static_cast<const uint8_t *>(sb);
  g.lda = lda;
  g.ld_sa = ld_sa;
  g.ldb = ldb;
  g.ld_sb = ld_sb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c = c;
  g.ldc = ldc;
  g.tiles_m = (int32_t)tiles_m;
  g.tiles_n = (int32_t)tiles_n;
  g.offs = offs;
  g.G = (int32_t)G;
  g.stride_b = stride_b;
  g.stride_sb = stride_sb;
  g.stride_c = stride_c;
  g.scale_vec = aligned16(sa) && aligned16(sb) && ld_sa % 16 == 0 && ld_sb % 16 == 0 && stride_sb % 16 == 0;
  g.cus = cus;
  void *kargs[] = {&g};
  // nontemporal C stores for tiles long in K (for the K-grouped form, the
  // mean group length)
  const bool nt = (mode == mx::kGemmGroupK ? K / G : K) >= 1024;
  const void *k = mode == mx::kGemmGroupM
                      ? (nt ? (const void *)&mx::k_mx_gemm<mx::kGemmGroupM, true>
                            : (const void *)&mx::k_mx_gemm<mx::kGemmGroupM, false>)
                  : mode == mx::kGemmGroupK
                      ? (nt ? (const void *)&mx::k_mx_gemm<mx::kGemmGroupK, true>
                            : (const void *)&mx::k_mx_gemm<mx::kGemmGroupK, false>)
                      : (nt ? (const void *)&mx::k_mx_gemm<mx::kGemmPlain, true>
                            : (const void *)&mx::k_mx_gemm<mx::kGemmPlain, false>);
  hipError_t err = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(mx::kGemmThreads), kargs, 0, (hipStream_t)stream);
  return err == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

}  // namespace

extern "C" {

mxfp8_status mxfp8_gemm(const void *a, int64_t lda, const void *sa, int64_t ld_sa, const void *b, int64_t ldb,
                        const void *sb, int64_t ld_sb, int64_t M, int64_t N, int64_t K, float *c, int64_t ldc,
                        void *stream) {
  return gemm_launch(mx::kGemmPlain, a, lda, sa, ld_sa, b, ldb, 0, sb, ld_sb, 0, nullptr, 0, M, N, K, c, ldc, 0,
                     stream);
}

mxfp8_status mxfp8_grouped_gemm(const void *a, int64_t lda, const void *sa, int64_t ld_sa, const void *b,
                                int64_t ldb, int64_t stride_b, const void *sb, int64_t ld_sb, int64_t stride_sb,
                                const int32_t *offsets, int64_t G, int64_t M, int64_t N, int64_t K, float *c,
                                int64_t ldc, void *stream) {
  if (G <= 0) return G == 0 ? MXFP8_OK : MXFP8_ERR_SHAPE;
  return gemm_launch(mx::kGemmGroupM, a, lda, sa, ld_sa, b, ldb, stride_b, sb, ld_sb, stride_sb, offsets, G, M, N,
                     K, c, ldc, 0, stream);
}

mxfp8_status mxfp8_grouped_gemm_k(const void *a, int64_t lda, const void *sa, int64_t ld_sa, const void *b,
                                  int64_t ldb, const void *sb, int64_t ld_sb, const int32_t *group_ends, int64_t G,
                                  int64_t M, int64_t N, int64_t T, float *c, int64_t ldc, int64_t stride_c,
                                  void *stream) {
  if (G <= 0) return G == 0 ? MXFP8_OK : MXFP8_ERR_SHAPE;
  return gemm_launch(mx::kGemmGroupK, a, lda, sa, ld_sa, b, ldb, 0, sb, ld_sb, 0, group_ends, G, M, N, T, c, ldc,
                     stride_c, stream);
}

const char *mxfp8_status_str(mxfp8_status status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_ERR_NULL: return "a required pointer is NULL";
    case MXFP8_ERR_SHAPE: return "invalid shape (negative, or a blocked dimension not a multiple of 32)";
    case MXFP8_ERR_STRIDE: return "invalid leading dimension (smaller than the row, or not a vector multiple)";
    case MXFP8_ERR_ALIGN: return "input or E4M3 output pointer is not 16-byte aligned";
    case MXFP8_ERR_LAYOUT: return "layout must be rowwise (1), colwise (2) or both (3)";
    case MXFP8_ERR_OVERFLOW: return "sizes overflow the addressable range or the launch grid";
    case MXFP8_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case MXFP8_ERR_ACT: return "activation must be MXFP8_ACT_SILU, _GELU_TANH, _GELU or _RELU";
  }
  return "unknown status";
}

}  // extern "C"
