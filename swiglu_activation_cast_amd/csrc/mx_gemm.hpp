// mx_gemm.hpp -- the consumer of the casts: C = A B^T on MXFP8 operands with
// gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Operands are stored with K contiguous, as the casts emit them: A [M, K]
// E4M3 with E8M0 scales sa [M, K/32] (the rowwise output of an [M, K]
// matrix), B [N, K] with sb [N, K/32] (the rowwise output of [N, K], or the
// colwise output of a [K, N] matrix, whose rows run along the blocked axis).
// Scales are read in the plain row-major layout the casts write: the MFMA
// takes one scale per lane in a register, so no swizzled scale layout is
// needed.  "[mxfp8 moe training] add compile support", Perf analysis (the
// cast outputs feed a scaled grouped GEMM); "Add swiglu + MXFP8 fused CuTe
// DSL kernel", Summary.
//
// Lane layout of the 32x32x64 fp8 MFMA (checked on gfx950 with an in-bounds
// probe against a double-precision host product): lane l holds row l % 32
// of A (column l % 32 of B^T); its bytes 0..15 are elements 16 (l / 32) ..
// +15 of the MFMA's first 32-element K block and bytes 16..31 the same
// positions of its second block.  The scale of (row m, block b) comes from
// lane m + 32 b (op_sel picks the register byte).  The 32x32 fp32 result
// sits in 16 registers: lane l, register v holds row 8 (v / 4) + 4 (l / 32)
// + v % 4, column l % 32.
#pragma once
#include "mx_kernels.hpp"

namespace mx {

struct GemmArgs {
  const uint8_t *a, *sa, *b, *sb;
  int64_t lda, ld_sa, ldb, ld_sb;
  int64_t M, N, K;
  float *c;
  int64_t ldc;
  int32_t tiles_m, tiles_n;
};

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kGT = 128;   // C tile per workgroup, both dimensions
constexpr int kGroup = 8;  // tile rows per group in the tile order

__device__ __forceinline__ u32x4_t gload16(const uint8_t *p) {
  return *gptr(reinterpret_cast<const u32x4_t *>(p));
}

__global__ __launch_bounds__(256) void k_mx_gemm(const GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  // Tile order: each XCD takes one contiguous range of tiles; inside it,
  // groups of kGroup tile rows are walked column by column, so the tiles in
  // flight on one XCD share a few A row-slabs and B column-slabs in its L2.
  const u32 L = xcd_remap(blockIdx.x, gridDim.x);
  const u32 per_group = (u32)kGroup * (u32)g.tiles_n;
  const u32 grp = L / per_group, in_grp = L % per_group;
  const u32 rows_in_grp = min((u32)kGroup, (u32)g.tiles_m - grp * (u32)kGroup);
  const int64_t tm = (int64_t)grp * kGroup + in_grp % rows_in_grp, tn = in_grp / rows_in_grp;
  const int64_t m0 = tm * kGT + (wave >> 1) * 64, n0 = tn * kGT + (wave & 1) * 64;

  // Operand rows of this lane.  Rows past M (N) are read as row M-1 (N-1):
  // in bounds, and their results are never stored.
  const uint8_t *arow[2], *brow[2], *sarow[2], *sbrow[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int64_t m = min(m0 + 32 * i + r, g.M - 1), n = min(n0 + 32 * i + r, g.N - 1);
    arow[i] = g.a + m * g.lda + 16 * h;
    sarow[i] = g.sa + m * g.ld_sa + h;
    brow[i] = g.b + n * g.ldb + 16 * h;
    sbrow[i] = g.sb + n * g.ld_sb + h;
  }

  v16f_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = v16f_t{};

  const int64_t nblk = g.K / 32;
  for (int64_t k0 = 0; k0 < g.K; k0 += 64) {
    const int64_t b0 = k0 / 32;
    const bool second = b0 + 1 < nblk;  // uniform: the MFMA's second block exists
    v8i_t av[2], bv[2];
    int as[2], bs[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const u32x4_t alo = gload16(arow[i] + k0);
      const u32x4_t ahi = second ? gload16(arow[i] + k0 + 32) : u32x4_t{0, 0, 0, 0};
      av[i] = v8i_t{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
      const u32x4_t blo = gload16(brow[i] + k0);
      const u32x4_t bhi = second ? gload16(brow[i] + k0 + 32) : u32x4_t{0, 0, 0, 0};
      bv[i] = v8i_t{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
      // lane m + 32 h carries the scale of block b0 + h; a missing second
      // block (K % 64 == 32) has zero data and takes scale 2^0
      as[i] = (h == 0 || second) ? (int)*gptr(sarow[i] + b0) : 127;
      bs[i] = (h == 0 || second) ? (int)*gptr(sbrow[i] + b0) : 127;
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv[j], acc[i][j], 0, 0, 0, as[i], 0, bs[j]);
  }

#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t col = n0 + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int64_t row = m0 + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);
        if (row < g.M && col < g.N) *gptr(g.c + row * g.ldc + col) = acc[i][j][v];
      }
    }
}

}  // namespace mx
