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
// lane m + 32 b (op_sel picks the register byte, 0 to 3).  The 32x32 fp32
// result sits in 16 registers: lane l, register v holds row
// 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
//
// Structure: a 256 x 256 C tile per 256-thread workgroup, one workgroup per
// CU (148 KB of LDS); each wavefront owns 128 x 128 of C, its 256
// accumulators in AGPRs.  K is staged 128 at a time (two MFMA steps) in a
// double-buffered LDS ring filled by direct global -> LDS loads; each stage
// reads all its operands from LDS, then issues the next stage's loads, then
// its 32 MFMAs, so the loads run under the matrix work.
#pragma once
#include "mx_kernels.hpp"

namespace mx {

struct GemmArgs {
  const uint8_t *a, *sa, *b, *sb;
  int64_t lda, ld_sa, ldb, ld_sb;
  int64_t M, N, K;
  float *c;
  int64_t ldc;
  int32_t tiles_m, tiles_n;  // tiles_m: an upper bound in the grouped form
  // grouped form: G groups of rows by cumulative end offsets (device
  // memory), group g against b + g * stride_b, sb + g * stride_sb
  const int32_t *offs;
  int32_t G;
  int64_t stride_b, stride_sb;
  // scale rows start 16-byte aligned (sa, sb, ld_sa, ld_sb, stride_sb all
  // multiples of 16): the scale table is then fetched 16 bytes at a time
  int32_t scale_vec;
  // K-grouped form: group g's result at c + g * stride_c
  int64_t stride_c;
};

// Kernel forms: the plain GEMM; rows of A grouped by device-side offsets
// (each group against its own expert's B: forward and input gradient); and
// the contraction axis grouped (each group of tokens gives its own C: the
// weight gradient).
enum GemmMode { kGemmPlain = 0, kGemmGroupM = 1, kGemmGroupK = 2 };

constexpr int kMaxGroups = 1024;

// 16 zero bytes in device memory: the source of operand chunks at or past K
__device__ __attribute__((aligned(16))) const uint8_t kZeroChunk[16] = {};

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;  // C tile per workgroup
constexpr int kBK = 128;              // K per LDS stage: two MFMA steps, whole 128-byte lines
constexpr int kGroup = 4;             // tile rows per group in the tile order
constexpr int kGemmThreads = 256;     // four wavefronts, 2 x 2, each 128 x 128 of C
constexpr int kStageA = kBM * kBK, kStageB = kBN * kBK;  // one stage of each operand in LDS (bytes)
constexpr int kSG = 16;                                  // scale blocks per LDS scale group
constexpr int kStagesPerGroup = kSG / (kBK / 32);
static_assert(kStagesPerGroup >= 2, "a scale group is written to LDS in its second stage");

__device__ __forceinline__ u32x4_t gload16(const uint8_t *p) {
  return *gptr(reinterpret_cast<const u32x4_t *>(p));
}

// LDS position of 16-byte chunk kc (0..7) of tile row `row`: rows of 128
// bytes, chunks XOR-permuted by (row / 2) % 8, so that the 16 lanes of one
// quarter-wave reading the same chunk of 16 consecutive rows hit 16
// different 4-bank groups.
__device__ __forceinline__ u32 lds_off(u32 row, u32 kc) { return row * kBK + ((kc ^ ((row >> 1) & 7u)) << 4); }

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void k_mx_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smemA[2][kStageA], smemB[2][kStageB];  // [buffer]
  // scale table of one group of kSG blocks: row q < kBM is A's tile row q,
  // row kBM + q is B's tile row q  [buffer][row][block]
  __shared__ __attribute__((aligned(16))) uint8_t smemS[2][kBM + kBN][kSG];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1, r = lane & 31, h = lane >> 5;

  // Tile order: each XCD takes one contiguous range of tiles; inside it,
  // groups of kGroup tile rows are walked column by column.  In the
  // K-grouped form the tiles of one token group come one after another.
  u32 L = xcd_remap(blockIdx.x, gridDim.x);
  int64_t kgrp = 0;
  if constexpr (MODE == kGemmGroupK) {
    const u32 per = (u32)g.tiles_m * (u32)g.tiles_n;
    kgrp = L / per;
    L %= per;
  }
  const u32 per_group = (u32)kGroup * (u32)g.tiles_n;
  const u32 grp = L / per_group, in_grp = L % per_group;
  const u32 rows_in_grp = min((u32)kGroup, (u32)g.tiles_m - grp * (u32)kGroup);
  const int64_t tm = (int64_t)grp * kGroup + in_grp % rows_in_grp;
  const int64_t n_base = (int64_t)(in_grp / rows_in_grp) * kBN;

  // Rows of this tile: [m_base, m_end).  In the grouped form tile row tm is
  // the (tm - tiles before)-th tile of the group it falls in, counting each
  // group's tiles from its own first row; the grid holds an upper bound of
  // tiles (rows / 256 + groups), and tiles past the real count do nothing.
  int64_t m_base = tm * kBM, m_end = g.M;
  const uint8_t *b_mat = g.b, *sb_mat = g.sb;
  // Contraction range [k_lo, k_lo + Kt) of the operands' columns, and the
  // column of its first scale block.
  int64_t k_lo = 0, Kt = g.K, s_lo = 0;
  float *c_mat = g.c;
  if constexpr (MODE == kGemmGroupM) {
    __shared__ int32_t offs_s[kMaxGroups];
    for (int e = t; e < g.G; e += kGemmThreads) offs_s[e] = g.offs[e];
    __syncthreads();
    int64_t start = 0, before = 0;
    int e_hit = -1;
    for (int e = 0; e < g.G; e++) {  // uniform: every lane walks the same offsets
      const int64_t end = min<int64_t>(max<int64_t>((int64_t)offs_s[e], start), g.M);
      const int64_t nt = (end - start + kBM - 1) / kBM;
      if (tm < before + nt) {
        e_hit = e;
        m_base = start + (tm - before) * kBM;
        m_end = end;
        break;
      }
      before += nt;
      start = end;
    }
    if (e_hit < 0) return;  // uniform over the workgroup: past the real tiles
    b_mat = g.b + (int64_t)e_hit * g.stride_b;
    sb_mat = g.sb + (int64_t)e_hit * g.stride_sb;
  }
  if constexpr (MODE == kGemmGroupK) {
    // Token group kgrp: the cumulative ends rounded down to a multiple of 32
    // (negative ends read as 0), made non-decreasing and at most K; its
    // scales start at 16 (kgrp + floor(start / 512)) of each scale row (the
    // per-group padded layout the grouped casts write).
    int64_t start = 0, end = 0;
    for (int64_t e = 0; e <= kgrp; e++) {  // uniform
      const int32_t v = g.offs[e];
      const int64_t r = v <= 0 ? 0 : (int64_t)(v & ~31);
      start = end;
      end = min<int64_t>(max<int64_t>(r, start), g.K);
    }
    k_lo = start;
    Kt = end - start;
    s_lo = 16 * (kgrp + start / 512);
    c_mat = g.c + kgrp * g.stride_c;
  }

  // Rows past M (N) are read as the last row: in bounds, never stored.
  const uint8_t *a_tile = g.a + m_base * g.lda + k_lo, *b_tile = b_mat + n_base * g.ldb + k_lo;  // uniform
  const u32 a_rows = (u32)min<int64_t>(m_end - m_base, kBM), b_rows = (u32)min<int64_t>(g.N - n_base, kBN);

  // ---- scales: moved to LDS kSG blocks (kStagesPerGroup stages) at a
  // time, thread t taking A's and B's tile row t.  Blocks past K / 32 read
  // as 127 (2^0) against zero data.  One byte load per lane per operand
  // tile and stage, from 32 rows at once, is far slower than this.
  const uint8_t *sa_tile = g.sa + m_base * g.ld_sa + s_lo, *sb_tile = sb_mat + n_base * g.ld_sb + s_lo;  // uniform
  const int64_t nblk = Kt / 32;
  const int nstage = (int)((Kt + kBK - 1) / kBK);
  const int ngroup = (int)((nblk + kSG - 1) / kSG);
  const u32 sa_row = min((u32)t, a_rows - 1), sb_row = min((u32)t, b_rows - 1);

  u32x4_t ssa, ssb;  // the next scale group, global -> registers -> LDS
  auto load_scales = [&](int grp) {
    const int64_t b0 = (int64_t)grp * kSG;
    if (g.scale_vec && b0 + kSG <= nblk) {  // uniform
      ssa = gload16(byte_off(sa_tile + b0, sa_row * (u32)g.ld_sa));
      ssb = gload16(byte_off(sb_tile + b0, sb_row * (u32)g.ld_sb));
    } else {
      // byte by byte, from clamped (in-bounds) positions; blocks past K / 32 read as 127
      u32 wa[4] = {0, 0, 0, 0}, wb[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kSG; j++) {
        const bool ok = b0 + j < nblk;
        const int64_t bj = min<int64_t>(b0 + j, nblk - 1);
        const u32 va = *gptr(byte_off(sa_tile + bj, sa_row * (u32)g.ld_sa));
        const u32 vb = *gptr(byte_off(sb_tile + bj, sb_row * (u32)g.ld_sb));
        wa[j / 4] |= (ok ? va : 127u) << (8 * (j % 4));
        wb[j / 4] |= (ok ? vb : 127u) << (8 * (j % 4));
      }
      ssa = u32x4_t{wa[0], wa[1], wa[2], wa[3]};
      ssb = u32x4_t{wb[0], wb[1], wb[2], wb[3]};
    }
  };
  // Table row q keeps its 4 dwords rotated by (q / 16) % 4, so that 32
  // consecutive rows read at one dword position hit 32 different banks.
  auto rot = [](u32x4_t v, u32 k) {  // dword j moves to position (j + k) % 4
    const u32 w0 = k == 0 ? v.x : k == 1 ? v.w : k == 2 ? v.z : v.y;
    const u32 w1 = k == 0 ? v.y : k == 1 ? v.x : k == 2 ? v.w : v.z;
    const u32 w2 = k == 0 ? v.z : k == 1 ? v.y : k == 2 ? v.x : v.w;
    const u32 w3 = k == 0 ? v.w : k == 1 ? v.z : k == 2 ? v.y : v.x;
    return u32x4_t{w0, w1, w2, w3};
  };
  auto store_scales = [&](int buf) {
    const u32 k = ((u32)t >> 4) & 3u;  // kBM is a multiple of 64: the same key for both halves
    *reinterpret_cast<u32x4_t *>(&smemS[buf][t][0]) = rot(ssa, k);
    *reinterpret_cast<u32x4_t *>(&smemS[buf][kBM + t][0]) = rot(ssb, k);
  };
  // this stage's 4 scale bytes of table row q, shifted so that the block of
  // step s for this lane's half (block 2 s + h) is byte 2 s (op_sel 2 s)
  auto read_scales = [&](int buf, u32 q, int in_grp_) {
    const u32 pos = ((u32)in_grp_ + (q >> 4)) & 3u;
    const u32 v = *reinterpret_cast<const u32 *>(&smemS[buf][q][4u * pos]);
    return (int)(v >> (8u * (u32)h));
  };
  // ---- operands: global -> LDS directly (global_load_lds_dwordx4: lane
  // l's 16 bytes land at the instruction's LDS base + 16 l).  Wave w fills
  // 1 KB slabs p = 8 w + q (q = 0..7) of each operand's stage buffer, i.e.
  // tile rows 8 p .. 8 p + 7; lane l writes slab bytes 16 l .. 16 l + 15,
  // which hold row 8 p + l / 8, stored chunk l % 8, i.e. logical chunk
  // (l % 8) ^ the row's XOR key.  Chunks at or past K, and so every chunk
  // of a stage past the last, are read from kZeroChunk.
  auto dma_stage = [&](int st_, int buf_) {
    const int64_t k0 = (int64_t)st_ * kBK;
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const u32 p = (u32)w * 8u + (u32)q;
      const u32 row = 8u * p + ((u32)lane >> 3), kc = ((u32)lane & 7u) ^ ((row >> 1) & 7u);
      const bool in_k = k0 + 16 * (int64_t)kc < Kt;
      const u32 ra = min(row, a_rows - 1), rb = min(row, b_rows - 1);
      const uint8_t *pa = in_k ? byte_off(a_tile + k0, ra * (u32)g.lda + kc * 16u) : kZeroChunk;
      const uint8_t *pb = in_k ? byte_off(b_tile + k0, rb * (u32)g.ldb + kc * 16u) : kZeroChunk;
      __builtin_amdgcn_global_load_lds((const MX_GLOBAL void *)gptr(pa),
                                       (__attribute__((address_space(3))) void *)&smemA[buf_][p * 1024u], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const MX_GLOBAL void *)gptr(pb),
                                       (__attribute__((address_space(3))) void *)&smemB[buf_][p * 1024u], 16, 0, 0);
    }
  };
  constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters not waited

  v16f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v16f_t{};

  if (nstage > 0) dma_stage(0, 0);
  if (ngroup > 0) load_scales(0);  // K = 0: no scale is read
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (ngroup > 0) store_scales(0);
  __syncthreads();

  for (int st = 0; st < nstage; st++) {
    const int buf = st & 1;
    const int grp = st / kStagesPerGroup, in_grp = st % kStagesPerGroup;
    const bool more_scales = grp + 1 < ngroup;  // uniform
    // the next scale group: fetched in the group's first stage, written to
    // LDS at the start of its second (the fetch completed with the first
    // stage's data), into the buffer whose last reads ended with the
    // previous group; first read after a later barrier
    if (more_scales && in_grp == 1) store_scales((grp + 1) & 1);
    if (more_scales && in_grp == 0) load_scales(grp + 1);
    // this stage's operands and scales for both MFMA steps, all read before
    // the first MFMA in the order the MFMAs consume them; in step s lane
    // r + 32 h takes block 4 in_grp + 2 s + h of its row in each 32-row
    // tile, byte 2 s of the scale word (op_sel 2 s)
    int csa[4], csb[4];
    v8i_t av[2][4], bv[2][4];
    auto read_op = [&](const uint8_t *base, u32 row, u32 s) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(&base[lds_off(row, 4u * s + h)]);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(&base[lds_off(row, 4u * s + 2u + h)]);
      return v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
#pragma unroll
    for (int i = 0; i < 4; i++) csa[i] = read_scales(grp & 1, (u32)(wm * 128 + 32 * i + r), in_grp);
#pragma unroll
    for (int j = 0; j < 4; j++) csb[j] = read_scales(grp & 1, (u32)(kBM + wn * 128 + 32 * j + r), in_grp);
#pragma unroll
    for (int s = 0; s < 2; s++) {
      av[s][0] = read_op(smemA[buf], (u32)(wm * 128 + r), s);
#pragma unroll
      for (int j = 0; j < 4; j++) bv[s][j] = read_op(smemB[buf], (u32)(wn * 128 + 32 * j + r), s);
#pragma unroll
      for (int i = 1; i < 4; i++) av[s][i] = read_op(smemA[buf], (u32)(wm * 128 + 32 * i + r), s);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The next stage's loads, into the other buffer (its last reads ended at
    // the previous barrier), issued after every LDS read of this stage: the
    // compiler waits for such loads before any later LDS read.  Not behind
    // a branch, so that the MFMAs cannot sink past the scheduling barriers
    // into a later block (after the last stage it loads zeros into the idle
    // buffer).
    dma_stage(st + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[0][i], bv[0][j], acc[i][j], 0, 0, 0, csa[i], 0,
                                                                     csb[j]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[1][i], bv[1][j], acc[i][j], 0, 0, 2, csa[i], 2,
                                                                     csb[j]);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads have landed; the barrier makes every wave's visible
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t col = n_base + wn * 128 + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int64_t row = m_base + wm * 128 + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);
        if (row < m_end && col < g.N) *gptr(c_mat + row * g.ldc + col) = acc[i][j][v];
      }
    }
}

}  // namespace mx
