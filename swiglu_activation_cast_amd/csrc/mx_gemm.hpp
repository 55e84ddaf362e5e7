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
// CU; each wavefront owns 128 x 128 of C, its 256 accumulators in AGPRs.  K
// is staged 64 at a time (one MFMA step) in a ring of four LDS slots filled
// by direct global -> LDS loads issued three stages ahead.  While a stage's
// 16 MFMAs run from registers, the wavefront reads the next stage's operands
// from LDS into a second register set and issues the loads of the stage
// three ahead (one after every other MFMA), so that the matrix cores, the
// LDS and the vector memory unit work at once.  A last round of tiles that
// would leave at least half the CUs idle runs as 256 x 128 half tiles (at
// least three quarters idle: 256 x 64 quarter tiles), and
// a tile of at most 128 rows computes and loads only the row blocks that
// can hold its rows.  In the M-grouped form every group's whole row tiles
// run before the groups' partial last rows.  Unaligned scale rows are read
// as 4-byte words.
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
  // compute units of the device: the tiles of a last partial round are
  // split in two when that round would leave at least half of them idle,
  // in four when at least three quarters
  int32_t cus;
};

// Kernel forms: the plain GEMM; rows of A grouped by device-side offsets
// (each group against its own expert's B: forward and input gradient); and
// the contraction axis grouped (each group of tokens gives its own C: the
// weight gradient).
enum GemmMode { kGemmPlain = 0, kGemmGroupM = 1, kGemmGroupK = 2 };

constexpr int kMaxGroups = 1024;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;  // C tile per workgroup
constexpr int kBK = 64;               // K per stage: one MFMA step
constexpr int kRing = 4;              // LDS stage slots
constexpr int kAhead = 3;             // stages whose loads are issued ahead of the one computed
constexpr int kGroup = 4;             // tile rows per group in the tile order
constexpr int kGemmThreads = 256;     // four wavefronts, 2 x 2, each 128 x 128 of C
constexpr int kSlot = kBM * kBK;      // bytes of one operand in one slot (16 KB)
constexpr int kSG = 16;               // scale blocks per LDS scale group
constexpr int kStagesPerGroup = kSG / (kBK / 32);
static_assert(kBM == kBN, "the operand load layout assumes square tiles");

// LDS position of 16-byte chunk kc (0..3) of tile row `row`: rows of 64
// bytes, chunks XOR-permuted by (row / 4) % 4, so that the 16 lanes of one
// quarter-wave reading the same chunk of 16 consecutive rows hit 16
// different 16-byte bank groups.
__device__ __forceinline__ u32 lds_off(u32 row, u32 kc) { return row * (u32)kBK + ((kc ^ ((row >> 2) & 3u)) << 4); }

__device__ __forceinline__ u32 lds_addr(const void *p) {
  return (u32)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Direct global -> LDS load: lane l's 16 bytes at base + off land at LDS
// byte `lds` + 16 l (global_load_lds_dwordx4, saddr form).  Written as asm so
// that the compiler does not wait for it before LDS reads of other slots;
// its completion is awaited with wait_vm.  M0 holds the LDS base: it is
// saved and restored, and an SALU write of M0 needs one wait state before
// an LDS DMA reads it.
__device__ __forceinline__ void load_lds(const uint8_t *base, u32 off, u32 lds) {
  u32 saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(base));
}
// Wait until at most N of this wavefront's vector memory operations are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 256-row tile of C, NJ 32-column blocks per wavefront: NJ = 4 is the
// whole 256 x 256 tile (each wavefront 128 x 128), NJ = 2 one half of it,
// 256 x 128, and NJ = 1 one quarter, 256 x 64 (`half`: which half or
// quarter; each wavefront 128 x 32 NJ), for the last partial round of
// tiles.  Every element of C gets the same sum in the same order either
// way.  L is the tile's index in the tile order over tiles_m rows of
// tiles (in the grouped form the real count, of which full_m are whole
// rows of 256, ordered before the groups' partial last rows).
//
// The tile's 32-row blocks alternate between the two wavefront rows
// (wavefront row wm takes blocks wm, wm + 2, wm + 4, wm + 6), so that a
// short tile (a group's last rows, or the last rows of A) has rows in both
// wavefront rows.  NI is the number of those blocks each wavefront
// computes: 4 for a tile of more than 128 rows, 2 for at most 128, 1 for at
// most 64.  A tile of 64 rows then takes 4 MFMAs and 5 loads per stage and
// wavefront instead of 16 and 8 (only the A rows it computes are loaded).
//
// NT: C written with nontemporal stores (K-long tiles: the stores then do
// not displace operand lines from L2); otherwise ordinary stores, faster
// when the tile is short in K.
template <int MODE, bool NT, int NJ, int NI = 4>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, uint8_t (*smA)[kSlot], uint8_t (*smB)[kSlot],
                                          uint8_t (*smS)[kBM + kBN][kSG], const int32_t *offs_s, u32 L, int half,
                                          int64_t tiles_m, int64_t full_m) {
  const u32 L_in = L;
  constexpr int BN = 64 * NJ;     // tile columns
  constexpr int WBN = 32 * NJ;    // columns per wavefront
  constexpr int kLoads = NI + NJ;  // direct loads per wavefront and stage: NI of A, NJ of B
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1, r = lane & 31, h = lane >> 5;

  // Tile order: each XCD takes one contiguous range of tiles; inside it,
  // groups of kGroup tile rows are walked column by column.  In the
  // K-grouped form L runs over the groups one after another (the kernel
  // hands each XCD an eighth of every group).
  int64_t kgrp = 0;
  if constexpr (MODE == kGemmGroupK) {
    const u32 per = (u32)tiles_m * (u32)g.tiles_n;
    kgrp = L / per;
    L %= per;
  }
  // In the M-grouped form the whole row tiles of every group come first and
  // the groups' partial last row tiles after them, each set in this order.
  u32 rows_set = (u32)tiles_m, row0 = 0;
  if constexpr (MODE == kGemmGroupM) {
    const u32 n_full = (u32)full_m * (u32)g.tiles_n;
    if (L >= n_full) {
      L -= n_full;
      rows_set = (u32)(tiles_m - full_m);
      row0 = (u32)full_m;
    } else {
      rows_set = (u32)full_m;
    }
  }
  const u32 per_group = (u32)kGroup * (u32)g.tiles_n;
  const u32 grp = L / per_group, in_grp = L % per_group;
  const u32 rows_in_grp = min((u32)kGroup, rows_set - grp * (u32)kGroup);
  const int64_t tm = (int64_t)row0 + (int64_t)grp * kGroup + in_grp % rows_in_grp;
  const int64_t n_base = (int64_t)(in_grp / rows_in_grp) * kBN + (int64_t)half * BN;
  if (n_base >= g.N) return;  // the second half of a tile narrower than 128 columns (uniform)

  // Rows of this tile: [m_base, m_end).  In the grouped form tile row tm is
  // the (tm - tiles before)-th tile of the group it falls in, counting each
  // group's tiles from its own first row.
  int64_t m_base = tm * kBM, m_end = g.M;
  const uint8_t *b_mat = g.b, *sb_mat = g.sb;
  // Contraction range [k_lo, k_lo + Kt) of the operands' columns, and the
  // column of its first scale block.
  int64_t k_lo = 0, Kt = g.K, s_lo = 0;
  float *c_mat = g.c;
  if constexpr (MODE == kGemmGroupM) {
    // row tile tm < full_m: the (tm - whole rows before)-th whole row of the
    // group it falls in; otherwise the partial last row of the
    // (tm - full_m)-th group that has one
    int64_t start = 0, before = 0;
    int e_hit = -1;
    const bool whole = tm < full_m;
    const int64_t want = whole ? tm : tm - full_m;
    for (int e = 0; e < g.G; e++) {  // uniform: every lane walks the same offsets
      const int64_t end = min<int64_t>(max<int64_t>((int64_t)offs_s[e], start), g.M);
      const int64_t nf = (end - start) / kBM;
      const int64_t nt = whole ? nf : (int64_t)((end - start) % kBM != 0);
      if (want < before + nt) {
        e_hit = e;
        m_base = start + (whole ? want - before : nf) * kBM;
        m_end = end;
        break;
      }
      before += nt;
      start = end;
    }
    // the walk is uniform; make that visible to the compiler, so that the
    // tile's bases live in scalar registers
    e_hit = __builtin_amdgcn_readfirstlane(e_hit);
    if (e_hit < 0) return;  // past the real tiles (not reached: L < the real count)
    m_base = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((u32)((uint64_t)m_base >> 32)) << 32) |
                       __builtin_amdgcn_readfirstlane((u32)m_base));
    m_end = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((u32)((uint64_t)m_end >> 32)) << 32) |
                      __builtin_amdgcn_readfirstlane((u32)m_end));
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
      const int64_t rr = v <= 0 ? 0 : (int64_t)(v & ~31);
      start = end;
      end = min<int64_t>(max<int64_t>(rr, start), g.K);
    }
    k_lo = start;
    Kt = end - start;
    s_lo = 16 * (kgrp + start / 512);
    c_mat = g.c + kgrp * g.stride_c;
  }

  // Rows past M (N) are read as the last row: in bounds, never stored.
  const uint8_t *a_tile = g.a + m_base * g.lda + k_lo, *b_tile = b_mat + n_base * g.ldb + k_lo;  // uniform
  const u32 a_rows = (u32)min<int64_t>(m_end - m_base, kBM), b_rows = (u32)min<int64_t>(g.N - n_base, BN);
  if constexpr (NI == 4) {
    if (a_rows <= 2u * 32u) {  // uniform: a short tile, one row block per wavefront
      gemm_tile<MODE, NT, NJ, 1>(g, smA, smB, smS, offs_s, L_in, half, tiles_m, full_m);
      return;
    }
    if (a_rows <= 4u * 32u) {  // two row blocks per wavefront
      gemm_tile<MODE, NT, NJ, 2>(g, smA, smB, smS, offs_s, L_in, half, tiles_m, full_m);
      return;
    }
  }
  const uint8_t *sa_tile = g.sa + m_base * g.ld_sa + s_lo, *sb_tile = sb_mat + n_base * g.ld_sb + s_lo;  // uniform
  const int64_t nblk = Kt / 32;
  const int nstage = (int)((Kt + kBK - 1) / kBK);
  const int ngroup = (int)((nblk + kSG - 1) / kSG);

  // ---- operand loads.  Slab p of a slot holds tile rows 16 p .. 16 p + 15:
  // A's slabs p = NI w + q (q < NI: the 64 NI rows the wavefronts compute),
  // B's p = NJ w + q (q < NJ: 4 per wavefront for a whole tile, 2 for a
  // half, 1 for a quarter);
  // lane l loads row 16 p + l / 4 into stored chunk l % 4, which holds
  // logical chunk (l % 4) ^ the row's key; the key (row / 4) % 4 =
  // (l / 16) % 4 is the same for every slab.
  const u32 kc16 = (((u32)lane & 3u) ^ (((u32)lane >> 4) & 3u)) * 16u;
  auto aslab = [&](int q) { return (u32)(NI * w + q); };
  auto bslab = [&](int q) { return (u32)(NJ * w + q); };
  u32 a_roff[NI], b_roff[NJ];
#pragma unroll
  for (int q = 0; q < NI; q++) a_roff[q] = min(16u * aslab(q) + ((u32)lane >> 2), a_rows - 1) * (u32)g.lda;
#pragma unroll
  for (int q = 0; q < NJ; q++) b_roff[q] = min(16u * bslab(q) + ((u32)lane >> 2), b_rows - 1) * (u32)g.ldb;
  // Stage st goes to slot st % kRing.  Loads of stages past the last re-read
  // the last one into a free slot (never read); chunks at or past K read
  // chunk 0 of their row and are zeroed in LDS before the stage is read.
  auto stage_base = [&](int st_, const uint8_t *&ba, const uint8_t *&bb, u32 &kc) {
    const int64_t k0 = (int64_t)min(st_, nstage - 1) * kBK;
    ba = a_tile + k0;
    bb = b_tile + k0;
    kc = (int64_t)kc16 < Kt - k0 ? kc16 : 0u;
  };
  auto load_stage = [&](int st_) {
    const uint8_t *ba, *bb;
    u32 kc;
    stage_base(st_, ba, bb, kc);
    const int slot = st_ & (kRing - 1);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if (q < NI) load_lds(ba, a_roff[q < NI ? q : 0] + kc, lds_addr(&smA[slot][aslab(q) * 1024u]));
      if (q < NJ) load_lds(bb, b_roff[q < NJ ? q : 0] + kc, lds_addr(&smB[slot][bslab(q) * 1024u]));
    }
  };
  auto zero_tail = [&](int st_) {  // this thread's chunks of stage st_ at or past K -> 0
    const int64_t kmax = Kt - (int64_t)st_ * kBK;
    const int slot = st_ & (kRing - 1);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if ((int64_t)kc16 >= kmax) {
        if (q < NI) *reinterpret_cast<u32x4_t *>(&smA[slot][aslab(q) * 1024u + 16u * (u32)lane]) = u32x4_t{0, 0, 0, 0};
        if (q < NJ) *reinterpret_cast<u32x4_t *>(&smB[slot][bslab(q) * 1024u + 16u * (u32)lane]) = u32x4_t{0, 0, 0, 0};
      }
    }
  };

  // ---- scales, kSG blocks (kStagesPerGroup stages) at a time, into buffer
  // group % 2.  Full groups of 16-byte-aligned scale rows go global -> LDS
  // directly: wavefront w fills table rows 128 w .. 128 w + 127, lane l one
  // row.  Otherwise thread t reads A's and B's tile row t: a full group
  // as 4-byte words, the last partial one byte by byte, blocks past K / 32
  // reading 127 (2^0) against zero data.
  auto group_vec = [&](int gi) { return g.scale_vec && (int64_t)(gi + 1) * kSG <= nblk; };
  const u32 sa_row = min((u32)t, a_rows - 1), sb_row = min((u32)t, b_rows - 1);
  auto load_scales = [&](int gi) {
    const int64_t b0 = (int64_t)gi * kSG;
    if (group_vec(gi)) {
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const u32 trow0 = 64u * (2u * (u32)w + (u32)q);  // uniform: 64 rows of one operand
        if (trow0 >= (u32)(kBM + BN)) continue;         // past a half tile's B rows
        const u32 trow = trow0 + (u32)lane;
        const bool is_a = trow0 < (u32)kBM;
        const uint8_t *base = is_a ? sa_tile + b0 : sb_tile + b0;
        const u32 off = is_a ? min(trow, a_rows - 1) * (u32)g.ld_sa : min(trow - kBM, b_rows - 1) * (u32)g.ld_sb;
        load_lds(base, off, lds_addr(&smS[gi & 1][trow0][0]));
      }
    } else if ((int64_t)(gi + 1) * kSG <= nblk) {
      // A whole group of scale rows that are not 16-byte aligned: thread t
      // takes the 16 bytes of A's and B's tile row t from the five 4-byte
      // words around them (the fifth only where the bytes are not word
      // aligned; each word read holds at least one of the row's bytes, so no
      // read reaches a page the row does not touch), joined by v_alignbyte.
      auto row16 = [&](const uint8_t *p) {
        const u32 sft = (u32)((uintptr_t)p & 3u);
        const u32 *q = reinterpret_cast<const u32 *>((uintptr_t)p - sft);
        const u32 d0 = *gptr(q), d1 = *gptr(q + 1), d2 = *gptr(q + 2), d3 = *gptr(q + 3);
        const u32 d4 = *gptr(q + (sft ? 4 : 3));
        return u32x4_t{__builtin_amdgcn_alignbyte(d1, d0, sft), __builtin_amdgcn_alignbyte(d2, d1, sft),
                       __builtin_amdgcn_alignbyte(d3, d2, sft), __builtin_amdgcn_alignbyte(d4, d3, sft)};
      };
      const u32x4_t va = row16(byte_off(sa_tile + b0, sa_row * (u32)g.ld_sa));
      const u32x4_t vb = row16(byte_off(sb_tile + b0, sb_row * (u32)g.ld_sb));
      *reinterpret_cast<u32x4_t *>(&smS[gi & 1][t][0]) = va;
      *reinterpret_cast<u32x4_t *>(&smS[gi & 1][kBM + t][0]) = vb;
    } else {  // the last, partial group: byte by byte, blocks past K / 32 as 127 (2^0)
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
      *reinterpret_cast<u32x4_t *>(&smS[gi & 1][t][0]) = u32x4_t{wa[0], wa[1], wa[2], wa[3]};
      *reinterpret_cast<u32x4_t *>(&smS[gi & 1][kBM + t][0]) = u32x4_t{wb[0], wb[1], wb[2], wb[3]};
    }
  };

  // One stage's operands and scales in registers.  Lane r + 32 h takes, for
  // each 32-row tile, chunks h and 2 + h of its row (block h of the step:
  // elements 16 h .. 16 h + 15 of each of the step's two 32-element
  // halves), and the scale byte of block 2 (stage % 8) + h of its row,
  // shifted to byte 0 (op_sel 0).
  struct Ops {
    v8i_t a[4], b[4];
    int sa[4], sb[4];
  };
  auto read_stage = [&](int st_, Ops &o) {
    const int slot = st_ & (kRing - 1), gi = st_ / kStagesPerGroup, in_g = st_ % kStagesPerGroup;
    const u32 sh = 8u * (u32)h + 16u * (u32)(in_g & 1);
#pragma unroll
    for (int x = 0; x < 4; x++) {
      if (x < NI) {
        const u32 ra = (u32)(32 * (2 * x + wm) + r);
        const u32x4_t la = *reinterpret_cast<const u32x4_t *>(&smA[slot][lds_off(ra, (u32)h)]);
        const u32x4_t ha = *reinterpret_cast<const u32x4_t *>(&smA[slot][lds_off(ra, 2u + (u32)h)]);
        o.a[x] = v8i_t{(int)la.x, (int)la.y, (int)la.z, (int)la.w, (int)ha.x, (int)ha.y, (int)ha.z, (int)ha.w};
        o.sa[x] = (int)(*reinterpret_cast<const u32 *>(&smS[gi & 1][ra][4 * (in_g / 2)]) >> sh);
      }
      if (x < NJ) {
        const u32 rb = (u32)(wn * WBN + 32 * x + r);
        const u32x4_t lb = *reinterpret_cast<const u32x4_t *>(&smB[slot][lds_off(rb, (u32)h)]);
        const u32x4_t hb = *reinterpret_cast<const u32x4_t *>(&smB[slot][lds_off(rb, 2u + (u32)h)]);
        o.b[x] = v8i_t{(int)lb.x, (int)lb.y, (int)lb.z, (int)lb.w, (int)hb.x, (int)hb.y, (int)hb.z, (int)hb.w};
        o.sb[x] = (int)(*reinterpret_cast<const u32 *>(&smS[gi & 1][kBM + rb][4 * (in_g / 2)]) >> sh);
      }
    }
  };

  v16f_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < NJ; j++) acc[i][j] = v16f_t{};

  // One stage: the MFMAs of stage st from `cur`; between them, the loads of
  // stage st + kAhead (its slot held stage st - 1, whose reads ended before
  // the previous barrier) and the reads of stage st + 1 into `nxt` (read
  // unconditionally: past the last stage the slot holds data never used).
  // Then wait until stage st + 2 has landed and meet the barrier.  st = -1
  // is a leading all-zero stage that makes the stage count even.
  auto body = [&](int st, Ops &cur, Ops &nxt) {
    if (st >= 0 && st % kStagesPerGroup == 0 && st / kStagesPerGroup + 1 < ngroup)
      load_scales(st / kStagesPerGroup + 1);  // its buffer was last read by the previous group
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *ba, *bb;
    u32 kc;
    stage_base(st + kAhead, ba, bb, kc);
    const int lslot = (st + kAhead) & (kRing - 1);
    const int rs = st + 1, rslot = rs & (kRing - 1), rgi = rs / kStagesPerGroup, rin = rs % kStagesPerGroup;
    u32x4_t la[4], ha[4], lb[NJ], hb[NJ];
    u32 wsa[4], wsb[NJ];
    auto read_a = [&](int x, int part) {  // part 0: chunk h and the scale word, 1: chunk 2 + h
      const u32 ra = (u32)(32 * (2 * x + wm) + r);
      if (part == 0) {
        la[x] = *reinterpret_cast<const u32x4_t *>(&smA[rslot][lds_off(ra, (u32)h)]);
        wsa[x] = *reinterpret_cast<const u32 *>(&smS[rgi & 1][ra][4 * (rin / 2)]);
      } else {
        ha[x] = *reinterpret_cast<const u32x4_t *>(&smA[rslot][lds_off(ra, 2u + (u32)h)]);
      }
    };
    auto read_b = [&](int x, int part) {
      const u32 rb = (u32)(wn * WBN + 32 * x + r);
      if (part == 0) {
        lb[x] = *reinterpret_cast<const u32x4_t *>(&smB[rslot][lds_off(rb, (u32)h)]);
        wsb[x] = *reinterpret_cast<const u32 *>(&smS[rgi & 1][kBM + rb][4 * (rin / 2)]);
      } else {
        hb[x] = *reinterpret_cast<const u32x4_t *>(&smB[rslot][lds_off(rb, 2u + (u32)h)]);
      }
    };
#pragma unroll
    for (int k = 0; k < 4 * NJ; k++) {
      const int i = k / NJ, j = k % NJ;
      if (i < NI) {  // resolved at compile time: the loop is unrolled
        const int ii = i < NI ? i : NI - 1;
        acc[ii][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[ii], cur.b[j], acc[ii][j], 0, 0, 0,
                                                                      cur.sa[ii], 0, cur.sb[j]);
      }
      if constexpr (NJ == 4) {
        if (k % 2 == 0) {  // load k / 2: A's slab q (if it has one), then B's
          const int q = k / 4;
          if (k % 4 == 0) {
            if (q < NI) load_lds(ba, a_roff[q < NI ? q : 0] + kc, lds_addr(&smA[lslot][aslab(q) * 1024u]));
          } else {
            load_lds(bb, b_roff[q] + kc, lds_addr(&smB[lslot][bslab(q) * 1024u]));
          }
        }
        const int x = k / 4, part = k % 4;
        if (part < 2) {
          if (x < NI) read_a(x, part);
        } else {
          read_b(x, part - 2);
        }
      } else if constexpr (NJ == 2) {
        // 8 MFMAs: after each of the first six one load (A's four slabs,
        // then B's two); after each the reads of one A tile's chunk, and
        // after the first four also one of B's
        if (k < 4) {
          if (k < NI) load_lds(ba, a_roff[k < NI ? k : 0] + kc, lds_addr(&smA[lslot][aslab(k) * 1024u]));
        } else if (k < 6) {
          load_lds(bb, b_roff[k - 4] + kc, lds_addr(&smB[lslot][bslab(k - 4) * 1024u]));
        }
        if (k / 2 < NI) read_a(k / 2, k % 2);
        if (k < 4) read_b(k / 2, k % 2);
      } else {
        // 4 MFMAs: after the first B's slab; after each A's slab k (if it
        // has one) and both chunks of A tile k; after the first two one
        // chunk of B's
        if (k == 0) load_lds(bb, b_roff[0] + kc, lds_addr(&smB[lslot][bslab(0) * 1024u]));
        if (k < NI) {
          load_lds(ba, a_roff[k < NI ? k : 0] + kc, lds_addr(&smA[lslot][aslab(k) * 1024u]));
          read_a(k, 0);
          read_a(k, 1);
        }
        if (k < 2) read_b(0, k);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep this order: loads and reads spread between the MFMAs
    }
    const u32 sh = 8u * (u32)h + 16u * (u32)(rin & 1);
#pragma unroll
    for (int x = 0; x < NI; x++) {
      nxt.a[x] = v8i_t{(int)la[x].x, (int)la[x].y, (int)la[x].z, (int)la[x].w,
                       (int)ha[x].x, (int)ha[x].y, (int)ha[x].z, (int)ha[x].w};
      nxt.sa[x] = (int)(wsa[x] >> sh);
    }
#pragma unroll
    for (int x = 0; x < NJ; x++) {
      nxt.b[x] = v8i_t{(int)lb[x].x, (int)lb[x].y, (int)lb[x].z, (int)lb[x].w,
                       (int)hb[x].x, (int)hb[x].y, (int)hb[x].z, (int)hb[x].w};
      nxt.sb[x] = (int)(wsb[x] >> sh);
    }
    __builtin_amdgcn_sched_barrier(0);
#if __HIP_DEVICE_COMPILE__
    // Uses of this stage's results here keep its MFMAs and reads in this
    // block: the branches below would otherwise let the compiler sink them
    // past the barrier, where nothing overlaps them.
#pragma unroll
    for (int x = 0; x < 4; x++) {
      if (x < NI) {
#pragma unroll
        for (int j = 0; j < NJ; j++) asm volatile("" ::"a"(acc[x < NI ? x : 0][j]));
        asm volatile("" ::"v"(nxt.a[x]), "v"(nxt.sa[x]));
      }
      if (x < NJ) asm volatile("" ::"v"(nxt.b[x]), "v"(nxt.sb[x]));
    }
#endif
    wait_vm<kLoads>();  // stage st + 2, and scales issued before stage st + kAhead, landed
    __syncthreads();
    if ((int64_t)(st + 3) * kBK > Kt && (int64_t)(st + 2) * kBK < Kt) {  // stage st + 2 is the partial last one
      zero_tail(st + 2);
      __syncthreads();
    }
  };

  Ops o0, o1;
  const int odd = nstage & 1;
  if (nstage > 0) {
    if (ngroup > 0) load_scales(0);
    load_stage(0);
    load_stage(1);
    // The first stage body reads the stage after the first one computed:
    // stage 1 (even stage count) or stage 0 (odd: the leading zero stage
    // comes first).  Wait until that one, the ones before it and the
    // scales have landed.
    if (!odd) {
      load_stage(2);
      wait_vm<kLoads>();  // stages 0 and 1 and the scales landed
    } else {
      wait_vm<kLoads>();  // stage 0 and the scales landed
    }
    __syncthreads();
    if ((int64_t)kBK > Kt) {  // stage 0 is partial (then it is the only one)
      zero_tail(0);
      __syncthreads();
    }
    if (!odd && (int64_t)2 * kBK > Kt) {  // two stages, the second partial (landed above)
      zero_tail(1);
      __syncthreads();
    }
    if (!odd) {
      read_stage(0, o0);
    } else {  // the leading zero stage
#pragma unroll
      for (int x = 0; x < 4; x++) {
        o0.a[x] = v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
        o0.b[x] = v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
        o0.sa[x] = 127;
        o0.sb[x] = 127;
      }
    }
  }
  for (int st = -odd; st < nstage; st += 2) {
    body(st, o0, o1);
    body(st + 1, o1, o0);
  }
  wait_vm<0>();  // no load may still be writing this workgroup's LDS when it ends

  // ---- C
  auto put = [&](float *p, float v) {
    if constexpr (NT) __builtin_nontemporal_store(v, gptr(p));
    else *gptr(p) = v;
  };
  if (a_rows == (u32)kBM && b_rows == (u32)BN && g.ldc < (int64_t(1) << 22)) {
    // whole tile: a uniform row base per (i, v) and a 32-bit lane offset
    float *c_tile = c_mat + m_base * g.ldc + n_base;
    const u32 lane_off = ((u32)(32 * wm + 4 * h) * (u32)g.ldc + (u32)(wn * WBN + r)) * 4u;
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        float *row_base = c_tile + (int64_t)(64 * i + 8 * (v / 4) + (v % 4)) * g.ldc;
#pragma unroll
        for (int j = 0; j < NJ; j++) put(byte_off(row_base, lane_off + 128u * (u32)j), acc[i][j][v]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const int64_t col = n_base + wn * WBN + 32 * j + r;
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int64_t row = m_base + 32 * (2 * i + wm) + 8 * (v / 4) + 4 * h + (v % 4);
          if (row < m_end && col < g.N) put(c_mat + row * g.ldc + col, acc[i][j][v]);
        }
      }
  }
}

// Work items of a launch: the tiles in the tile order, R of them (in the
// grouped form counted from the device-side offsets, so that the host never
// reads them; its grid is an upper bound and items past the count exit).
// With C compute units, the first R - R % C tiles run whole, one round of C
// after another, in XCD-contiguous ranges.  If the remaining T = R % C tiles
// would leave at least half the CUs idle in their round (T <= C / 2), they
// run as 2 T half tiles instead (two consecutive items per tile), and as
// 4 T quarter tiles if at least three quarters (T <= C / 4): that round
// then ends in a little over half (a quarter of) the time.
template <int MODE, bool NT>
__global__ __launch_bounds__(kGemmThreads, 1) void k_mx_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smA[kRing][kSlot], smB[kRing][kSlot];  // [slot]
  // scale table of one group of kSG blocks: row q < kBM is A's tile row q,
  // row kBM + q is B's tile row q  [buffer][row][block]
  __shared__ __attribute__((aligned(1024))) uint8_t smS[2][kBM + kBN][kSG];
  __shared__ int32_t offs_s[MODE == kGemmGroupM ? kMaxGroups : 1];

  int64_t tiles_m = g.tiles_m, full_m = g.tiles_m;
  if constexpr (MODE == kGemmGroupM) {
    for (int e = threadIdx.x; e < g.G; e += kGemmThreads) offs_s[e] = g.offs[e];
    __syncthreads();
    // real tile rows: every group's rows rounded up to whole tiles, with the
    // offsets clamped into ordered groups within [0, M] as the tiles see
    // them; full_m of them hold 256 rows
    int64_t start = 0, n = 0, nf = 0;
    for (int e = 0; e < g.G; e++) {  // uniform
      const int64_t end = min<int64_t>(max<int64_t>((int64_t)offs_s[e], start), g.M);
      n += (end - start + kBM - 1) / kBM;
      nf += (end - start) / kBM;
      start = end;
    }
    tiles_m = n;
    full_m = nf;
  }
  const u32 R = (u32)(MODE == kGemmGroupK ? (int64_t)g.G : 1) * (u32)tiles_m * (u32)g.tiles_n;
  const u32 C = g.cus > 1 ? (u32)g.cus : 1u;
  const u32 R0 = R - R % C, T = R - R0;
  const u32 parts = C <= 1 || T == 0 ? 1u : T <= C / 4 ? 4u : T <= C / 2 ? 2u : 1u;  // items per last-round tile
  const u32 b = blockIdx.x;
  if (b >= R0 + parts * T) return;  // past the work items (uniform)
  if (b < R0) {
    u32 L = xcd_remap(b, R0);
    if constexpr (MODE == kGemmGroupK) {
      // The groups' tiles differ in depth, and each XCD takes a fixed
      // eighth of the work items (the dispatcher deals workgroups to the
      // XCDs in turn), so a contiguous eighth per XCD would leave the XCDs
      // holding the deepest group working while the others idle.  When the
      // counts divide, XCD x takes instead the x-th eighth of every group,
      // each eighth a contiguous run of that group's tile order.
      const u32 per = (u32)tiles_m * (u32)g.tiles_n, share = per / 8u, range = R0 / 8u;
      if (R0 % 8u == 0 && per % 8u == 0 && range == share * (u32)g.G) {
        const u32 x = L / range, p = L % range;
        L = (p / share) * per + x * share + p % share;
      }
    }
    gemm_tile<MODE, NT, 4>(g, smA, smB, smS, offs_s, L, 0, tiles_m, full_m);
  } else if (parts == 1) {
    gemm_tile<MODE, NT, 4>(g, smA, smB, smS, offs_s, b, 0, tiles_m, full_m);
  } else if (parts == 2) {
    gemm_tile<MODE, NT, 2>(g, smA, smB, smS, offs_s, R0 + (b - R0) / 2, (int)((b - R0) & 1u), tiles_m, full_m);
  } else {
    gemm_tile<MODE, NT, 1>(g, smA, smB, smS, offs_s, R0 + (b - R0) / 4, (int)((b - R0) & 3u), tiles_m, full_m);
  }
}

}  // namespace mx
