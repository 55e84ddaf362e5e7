// mx_kernels.hpp -- the gfx950 kernels behind the C ABI.
//
// Two kernel families, both templated on the value producer (mx_ops.hpp):
//
//  k_rowwise  rowwise-only (1x32 blocks).  One wavefront streams one row:
//             each lane owns 8 consecutive columns (one 16-byte load per
//             input), four lanes form a 32-column block, the block amax is
//             two DPP lane swaps.  No LDS, no barrier.
//
//  k_tiled    colwise (32x1) with or without rowwise.  A 256-thread
//             workgroup owns a 128-row x 64-column tile: it loads the tile
//             once with row-contiguous 16-byte loads, computes the values,
//             (optionally) emits the rowwise blocks straight from registers,
//             and writes the values transposed into LDS.  After one barrier
//             each lane reads 16 consecutive rows of one column (two 16-byte
//             LDS reads), pairs with its neighbour lane for the 32-row block
//             amax, and stores 16 E4M3 bytes; eight lanes cover 128 rows of
//             one output row, a full 128-byte line.  The same kernel, with a
//             batch index, is the 3D per-expert colwise cast.
//
// Layout facts: "Add swiglu + MXFP8 fused CuTe DSL kernel" (Summary: 1x32,
// 32x1 or both from a single pass); "[mxfp8 moe training] update 3d quant
// colwise scaling kernel to use single input/output TMA descriptors"
// (Summary: one launch for all experts, transposed through on-chip memory
// before the column-major-per-expert store).
#pragma once
#include "mx_ops.hpp"

namespace mx {

struct Args {
  const uint16_t *in[3];
  int64_t ld_in[3];
  int64_t M, N;  // rows, source columns (the output width is Op::OUT * N)
  uint8_t *q_row;
  int64_t ld_q_row;
  uint8_t *s_row;
  int64_t ld_s_row;
  uint8_t *q_col;
  int64_t ld_q_col;
  uint8_t *s_col;
  int64_t ld_s_col;
  int64_t bstride_in, bstride_q, bstride_s;  // per-batch offsets (3D cast)
  int32_t n_rt, n_ct;                        // row tiles, column tiles
  int32_t n_seg;                             // column segments per row strip (strip kernel)
};

__device__ __forceinline__ V4 load16(const uint16_t *p) { return *reinterpret_cast<const V4 *>(p); }

// Blocks are dispatched round-robin over the 8 XCDs; renumber them so each
// XCD works through one contiguous range of tiles (neighbouring tiles share
// scale lines in that XCD's L2).
__device__ __forceinline__ u32 xcd_remap(u32 b, u32 n) {
  constexpr u32 X = 8;
  u32 full = n - n % X;
  if (b >= full) return b;
  return (b % X) * (full / X) + b / X;
}

// ------------------------------------------------------------------ rowwise
constexpr int kRowWaves = 4;  // rows per 256-thread workgroup

template <class Op, int U>
__global__ __launch_bounds__(256) void k_rowwise(const Args a) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (m >= a.M) return;  // wave-uniform
  const int64_t nch = a.N >> 3;
  const uint16_t *row[Op::IN];
#pragma unroll
  for (int j = 0; j < Op::IN; j++) row[j] = a.in[j] + m * a.ld_in[j];
  uint8_t *qr = a.q_row + m * a.ld_q_row;
  uint8_t *sr = a.s_row + m * a.ld_s_row;

  for (int64_t c0 = 0; c0 < nch; c0 += 64 * U) {
    V4 in[U][Op::IN];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t c = c0 + 64 * u + lane;
#pragma unroll
      for (int j = 0; j < Op::IN; j++) in[u][j] = (c < nch) ? load16(row[j] + c * 8) : V4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t c = c0 + 64 * u + lane;
      V4 out[Op::OUT];
      Op::apply(in[u], out);
#pragma unroll
      for (int o = 0; o < Op::OUT; o++) {
        u32 am = max_xor2(max_xor1(amax_bits<4>(&out[o].x)));
        u32 b = e8m0_rceil(am);
        uint2 q = quant8(&out[o].x, b);
        if (c < nch) {
          const int64_t col = o * a.N + c * 8;
          *reinterpret_cast<uint2 *>(qr + col) = q;
          if ((lane & 3) == 0) sr[col >> 5] = (uint8_t)b;
        }
      }
    }
  }
}

// -------------------------------------------------------------------- tiled
constexpr int kTM = 128;       // tile rows (four 32-row blocks)
constexpr int kTC = 64;        // tile source columns
constexpr int kRS = kTM + 8;   // LDS row stride of one transposed column (bf16)
constexpr int kRPT = 4;        // rows per thread in the load phase

template <class Op, bool ROWS>
__global__ __launch_bounds__(256) void k_tiled(const Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[Op::OUT][kTC][kRS];
  const int t = threadIdx.x;
  const u32 L = xcd_remap(blockIdx.x, gridDim.x);
  const u32 rt = L % (u32)a.n_rt;
  const u32 rest = L / (u32)a.n_rt;
  const u32 ct = rest % (u32)a.n_ct;
  const int64_t e = rest / (u32)a.n_ct;
  const int64_t m0 = (int64_t)rt * kTM, n0 = (int64_t)ct * kTC;

  // ---- load + compute: thread owns rows m0 + 4*rg + i (i < 4), columns col..col+7
  const int cc = t & 7, rg = t >> 3;
  const int64_t col = n0 + cc * 8;
  const bool colok = col < a.N;
  V4 out[kRPT][Op::OUT];
  {
    V4 in[kRPT][Op::IN];
#pragma unroll
    for (int i = 0; i < kRPT; i++) {
      const int64_t m = m0 + rg * kRPT + i;
      const bool ok = colok && m < a.M;
#pragma unroll
      for (int j = 0; j < Op::IN; j++)
        in[i][j] = ok ? load16(a.in[j] + e * a.bstride_in + m * a.ld_in[j] + col) : V4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kRPT; i++) Op::apply(in[i], out[i]);
  }

  if constexpr (ROWS) {
#pragma unroll
    for (int i = 0; i < kRPT; i++) {
      const int64_t m = m0 + rg * kRPT + i;
#pragma unroll
      for (int o = 0; o < Op::OUT; o++) {
        u32 am = max_xor2(max_xor1(amax_bits<4>(&out[i][o].x)));
        u32 b = e8m0_rceil(am);
        uint2 q = quant8(&out[i][o].x, b);
        if (colok && m < a.M) {
          const int64_t oc = o * a.N + col;
          *reinterpret_cast<uint2 *>(a.q_row + m * a.ld_q_row + oc) = q;
          if ((cc & 3) == 0) a.s_row[m * a.ld_s_row + (oc >> 5)] = (uint8_t)b;
        }
      }
    }
  }

  // ---- transpose into LDS: column (8*cc + k), rows 4*rg .. 4*rg+3
#pragma unroll
  for (int o = 0; o < Op::OUT; o++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const u32 *r0 = &out[0][o].x, *r1 = &out[1][o].x, *r2 = &out[2][o].x, *r3 = &out[3][o].x;
      const int w = k >> 1;
      u32 p01, p23;
      if (k & 1) {
        p01 = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
        p23 = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
      } else {
        p01 = (r0[w] & 0xffffu) | (r1[w] << 16);
        p23 = (r2[w] & 0xffffu) | (r3[w] << 16);
      }
      *reinterpret_cast<uint2 *>(&lds[o][cc * 8 + k][rg * kRPT]) = make_uint2(p01, p23);
    }
  }
  __syncthreads();

  // ---- colwise: item = (output o, column c, 16-row group g); lanes g, g^1 share a block
#pragma unroll
  for (int p = 0; p < 2 * Op::OUT; p++) {
    const int i = t + 256 * p;
    const int g = i & 7, c = (i >> 3) & (kTC - 1), o = i >> 9;
    const V4 v0 = *reinterpret_cast<const V4 *>(&lds[o][c][16 * g]);
    const V4 v1 = *reinterpret_cast<const V4 *>(&lds[o][c][16 * g + 8]);
    const u32 v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    u32 am = max_xor1(amax_bits<8>(v));
    u32 b = e8m0_rceil(am);
    uint2 q0 = quant8(v, b), q1 = quant8(v + 4, b);
    const int64_t n = n0 + c, mr = m0 + 16 * g;
    if (n < a.N && mr < a.M) {
      const int64_t orow = o * a.N + n;
      *reinterpret_cast<uint4 *>(a.q_col + e * a.bstride_q + orow * a.ld_q_col + mr) = make_uint4(q0.x, q0.y, q1.x, q1.y);
      if ((g & 1) == 0) a.s_col[e * a.bstride_s + orow * a.ld_s_col + (mr >> 5)] = (uint8_t)b;
    }
  }
}


// -------------------------------------------------------------------- strip
// Colwise (32x1) with or without rowwise, no LDS.  A wavefront owns a
// 32-row x 256-column tile: lane l covers columns 8*(l%32) .. +7 of rows
// 16*(l/32) .. +15, so the two wave halves hold the two 16-row halves of
// every 32-row column block and one cross-half swap finishes the column
// amax.  Values stay in registers as packed bf16 until the column scales
// are known; the E4M3 converts then take two rows of one column at a time,
// so each lane's 16 column bytes come out already in column-major order and
// leave as one 16-byte store.  Four waves stack to 128 rows, so the four
// 32-byte pieces of each output column line are written together.  A
// workgroup walks its row strip across a range of column tiles, completing
// each rowwise scale line and letting neighbouring strips (same XCD after
// the remap) complete the colwise scale lines at about the same time.
constexpr int kSC = 256;  // strip tile source columns
constexpr int kSM = 128;  // strip tile rows (4 waves x 32)
constexpr int kSG = 4;    // rows loaded per group

__device__ __forceinline__ u32 swap_halves(u32 v) {
  // lane l <-> lane l ^ 32
  return (u32)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32u) << 2), (int)v);
}

template <class Op, bool ROWS>
__global__ __launch_bounds__(256) void k_strip(const Args a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = lane >> 5;
  const u32 L = xcd_remap(blockIdx.x, gridDim.x);
  // order: row strip fastest, then column segment, then batch
  const u32 rt = L % (u32)a.n_rt;
  const u32 rest = L / (u32)a.n_rt;
  const u32 seg = rest % (u32)a.n_seg;
  const int64_t e = rest / (u32)a.n_seg;
  const int64_t mblk = (int64_t)rt * kSM + 32 * w;  // first row of this wave's 32-row block
  if (mblk >= a.M) return;                           // wave-uniform; no barriers in this kernel
  const int64_t mr = mblk + 16 * half;               // first of this lane's 16 rows
  const int ct0 = (int)(((int64_t)seg * a.n_ct) / a.n_seg);
  const int ct1 = (int)(((int64_t)(seg + 1) * a.n_ct) / a.n_seg);

  const uint16_t *in[Op::IN];
#pragma unroll
  for (int j = 0; j < Op::IN; j++) in[j] = a.in[j] + e * a.bstride_in + mr * a.ld_in[j];
  uint8_t *qc = a.q_col + e * a.bstride_q;
  uint8_t *sc = a.s_col + e * a.bstride_s;

  for (int ct = ct0; ct < ct1; ct++) {
    const int64_t col = (int64_t)ct * kSC + 8 * (lane & 31);
    const bool colok = col < a.N;
    u32 val[Op::OUT][16][4];
    u32 cmax[Op::OUT][4];
#pragma unroll
    for (int o = 0; o < Op::OUT; o++)
#pragma unroll
      for (int k = 0; k < 4; k++) cmax[o][k] = 0;

#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += kSG) {
      V4 x[kSG][Op::IN];
#pragma unroll
      for (int r = 0; r < kSG; r++)
#pragma unroll
        for (int j = 0; j < Op::IN; j++)
          x[r][j] = colok ? load16(in[j] + (int64_t)(r0 + r) * a.ld_in[j] + col) : V4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < kSG; r++) {
        V4 y[Op::OUT];
        Op::apply(x[r], y);
#pragma unroll
        for (int o = 0; o < Op::OUT; o++) {
          const u32 *v = &y[o].x;
#pragma unroll
          for (int k = 0; k < 4; k++) {
            val[o][r0 + r][k] = v[k];
            cmax[o][k] = pk_max(cmax[o][k], v[k] & 0x7fff7fffu);
          }
          if constexpr (ROWS) {
            u32 am = max_xor2(max_xor1(amax_bits<4>(v)));
            u32 b = e8m0_rceil(am);
            uint2 q = quant8(v, b);
            if (colok) {
              const int64_t m = mr + r0 + r, oc = o * a.N + col;
              *reinterpret_cast<uint2 *>(a.q_row + m * a.ld_q_row + oc) = q;
              if ((lane & 3) == 0) a.s_row[m * a.ld_s_row + (oc >> 5)] = (uint8_t)b;
            }
          }
        }
      }
      // keep one group of loads in flight per wave: without this fence the
      // scheduler hoists all 16 rows' loads and the kernel runs at one wave
      // per SIMD (or spills)
      __builtin_amdgcn_sched_barrier(0);
    }

    // column blocks: combine the two 16-row halves, then quantize down each column
#pragma unroll
    for (int o = 0; o < Op::OUT; o++)
#pragma unroll
      for (int r = 0; r < 16; r++)
#pragma unroll
        for (int k = 0; k < 4; k++)
          // opaque to the optimizer: the fp32 unpacks are redone column by
          // column instead of keeping all 128 unpacked values live
          asm volatile("" : "+v"(val[o][r][k]));
#pragma unroll
    for (int o = 0; o < Op::OUT; o++) {
#pragma unroll
      for (int k = 0; k < 4; k++) cmax[o][k] = pk_max(cmax[o][k], swap_halves(cmax[o][k]));
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const u32 am = (c & 1) ? (cmax[o][c >> 1] >> 16) : (cmax[o][c >> 1] & 0xffffu);
        const u32 b = e8m0_rceil(am);
        const float d = descale_of(b);
        u32 q[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const u32 *v0 = val[o][4 * i], *v1 = val[o][4 * i + 1], *v2 = val[o][4 * i + 2], *v3 = val[o][4 * i + 3];
          const int k = c >> 1;
          float f0, f1, f2, f3;
          if (c & 1) {
            f0 = hi_f(v0[k]); f1 = hi_f(v1[k]); f2 = hi_f(v2[k]); f3 = hi_f(v3[k]);
          } else {
            f0 = lo_f(v0[k]); f1 = lo_f(v1[k]); f2 = lo_f(v2[k]); f3 = lo_f(v3[k]);
          }
          int t = __builtin_amdgcn_cvt_pk_fp8_f32(f0 * d, f1 * d, 0, false);
          q[i] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(f2 * d, f3 * d, t, true);
        }
        if (b == 255u) q[0] = q[1] = q[2] = q[3] = 0x7f7f7f7fu;
        if (colok) {
          const int64_t orow = o * a.N + col + c;
          *reinterpret_cast<uint4 *>(qc + orow * a.ld_q_col + mr) = make_uint4(q[0], q[1], q[2], q[3]);
          if (half == 0) sc[orow * a.ld_s_col + (mblk >> 5)] = (uint8_t)b;
        }
        __builtin_amdgcn_sched_barrier(0);  // one column's floats live at a time
      }
    }
  }
}

}  // namespace mx
