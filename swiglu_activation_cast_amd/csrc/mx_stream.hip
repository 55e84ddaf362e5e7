// mx_stream.hip -- libmxstream.so: the streaming bandwidth probe declared in
// mxstream.h.  Each workgroup walks chunks b, b + grid, ... of every buffer;
// a chunk is 256 threads x U consecutive 16-byte accesses (4096 U bytes),
// thread t touching bytes 16 (t + 256 u) of the chunk, so each wavefront's
// access is 1 KiB contiguous.  All loads of a chunk are issued before its
// stores.  The chunk count divides the buffers exactly, so every access is
// in bounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxstream.h"

namespace {

typedef uint32_t u32;
typedef u32 u32x4_t __attribute__((ext_vector_type(4)));
#define MXS_GLOBAL __attribute__((address_space(1)))

struct StreamArgs {
  const u32x4_t *in[4];
  u32x4_t *out[2];
  int64_t n_chunks;
};

template <int NR, int NW, int U>
__global__ __launch_bounds__(256) void k_stream(const StreamArgs a) {
  for (int64_t c = blockIdx.x; c < a.n_chunks; c += gridDim.x) {
    const int64_t base = c * (256 * U) + threadIdx.x;
    u32x4_t v[NR][U];
#pragma unroll
    for (int j = 0; j < NR; j++)
#pragma unroll
      for (int u = 0; u < U; u++)
        v[j][u] = __builtin_nontemporal_load((const MXS_GLOBAL u32x4_t *)(a.in[j] + base + 256 * u));
#pragma unroll
    for (int j = 0; j < NW; j++)
#pragma unroll
      for (int u = 0; u < U; u++) {
        // every input feeds one output, so no load is dead
        u32x4_t x = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NR; i++)
          if (NR >= NW ? (i % NW == j) : (i == j % NR)) x ^= v[i][u];
        __builtin_nontemporal_store(x, (MXS_GLOBAL u32x4_t *)(a.out[j] + base + 256 * u));
      }
  }
}

template <int U>
const void *pick(int nr, int nw) {
#define MXS_CASE(R, W) \
  if (nr == R && nw == W) return (const void *)&k_stream<R, W, U>;
  MXS_CASE(1, 1) MXS_CASE(2, 1) MXS_CASE(3, 1) MXS_CASE(4, 1)
  MXS_CASE(1, 2) MXS_CASE(2, 2) MXS_CASE(3, 2) MXS_CASE(4, 2)
#undef MXS_CASE
  return nullptr;
}

}  // namespace

extern "C" int mxstream_mix(const void *const *in, int n_in, void *const *out, int n_out, int64_t bytes, int unroll,
                            int grid, void *stream) {
  if (!in || !out) return 1;
  if (n_in < 1 || n_in > 4 || n_out < 1 || n_out > 2 || (unroll != 2 && unroll != 4 && unroll != 8)) return 2;
  if (grid < 1 || grid > (1 << 20) || bytes <= 0 || bytes % (4096 * (int64_t)unroll) != 0) return 2;
  StreamArgs a{};
  for (int j = 0; j < n_in; j++) {
    if (!in[j]) return 1;
    if ((uintptr_t)in[j] & 15u) return 2;
    a.in[j] = static_cast<const u32x4_t *>(in[j]);
  }
  for (int j = 0; j < n_out; j++) {
    if (!out[j]) return 1;
    if ((uintptr_t)out[j] & 15u) return 2;
    a.out[j] = static_cast<u32x4_t *>(out[j]);
  }
  a.n_chunks = bytes / (4096 * (int64_t)unroll);
  const void *k = unroll == 2 ? pick<2>(n_in, n_out) : unroll == 4 ? pick<4>(n_in, n_out) : pick<8>(n_in, n_out);
  void *kargs[] = {&a};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(256), kargs, 0, (hipStream_t)stream) == hipSuccess ? 0 : 7;
}
