/* mxstream.h -- streaming bandwidth probe of libmxstream.so.
 *
 * Measurement infrastructure beside the MXFP8 casts (not part of their
 * boundary): it moves bytes between HBM buffers in a fixed read:write mix,
 * with the access widths and cache policy the casts use, so that a cast's
 * achieved bandwidth can be set against what plain streaming reaches at the
 * same mix.  The pages judge their casts against the device's peak HBM
 * bandwidth ("[mxfp8 moe training] add compile support", Perf analysis);
 * this probe measures the part of that peak a streaming kernel reaches.
 *
 * All pointers are device pointers; the call only enqueues work.
 */
#ifndef MXSTREAM_H
#define MXSTREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads n_in buffers in[0..n_in-1] and writes n_out buffers
 * out[0..n_out-1], `bytes` bytes each, once.  With n_in >= n_out, out[j]
 * is the XOR of the inputs i with i % n_out == j; otherwise out[j] is a copy
 * of in[j % n_in].  Every input byte is used.
 *
 *   n_in  in 1..4, n_out in 1..2: the read:write byte mix is n_in : n_out.
 *   bytes a positive multiple of 4096 * unroll; every buffer 16-byte aligned.
 *   unroll 2, 4 or 8: 16-byte accesses per buffer in flight in each thread.
 *   grid  workgroups (256 threads each), 1 .. 2^20; workgroup b handles
 *         chunks b, b + grid, ... of 4096 * unroll bytes of every buffer.
 *   stream a hipStream_t (NULL: the default stream).
 *
 * Loads and stores are nontemporal 16-byte global accesses.  Returns 0 on
 * success, 1 for a NULL pointer, 2 for a bad count, size or alignment, 7 if
 * the launch was refused.  Nothing is allocated or synchronized. */
int mxstream_mix(const void *const *in, int n_in, void *const *out, int n_out, int64_t bytes, int unroll,
                 int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXSTREAM_H */
