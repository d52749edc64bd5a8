/*
 * smla_ceiling.h -- measured ceilings of the device (libsmla_ceiling.so), the
 * denominators beside the published peaks when the benchmark reports how close
 * the sparse MLA forward pass comes to its roofline.  Not part of the forward
 * pass and not called by libsparsemla.
 *
 * All pointers are DEVICE pointers owned by the caller; each call launches one
 * kernel on `stream` (NULL = default stream) and returns at once.  Return
 * value: 0 = launched, 1 = bad argument, 2 = sink too small, 3 = launch failed.
 * `sink` receives one 32-bit word per thread (garbage to the caller; it keeps
 * the loads and products live).
 */
#ifndef SMLA_CEILING_H
#define SMLA_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every byte of src[0, bytes) once, 16-byte loads, 4096
 * workgroups of 256 threads.  bytes a multiple of 16, src 16-byte aligned;
 * sink >= 4096 * 256 * 4 bytes.  Rate = bytes / kernel time. */
int smla_ceiling_stream_read(const void* src, int64_t bytes, void* sink, int64_t sink_bytes, void* stream);

/* Gather with no arithmetic: the rows that a flattened top-k list names,
 * idx[0, n_entries) (slot ids into a pool of N rows of row_bytes each; ids
 * outside [0, N) are skipped), read once with 64 lanes x 16 bytes per load,
 * the entries split evenly over `waves` waves (a multiple of 4).  pattern:
 * 0 / 1 = one row per load, 8 / 16 rows in flight per wave; 2 / 3 = eight
 * rows x 128 bytes per load, 8 / 16 rows in flight.  row_bytes in {512, 576,
 * 1024, 1152}; sink >= waves * 256 bytes.  Rate = valid entries * row_bytes /
 * kernel time. */
int smla_ceiling_gather(const void* kv_pool, int64_t N, int32_t row_bytes, const int32_t* idx, int64_t n_entries,
                        int32_t waves, int32_t pattern, void* sink, int64_t sink_bytes, void* stream);

/* LDS read bandwidth: `blocks` workgroups of `threads` (64 .. 1024, a multiple
 * of 64) threads, each wave `iters` rounds of 8 x 16-byte LDS reads per lane at
 * conflict-free addresses of a 64 KiB buffer (one workgroup per compute unit).
 * sink >= blocks * threads * 4 bytes.  Rate = blocks * threads * iters * 128
 * bytes / kernel time. */
int smla_ceiling_lds_read(int32_t blocks, int32_t threads, int32_t iters, void* sink, int64_t sink_bytes,
                          void* stream);

/* MFMA throughput: `blocks` workgroups of four waves, each wave `iters` rounds
 * of 8 independent v_mfma_f32_16x16x32_bf16 (fp8 = 0: 16384 FLOP each) or
 * v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 (fp8 != 0: 65536 FLOP each).
 * sink >= blocks * 1024 bytes. */
int smla_ceiling_mfma(int32_t fp8, int32_t blocks, int32_t iters, void* sink, int64_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SMLA_CEILING_H */
