// smla_ceiling.hip -- measured ceilings of one MI355X for the forward pass's
// roofline fractions (include/smla_ceiling.h).  Not part of the forward pass:
// the benchmark loads this library beside libsparsemla to put its achieved
// rates next to what the same device reaches on the bare resource.
//
//   stream read   every byte of a buffer read once with 16-byte loads
//   gather        the rows a top-k index stream names, read once with 16-byte
//                 loads in two access patterns (one row per 64-lane load, or
//                 eight rows x 128 bytes per load), no arithmetic beyond
//                 folding the bytes into one word per lane so the loads are live
//   lds read      16-byte LDS reads at conflict-free addresses, 1 - 16 waves
//                 per compute unit
//   mfma          back-to-back v_mfma_f32_16x16x32_bf16 (or the e4m3
//                 16x16x128 form) on independent accumulators
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_ceiling.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

constexpr int kThreads = 256;

// Grid-stride read of n16 16-byte chunks, 8 loads in flight per lane.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Gather: wave w of the grid reads list entries [e0, e1) of the flattened
// [T, K] index list, RIF rows in flight per wave; invalid entries are skipped.
// Two access patterns over the same bytes:
//   SPREAD = false  one row per 64-lane load (lane l: 16 bytes at 16 l of a
//                   1 KiB piece of one row)
//   SPREAD = true   eight rows per 64-lane load (lane l: row l / 8, 16 bytes
//                   at 16 (l mod 8) of a 128-byte piece), every row covered by
//                   ROW / 128 such loads
template <int ROW, bool SPREAD, int RIF>
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint8_t* __restrict__ kv, int64_t N,
                                                          const int32_t* __restrict__ idx, int64_t n_entries,
                                                          int64_t per_wave, uint32_t* __restrict__ sink) {
  constexpr int NL = SPREAD ? (RIF / 8) * ((ROW + 127) / 128) : RIF * ((ROW + 1023) / 1024);   // loads per batch
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t e0 = wave * per_wave;
  const int64_t e1 = e0 + per_wave < n_entries ? e0 + per_wave : n_entries;
  uint32_t acc = 0;
  for (int64_t e = e0; e < e1; e += 64) {
    const int my = (e + lane < e1) ? idx[e + lane] : -1;
    const int cnt = (int)((e1 - e) < 64 ? (e1 - e) : 64);
    for (int r0 = 0; r0 < cnt; r0 += RIF) {
      u32x4 v[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        int rr, off;
        if constexpr (SPREAD) {
          constexpr int PPR = (ROW + 127) / 128;     // 128-byte pieces per row
          rr = r0 + 8 * (j / PPR) + (lane >> 3);
          off = 128 * (j % PPR) + 16 * (lane & 7);
        } else {
          constexpr int PPR = (ROW + 1023) / 1024;   // 1 KiB pieces per row
          rr = r0 + j / PPR;
          off = 1024 * (j % PPR) + 16 * lane;
        }
        const int sl = __shfl(my, rr & 63);
        const bool ok = rr < cnt && sl >= 0 && (int64_t)sl < N && off < ROW;
        const uint8_t* row = kv + (ok ? (int64_t)sl * ROW : 0);
        v[j] = ok ? *reinterpret_cast<const u32x4*>(row + off) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// LDS reads: each wave reads `iters` rounds of 8 x 16 bytes per lane from a
// 64 KiB workgroup buffer at conflict-free addresses (lane l, read j: chunk
// (l + 64 j + 512 wave) mod 4096), folding them into one word.
__global__ __launch_bounds__(1024) void lds_read_kernel(int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
  for (int i = threadIdx.x; i < 4096; i += blockDim.x)
    *reinterpret_cast<u32x4*>(buf + 16 * i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = *reinterpret_cast<const u32x4*>(buf + 16 * ((lane + 64 * j + 512 * wave + it) & 4095));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][3];
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// MFMA: each wave runs `iters` rounds of 8 independent accumulator chains.
template <bool FP8>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!FP8) {
    const u32x4 a = {0x3f803f80u + lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const u32x4 b = {0x3c003c00u, 0x3c003c00u + lane, 0x3c003c00u, 0x3c003c00u};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
    }
  } else {
    const i32x8 a = {0x38383838 + lane, 0x38383838, 0x38383838, 0x38383838,
                     0x38383838, 0x38383838, 0x38383838, 0x38383838};
    const i32x8 b = {0x30303030, 0x30303030 + lane, 0x30303030, 0x30303030,
                     0x30303030, 0x30303030, 0x30303030, 0x30303030};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int smla_ceiling_stream_read(const void* src, int64_t bytes, void* sink, int64_t sink_bytes, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || ((uintptr_t)src % 16)) return 1;
  const int blocks = 4096;
  if (sink_bytes < (int64_t)blocks * kThreads * 4) return 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int smla_ceiling_gather(const void* kv_pool, int64_t N, int32_t row_bytes, const int32_t* idx, int64_t n_entries,
                        int32_t waves, int32_t pattern, void* sink, int64_t sink_bytes, void* stream) {
  if (!kv_pool || !idx || !sink || N < 1 || n_entries < 1 || waves < 4 || waves % 4 || pattern < 0 || pattern > 3)
    return 1;
  if (sink_bytes < (int64_t)waves * 64 * 4) return 2;
  const int64_t per_wave = (n_entries + waves - 1) / waves;
  const dim3 gd((unsigned)(waves / 4)), bd(kThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* kv = static_cast<const uint8_t*>(kv_pool);
  uint32_t* out = static_cast<uint32_t*>(sink);
#define SMLA_GATHER(ROWB)                                                                                     \
  case ROWB:                                                                                                  \
    if (pattern == 0)                                                                                         \
      hipLaunchKernelGGL((gather_kernel<ROWB, false, 8>), gd, bd, 0, s, kv, N, idx, n_entries, per_wave, out); \
    else if (pattern == 1)                                                                                    \
      hipLaunchKernelGGL((gather_kernel<ROWB, false, 16>), gd, bd, 0, s, kv, N, idx, n_entries, per_wave, out); \
    else if (pattern == 2)                                                                                    \
      hipLaunchKernelGGL((gather_kernel<ROWB, true, 8>), gd, bd, 0, s, kv, N, idx, n_entries, per_wave, out); \
    else                                                                                                      \
      hipLaunchKernelGGL((gather_kernel<ROWB, true, 16>), gd, bd, 0, s, kv, N, idx, n_entries, per_wave, out); \
    break;
  switch (row_bytes) {
    SMLA_GATHER(1024)
    SMLA_GATHER(512)
    SMLA_GATHER(1152)
    SMLA_GATHER(576)
    default: return 1;
  }
#undef SMLA_GATHER
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int smla_ceiling_lds_read(int32_t blocks, int32_t threads, int32_t iters, void* sink, int64_t sink_bytes,
                          void* stream) {
  if (!sink || blocks < 1 || iters < 1 || threads < 64 || threads > 1024 || threads % 64) return 1;
  if (sink_bytes < (int64_t)blocks * threads * 4) return 2;
  hipLaunchKernelGGL(lds_read_kernel, dim3(blocks), dim3(threads), 0, static_cast<hipStream_t>(stream), iters,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int smla_ceiling_mfma(int32_t fp8, int32_t blocks, int32_t iters, void* sink, int64_t sink_bytes, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return 1;
  if (sink_bytes < (int64_t)blocks * kThreads * 4) return 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, iters, static_cast<float*>(sink));
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, iters, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
