// smla_kernels.h -- host-side view of the libsparsemla kernels (launch wrappers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kDV = 512;        // V / out width
constexpr int kBK = 64;         // top-k entries (gathered rows) per pipeline tile
constexpr int kThreads = 256;   // 4 wavefronts per workgroup

struct FwdParams {
  const uint16_t* q;            // bf16 [T, H, Dqk], strides in elements
  int64_t q_st, q_sh;
  const uint8_t* kv;            // [N, Dqk] rows, bf16 or e4m3
  int64_t N;                    // number of slots
  const int32_t* idx;           // [T, K], row stride idx_st
  int64_t idx_st;
  int32_t T, H, K;
  int32_t S;                    // split-K factor (1 = write out/lse directly)
  int32_t rps;                  // top-k entries per split, multiple of kBK
  float sm_scale, kv_scale;
  uint16_t* out;                // bf16 [T, H, 512]
  float* lse;                   // fp32 [T, H]
  uint16_t* part_o;             // fp16 [P, H/16, 128, 16, 4] (split calls): 4-column chunk c
                                // of the 16 heads of a group side by side
  float* part_scale;            // fp32 [P, H, 4]: power-of-two scale of each 128-column quarter
  float* part_lse;              // fp32 [P, H]
  const float* sinks;           // fp32 [H] per-head sink logits (natural log), or null
  float q_scale;                // > 0: q holds e4m3 codes (byte strides), qhat = q_scale * code
  // per-token split plan (null = the uniform plan above): unit u covers
  // entries [kbeg, kend) of token t; a split token's units write partial rows
  // tok_first[t] .., a token's only unit (row -1) writes out / lse itself
  const int4* units;            // [max_units] {t, kbeg, kend, partial row or -1 = direct}
  const int32_t* num_units;     // U (device)
  const int32_t* tok_first;     // [T] first partial row of each split token
  const int32_t* tok_count;     // [T] its unit count
  int32_t max_units;            // upper bound on U (the grid is sized for it)
  int32_t max_prows;            // partial rows in the workspace
  int32_t prefill16;            // 1: 16-head groups of whole long bf16 lists, two
                                // workgroups per compute unit (smla_prefill.hip)
};

// The fused q-RoPE / q-concat / KV-concat / cache write (strides in elements).
struct RopeCacheParams {
  const uint16_t* ql_nope;      // bf16 [T, H, 512]
  int64_t ql_st, ql_sh;
  const uint16_t* q_pe;         // bf16 [T, H, 64]
  int64_t qpe_st, qpe_sh;
  const uint16_t* kv_c;         // bf16 [T, 512]
  int64_t kvc_st;
  const uint16_t* k_pe;         // bf16 [T, 64]
  int64_t kpe_st;
  const int64_t* positions;     // [T]
  const float* cos_sin;         // fp32 [max_pos, 64]: cos 0..31, sin 32..63
  int64_t max_pos;
  int32_t T, H;
  uint8_t* q_out;               // [T, H, 576] bf16 or e4m3
  float q_scale;
  const int64_t* slot_mapping;  // [T]
  uint8_t* kv_cache;            // [N, 576] bf16 or e4m3
  int64_t N;
  float kv_scale;
};

// Heads per workgroup for a head count (a multiple of 16).
inline int heads_per_workgroup(int64_t H) { return (H % 64 == 0) ? 64 : (H % 32 == 0) ? 32 : 16; }

// bf16_dots: e4m3 KV with bf16 QK dots (kv_fp8 must be set).  ev0 / ev1
// (both or neither): events that take the main kernel's own start and end
// timestamps.
hipError_t launch_fwd(const FwdParams& p, bool kv_fp8, bool bf16_dots, int dqk, hipStream_t stream,
                      hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_combine(const FwdParams& p, hipStream_t stream);
// 16-head groups on whole long lists of 512-wide bf16 rows (smla_prefill.hip)
hipError_t launch_prefill(const FwdParams& p, dim3 grid, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// the per-token split plan from list lengths (one workgroup)
struct PlanParams {
  const int32_t* lens;          // [T]
  int32_t T, K, HG, cus;
  int32_t max_units, max_prows;
  int4* units;                  // [max_units] {t, kbeg, kend, partial row or -1}
  int32_t* num_units;
  int32_t* tok_first;           // [T] first partial row of a split token
  int32_t* tok_count;           // [T] units of the token
};
hipError_t launch_plan(const PlanParams& q, hipStream_t stream);
hipError_t launch_rope_cache(const RopeCacheParams& p, bool neox, bool q8, bool kv8, hipStream_t stream);
hipError_t launch_quantize_q(const uint16_t* q, int64_t q_st, int64_t q_sh, int32_t T, int32_t H,
                             int dqk, uint8_t* codes, float* scales, hipStream_t stream);

}  // namespace smla
