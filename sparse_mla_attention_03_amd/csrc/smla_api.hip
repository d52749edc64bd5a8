// smla_api.hip -- the C ABI of libsparsemla: argument validation, split-K
// planning, workspace carving and kernel launches (include/sparse_mla.h).
//
// Every check runs on the host before anything is launched; a failed check
// returns a status, records a reason for sparse_mla_last_error() and leaves
// out/lse untouched.  The library allocates no device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "sparse_mla.h"
#include "smla_kernels.h"

namespace {

thread_local std::string g_last_error;

smla_status_t fail(smla_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
smla_status_t fail(smla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, cached per device id (read-only after
// the first query; benign races write the same value).
constexpr int kMaxDevices = 64;
// workspace bytes per (split, token, head) partial row: 512 fp16 values, four
// fp32 quarter scales and one fp32 lse
constexpr size_t kPartRowBytes = smla::kDV * sizeof(uint16_t) + 4 * sizeof(float) + sizeof(float);
std::atomic<int> g_cu_count[kMaxDevices];

smla_status_t device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) { *cus = c; return SMLA_OK; }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || c <= 0)
    return fail(SMLA_ERR_HIP, "hipDeviceGetAttribute(CU count): %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return SMLA_OK;
}

// ---- the allocation-free entry point's scratch ---------------------------------
// Split partials of sparse_mla_fwd_noalloc live in this array instead of a caller
// workspace.  Each device the library runs on holds its own copy until the
// process ends.  Host code never uses the array's name as an address (on the host
// it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = SMLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

smla_status_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SMLA_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table covers", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(SMLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *ptr = p;
  return SMLA_OK;
}

struct Plan {
  int32_t S = 1;        // split-K factor
  int32_t rps = 0;      // top-k entries per split (multiple of kBK)
  size_t ws_bytes = 0;  // workspace: S*T*H*512 fp16 partials, S*T*H*4 fp32 scales, S*T*H fp32 lse
};

smla_status_t check_sizes(int64_t T, int64_t H, int64_t K, int64_t Dqk, int32_t kv_dtype) {
  if (T < 0 || H <= 0 || K < 0 || Dqk <= 0)
    return fail(SMLA_ERR_SHAPE, "bad sizes T=%lld H=%lld K=%lld Dqk=%lld", (long long)T,
                (long long)H, (long long)K, (long long)Dqk);
  if (kv_dtype != SMLA_KV_BF16 && kv_dtype != SMLA_KV_FP8_E4M3)
    return fail(SMLA_ERR_DTYPE, "unknown kv dtype %d", kv_dtype);
  if (H % 16 != 0)
    return fail(SMLA_ERR_UNSUPPORTED, "H=%lld unsupported: heads must be a multiple of 16", (long long)H);
  if (Dqk != 512 && Dqk != 576)
    return fail(SMLA_ERR_UNSUPPORTED, "Dqk=%lld unsupported: rows must be 512 or 576 wide", (long long)Dqk);
  if (T > (1 << 24) || H > 4096 || K > (1 << 24))
    return fail(SMLA_ERR_SHAPE, "sizes out of range T=%lld H=%lld K=%lld", (long long)T,
                (long long)H, (long long)K);
  return SMLA_OK;
}

// Split-K choice: enough (token, head group, split) units to give every
// compute unit one workgroup, but at least 256 list entries per split (below
// that a split's fixed cost and the combine outweigh the parallelism gained).
smla_status_t make_plan(int64_t T, int64_t H, int64_t K, int32_t req, Plan* plan) {
  const int64_t tiles = (K + smla::kBK - 1) / smla::kBK;
  const int64_t HG = H / smla::heads_per_workgroup(H);
  int64_t S = 1;
  if (req < 0 || req > SMLA_MAX_SPLITS)
    return fail(SMLA_ERR_INVALID_ARG, "num_splits=%d outside 0..%d", req, SMLA_MAX_SPLITS);
  if (req > 0) {
    S = req;
  } else if (T > 0 && tiles > 1) {
    int cus = 0;
    smla_status_t st = device_cu_count(&cus);
    if (st != SMLA_OK) return st;
    const int64_t units = T * HG;
    if (units < cus) S = (cus + units - 1) / units;
    const int64_t max_by_size = tiles / 4;   // 4 x 64 entries per split at least
    if (S > max_by_size) S = max_by_size > 0 ? max_by_size : 1;
  }
  if (S > tiles) S = tiles > 0 ? tiles : 1;
  if (S > SMLA_MAX_SPLITS) S = SMLA_MAX_SPLITS;
  const int64_t tps = tiles > 0 ? (tiles + S - 1) / S : 1;   // tiles per split
  if (tiles > 0) S = (tiles + tps - 1) / tps;                 // drop empty splits
  plan->S = (int32_t)S;
  plan->rps = (int32_t)(tps * smla::kBK);
  plan->ws_bytes = S > 1 ? (size_t)S * T * H * kPartRowBytes : 0;
  return SMLA_OK;
}

// Per-token lengths: the planning kernel picks the unit length from the
// batch's total; the host only sizes for it.  With HG head groups and C compute
// units the batch has at most T + C / HG units and its split tokens fewer than
// 2 C / HG partial rows (see smla_plan_kernel).  Workspace: the unit table, the
// unit count, per-token first row / count, then partials and lse per row.
struct VarlenLayout {
  size_t units, count, first, tcount, part_o, part_scale, part_lse, total;
  int32_t max_units, max_prows, HG, cus;
};
smla_status_t varlen_layout(int64_t T, int64_t H, VarlenLayout* L) {
  auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
  int cus = 0;
  smla_status_t st = device_cu_count(&cus);
  if (st != SMLA_OK) return st;
  const int64_t HG = H / smla::heads_per_workgroup(H);
  const int64_t per = (cus + HG - 1) / HG;
  int64_t U = T + per + 1;
  const int64_t P = 2 * per + 1;
  // a smaller unit table, for tests of what a dropped unit does (never larger)
  if (const char* cap = getenv("SPARSEMLA_TEST_UNIT_TABLE")) {
    const long long c = atoll(cap);
    if (c >= 1 && c < U) U = c;
  }
  L->max_units = (int32_t)U;
  L->max_prows = (int32_t)P;
  L->HG = (int32_t)HG;
  L->cus = cus;
  L->units = 0;
  L->count = up16((size_t)U * 16);
  L->first = L->count + 16;
  L->tcount = up16(L->first + (size_t)T * 4);
  L->part_o = up16(L->tcount + (size_t)T * 4);
  L->part_scale = L->part_o + (size_t)P * H * smla::kDV * sizeof(uint16_t);
  L->part_lse = L->part_scale + (size_t)P * H * 4 * sizeof(float);
  L->total = L->part_lse + (size_t)P * H * sizeof(float);
  return SMLA_OK;
}

smla_status_t fwd_impl(const void* q, int64_t T, int64_t H, int64_t Dqk, int64_t q_stride_t,
                       int64_t q_stride_h, const void* kv_pool, int32_t kv_dtype, int64_t num_blocks,
                       int64_t block_size, const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                       float sm_scale, float kv_scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream, const smla_options_t* opts,
                       const int32_t* topk_len = nullptr, bool noalloc = false) {
  g_last_error.clear();
  smla_status_t st = check_sizes(T, H, K, Dqk, kv_dtype);
  if (st != SMLA_OK) return st;
  if (num_blocks < 0 || block_size <= 0)
    return fail(SMLA_ERR_SHAPE, "bad pool shape num_blocks=%lld block_size=%lld",
                (long long)num_blocks, (long long)block_size);
  if (q_stride_t < 0 || q_stride_h < 0 || idx_stride_t < 0)
    return fail(SMLA_ERR_SHAPE, "negative stride");
  if (!std::isfinite(sm_scale) || !std::isfinite(kv_scale))
    return fail(SMLA_ERR_INVALID_ARG, "sm_scale and kv_scale must be finite");
  int32_t req = 0;
  bool bf16_dots = false;
  float q_scale = 0.0f;   // > 0: q holds e4m3 codes
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (opts) {
    if (opts->dot_precision != SMLA_DOTS_DEFAULT && opts->dot_precision != SMLA_DOTS_BF16)
      return fail(SMLA_ERR_INVALID_ARG, "options.dot_precision=%d unknown", opts->dot_precision);
    if (opts->dot_precision == SMLA_DOTS_BF16 && kv_dtype != SMLA_KV_FP8_E4M3)
      return fail(SMLA_ERR_INVALID_ARG, "options.dot_precision selects bf16 dots for e4m3 KV only");
    if (opts->sinks && !aligned(opts->sinks, 4)) return fail(SMLA_ERR_ALIGN, "sinks must be 4-byte aligned");
    for (int i = 0; i < 3; ++i)
      if (opts->reserved[i] != 0) return fail(SMLA_ERR_INVALID_ARG, "options.reserved[%d] must be 0", i);
    if (!(opts->q_scale == 0.0f) && !(opts->q_scale > 0.0f && std::isfinite(opts->q_scale)))
      return fail(SMLA_ERR_INVALID_ARG, "options.q_scale must be 0 or positive and finite");
    if (opts->q_scale > 0.0f && (kv_dtype != SMLA_KV_FP8_E4M3 || opts->dot_precision != SMLA_DOTS_DEFAULT))
      return fail(SMLA_ERR_INVALID_ARG, "pre-quantised q (options.q_scale) needs e4m3 KV with e4m3 dots");
    req = opts->num_splits;
    bf16_dots = opts->dot_precision == SMLA_DOTS_BF16;
    q_scale = opts->q_scale;
    ev0 = static_cast<hipEvent_t>(opts->kernel_events[0]);
    ev1 = static_cast<hipEvent_t>(opts->kernel_events[1]);
    if ((ev0 == nullptr) != (ev1 == nullptr))
      return fail(SMLA_ERR_INVALID_ARG, "options.kernel_events: give both events or neither");
  }
  if (req < 0 || req > SMLA_MAX_SPLITS)
    return fail(SMLA_ERR_INVALID_ARG, "num_splits=%d outside 0..%d", req, SMLA_MAX_SPLITS);
  if (T == 0) return SMLA_OK;
  if (!q || !kv_pool || !out || !lse || (K > 0 && !topk_idx))
    return fail(SMLA_ERR_NULL, "null tensor pointer (q, kv_pool, topk_idx, out and lse are required)");
  if (!aligned(q, 16) || q_stride_t % 8 || q_stride_h % 8)
    return fail(SMLA_ERR_ALIGN, "q must be 16-byte aligned with strides that are multiples of 8 elements");
  if (q_scale > 0.0f && (q_stride_t % 16 || q_stride_h % 16))
    return fail(SMLA_ERR_ALIGN, "pre-quantised q needs strides that are multiples of 16 bytes");
  if (!aligned(kv_pool, 16)) return fail(SMLA_ERR_ALIGN, "kv_pool must be 16-byte aligned");
  if (!aligned(out, 16)) return fail(SMLA_ERR_ALIGN, "out must be 16-byte aligned");
  if (!aligned(lse, 4) || (topk_idx && !aligned(topk_idx, 4)))
    return fail(SMLA_ERR_ALIGN, "lse and topk_idx must be 4-byte aligned");
  const bool varlen = topk_len != nullptr;
  VarlenLayout VL{};
  if (varlen && !aligned(topk_len, 4)) return fail(SMLA_ERR_ALIGN, "topk_len must be 4-byte aligned");
  if (varlen && req != 0)
    return fail(SMLA_ERR_INVALID_ARG, "num_splits must be 0 with per-token lengths (the split is per token)");
  if (varlen && T > 0x7fffffffLL / 64)
    return fail(SMLA_ERR_UNSUPPORTED, "T=%lld too large for the per-token plan", (long long)T);

  Plan plan;
  if (varlen) {
    st = varlen_layout(T, H, &VL);
    plan.S = 1;
    plan.rps = 0;
    plan.ws_bytes = VL.total;
  } else {
    st = make_plan(T, H, K, req, &plan);
    if (st == SMLA_OK && noalloc && plan.ws_bytes > kScratchBytes) {
      // the library's own split choice is capped so its partials fit the scratch
      // (one split needs none); an explicit request that does not fit is refused
      if (req != 0)
        return fail(SMLA_ERR_WORKSPACE, "%d splits need %zu bytes of partials, beyond the %zu-byte scratch",
                    plan.S, plan.ws_bytes, kScratchBytes);
      const int64_t fit = (int64_t)(kScratchBytes / ((size_t)T * H * kPartRowBytes));
      st = make_plan(T, H, K, (int32_t)(fit > 1 ? fit : 1), &plan);
    }
  }
  if (st != SMLA_OK) return st;
  if (noalloc && plan.ws_bytes > 0) {
    st = device_scratch(&workspace);
    if (st != SMLA_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(SMLA_ERR_WORKSPACE, "workspace of %zu bytes needed for %d splits, got %zu",
                  plan.ws_bytes, plan.S, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(SMLA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }

  smla::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_st = q_stride_t;
  p.q_sh = q_stride_h;
  p.kv = static_cast<const uint8_t*>(kv_pool);
  p.N = num_blocks * block_size;
  p.idx = topk_idx;
  p.idx_st = idx_stride_t;
  p.T = (int32_t)T;
  p.H = (int32_t)H;
  p.K = (int32_t)K;
  p.S = plan.S;
  p.rps = plan.rps;
  p.sm_scale = sm_scale;
  p.kv_scale = kv_scale;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.sinks = opts ? opts->sinks : nullptr;
  p.q_scale = q_scale;
  const bool combine = varlen || plan.S > 1;
  if (varlen) {
    const VarlenLayout& L = VL;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    p.units = reinterpret_cast<const int4*>(ws + L.units);
    p.num_units = reinterpret_cast<const int32_t*>(ws + L.count);
    p.tok_first = reinterpret_cast<const int32_t*>(ws + L.first);
    p.tok_count = reinterpret_cast<const int32_t*>(ws + L.tcount);
    p.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
    p.part_scale = reinterpret_cast<float*>(ws + L.part_scale);
    p.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
    p.max_units = L.max_units;
    p.max_prows = L.max_prows;
  } else if (plan.S > 1) {
    const size_t rows = (size_t)plan.S * T * H;   // (split, token, head) partial rows
    p.part_o = static_cast<uint16_t*>(workspace);
    p.part_scale = reinterpret_cast<float*>(p.part_o + rows * smla::kDV);
    p.part_lse = p.part_scale + rows * 4;
  }
  // whole long lists of 512-wide bf16 rows in 16-head groups, with at least
  // two workgroups per compute unit: the kernel that runs two per unit
  if (plan.S == 1 && !varlen && kv_dtype == SMLA_KV_BF16 && Dqk == 512 && smla::heads_per_workgroup(H) == 16 &&
      K > 128) {
    int cus = 0;
    st = device_cu_count(&cus);
    if (st != SMLA_OK) return st;
    p.prefill16 = T * (H / 16) >= 2 * (int64_t)cus ? 1 : 0;
  }
  if (getenv("SPARSEMLA_LOG"))
    fprintf(stderr, "[sparsemla] T=%lld H=%lld Dqk=%lld K=%lld kv=%s splits=%d rows/split=%d prefill16=%d\n",
            (long long)T, (long long)H, (long long)Dqk, (long long)K, kv_dtype ? "e4m3" : "bf16",
            plan.S, plan.rps, p.prefill16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (varlen) {
    smla::PlanParams q{};
    q.lens = topk_len;
    q.T = (int32_t)T;
    q.K = (int32_t)K;
    q.HG = VL.HG;
    q.cus = VL.cus;
    q.max_units = VL.max_units;
    q.max_prows = VL.max_prows;
    q.units = const_cast<int4*>(p.units);
    q.num_units = const_cast<int32_t*>(p.num_units);
    q.tok_first = const_cast<int32_t*>(p.tok_first);
    q.tok_count = const_cast<int32_t*>(p.tok_count);
    e = smla::launch_plan(q, s);
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "plan kernel launch: %s", hipGetErrorString(e));
  }
  e = smla::launch_fwd(p, kv_dtype == SMLA_KV_FP8_E4M3, bf16_dots, (int)Dqk, s, ev0, ev1);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "forward kernel launch: %s", hipGetErrorString(e));
  if (combine) {
    e = smla::launch_combine(p, s);
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  }
  return SMLA_OK;
}

}  // namespace

extern "C" {

smla_status_t sparse_mla_fwd_varlen(const void* q, int64_t T, int64_t H, int64_t Dqk, int64_t q_stride_t,
                                    int64_t q_stride_h, const void* kv_pool, int32_t kv_dtype,
                                    int64_t num_blocks, int64_t block_size, const int32_t* topk_idx, int64_t K,
                                    int64_t idx_stride_t, const int32_t* topk_len, float sm_scale,
                                    float kv_scale, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream, const smla_options_t* opts) {
  if (T > 0 && !topk_len) {
    g_last_error.clear();
    return fail(SMLA_ERR_NULL, "topk_len is required");
  }
  static const int32_t kNone = 0;
  return fwd_impl(q, T, H, Dqk, q_stride_t, q_stride_h, kv_pool, kv_dtype, num_blocks, block_size, topk_idx,
                  K, idx_stride_t, sm_scale, kv_scale, out, lse, workspace, workspace_bytes, stream, opts,
                  T > 0 ? topk_len : &kNone);
}

size_t sparse_mla_workspace_bytes_varlen(int64_t T, int64_t H, int64_t K, int64_t Dqk, int32_t kv_dtype) {
  g_last_error.clear();
  if (check_sizes(T, H, K, Dqk, kv_dtype) != SMLA_OK) return (size_t)-1;
  if (T == 0) return 0;
  VarlenLayout L{};
  if (varlen_layout(T, H, &L) != SMLA_OK) return (size_t)-1;
  return L.total;
}

smla_status_t sparse_mla_fwd(const void* q, int64_t T, int64_t H, int64_t Dqk, int64_t q_stride_t,
                             int64_t q_stride_h, const void* kv_pool, int32_t kv_dtype,
                             int64_t num_blocks, int64_t block_size, const int32_t* topk_idx,
                             int64_t K, int64_t idx_stride_t, float sm_scale, float kv_scale,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return fwd_impl(q, T, H, Dqk, q_stride_t, q_stride_h, kv_pool, kv_dtype, num_blocks, block_size,
                  topk_idx, K, idx_stride_t, sm_scale, kv_scale, out, lse, workspace,
                  workspace_bytes, stream, nullptr);
}

smla_status_t sparse_mla_fwd_ex(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                int64_t q_stride_t, int64_t q_stride_h, const void* kv_pool,
                                int32_t kv_dtype, int64_t num_blocks, int64_t block_size,
                                const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                                float sm_scale, float kv_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream,
                                const smla_options_t* opts) {
  return fwd_impl(q, T, H, Dqk, q_stride_t, q_stride_h, kv_pool, kv_dtype, num_blocks, block_size,
                  topk_idx, K, idx_stride_t, sm_scale, kv_scale, out, lse, workspace,
                  workspace_bytes, stream, opts);
}

smla_status_t sparse_mla_fwd_noalloc(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                     int64_t q_stride_t, int64_t q_stride_h, const void* kv_pool,
                                     int32_t kv_dtype, int64_t num_blocks, int64_t block_size,
                                     const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                                     float sm_scale, float kv_scale, void* out, float* lse,
                                     void* stream, const smla_options_t* opts) {
  return fwd_impl(q, T, H, Dqk, q_stride_t, q_stride_h, kv_pool, kv_dtype, num_blocks, block_size,
                  topk_idx, K, idx_stride_t, sm_scale, kv_scale, out, lse, nullptr, 0, stream, opts,
                  nullptr, true);
}

int32_t sparse_mla_num_splits(int64_t T, int64_t H, int64_t K, int64_t Dqk, int32_t kv_dtype,
                              int32_t num_splits) {
  g_last_error.clear();
  if (check_sizes(T, H, K, Dqk, kv_dtype) != SMLA_OK) return 0;
  Plan plan;
  if (make_plan(T, H, K, num_splits, &plan) != SMLA_OK) return 0;
  return plan.S;
}

size_t sparse_mla_workspace_bytes(int64_t T, int64_t H, int64_t K, int64_t Dqk, int32_t kv_dtype,
                                  int32_t num_splits) {
  g_last_error.clear();
  if (check_sizes(T, H, K, Dqk, kv_dtype) != SMLA_OK) return (size_t)-1;
  Plan plan;
  if (make_plan(T, H, K, num_splits, &plan) != SMLA_OK) return (size_t)-1;
  return plan.ws_bytes;
}

smla_status_t sparse_mla_quantize_q_fp8(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                        int64_t q_stride_t, int64_t q_stride_h, uint8_t* codes,
                                        float* scales, void* stream) {
  g_last_error.clear();
  smla_status_t st = check_sizes(T, H, 0, Dqk, SMLA_KV_FP8_E4M3);
  if (st != SMLA_OK) return st;
  if (q_stride_t < 0 || q_stride_h < 0) return fail(SMLA_ERR_SHAPE, "negative stride");
  if (T == 0) return SMLA_OK;
  if (!q || !codes || !scales) return fail(SMLA_ERR_NULL, "null pointer (q, codes, scales)");
  if (!aligned(q, 16) || q_stride_t % 8 || q_stride_h % 8)
    return fail(SMLA_ERR_ALIGN, "q must be 16-byte aligned with strides that are multiples of 8 elements");
  if (!aligned(codes, 8) || !aligned(scales, 4))
    return fail(SMLA_ERR_ALIGN, "codes must be 8-byte and scales 4-byte aligned");
  hipError_t e = smla::launch_quantize_q(static_cast<const uint16_t*>(q), q_stride_t, q_stride_h,
                                         (int32_t)T, (int32_t)H, (int)Dqk, codes, scales,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "quantize kernel launch: %s", hipGetErrorString(e));
  return SMLA_OK;
}

smla_status_t sparse_mla_rope_concat_cache(const void* ql_nope, int64_t ql_stride_t, int64_t ql_stride_h,
                                           const void* q_pe, int64_t qpe_stride_t, int64_t qpe_stride_h,
                                           const void* kv_c, int64_t kvc_stride_t,
                                           const void* k_pe, int64_t kpe_stride_t,
                                           const int64_t* positions, const float* cos_sin_cache,
                                           int64_t max_pos, int32_t is_neox, int64_t T, int64_t H,
                                           void* q_out, int32_t q_out_dtype, float q_scale,
                                           const int64_t* slot_mapping, void* kv_cache, int32_t kv_dtype,
                                           int64_t num_blocks, int64_t block_size, float kv_scale,
                                           void* stream) {
  g_last_error.clear();
  if (T < 0 || H <= 0 || T > 0x7fffffff || H > 0x7fffffff || max_pos <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(SMLA_ERR_SHAPE, "bad sizes T=%lld H=%lld max_pos=%lld num_blocks=%lld block_size=%lld",
                (long long)T, (long long)H, (long long)max_pos, (long long)num_blocks, (long long)block_size);
  if (ql_stride_t < 0 || ql_stride_h < 0 || qpe_stride_t < 0 || qpe_stride_h < 0 || kvc_stride_t < 0 ||
      kpe_stride_t < 0)
    return fail(SMLA_ERR_SHAPE, "negative stride");
  if ((q_out_dtype != SMLA_KV_BF16 && q_out_dtype != SMLA_KV_FP8_E4M3) ||
      (kv_dtype != SMLA_KV_BF16 && kv_dtype != SMLA_KV_FP8_E4M3))
    return fail(SMLA_ERR_DTYPE, "q_out_dtype=%d / kv_dtype=%d unknown", q_out_dtype, kv_dtype);
  if (!(q_scale > 0.0f && std::isfinite(q_scale)) || !(kv_scale > 0.0f && std::isfinite(kv_scale)))
    return fail(SMLA_ERR_INVALID_ARG, "q_scale and kv_scale must be positive and finite");
  if (T > 0 && H + 1 > 0xffffffffLL / (72 * T))   // T (H + 1) 72 > 2^32 - 1, without forming the product
    return fail(SMLA_ERR_UNSUPPORTED, "T=%lld x H=%lld is beyond one launch (T*(H+1)*72 < 2^32)",
                (long long)T, (long long)H);
  if (T == 0) return SMLA_OK;
  if (!ql_nope || !q_pe || !kv_c || !k_pe || !positions || !cos_sin_cache || !q_out || !slot_mapping ||
      !kv_cache)
    return fail(SMLA_ERR_NULL, "null tensor pointer");
  const bool rows_ok = aligned(ql_nope, 16) && aligned(q_pe, 16) && aligned(kv_c, 16) && aligned(k_pe, 16) &&
                       ql_stride_t % 8 == 0 && ql_stride_h % 8 == 0 && qpe_stride_t % 8 == 0 &&
                       qpe_stride_h % 8 == 0 && kvc_stride_t % 8 == 0 && kpe_stride_t % 8 == 0;
  if (!rows_ok)
    return fail(SMLA_ERR_ALIGN, "ql_nope, q_pe, kv_c and k_pe rows must be 16-byte aligned (strides multiples of 8)");
  if (!aligned(cos_sin_cache, 16) || !aligned(q_out, 16) || !aligned(kv_cache, 16) || !aligned(positions, 8) ||
      !aligned(slot_mapping, 8))
    return fail(SMLA_ERR_ALIGN, "cos_sin_cache, q_out and kv_cache must be 16-byte aligned, positions and slot_mapping 8-byte");
  smla::RopeCacheParams p{};
  p.ql_nope = static_cast<const uint16_t*>(ql_nope);
  p.ql_st = ql_stride_t;
  p.ql_sh = ql_stride_h;
  p.q_pe = static_cast<const uint16_t*>(q_pe);
  p.qpe_st = qpe_stride_t;
  p.qpe_sh = qpe_stride_h;
  p.kv_c = static_cast<const uint16_t*>(kv_c);
  p.kvc_st = kvc_stride_t;
  p.k_pe = static_cast<const uint16_t*>(k_pe);
  p.kpe_st = kpe_stride_t;
  p.positions = positions;
  p.cos_sin = cos_sin_cache;
  p.max_pos = max_pos;
  p.T = (int32_t)T;
  p.H = (int32_t)H;
  p.q_out = static_cast<uint8_t*>(q_out);
  p.q_scale = q_scale;
  p.slot_mapping = slot_mapping;
  p.kv_cache = static_cast<uint8_t*>(kv_cache);
  p.N = num_blocks * block_size;
  p.kv_scale = kv_scale;
  hipError_t e = smla::launch_rope_cache(p, is_neox != 0, q_out_dtype == SMLA_KV_FP8_E4M3,
                                         kv_dtype == SMLA_KV_FP8_E4M3, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return SMLA_OK;
}

const char* sparse_mla_status_string(smla_status_t status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL: return "null pointer";
    case SMLA_ERR_SHAPE: return "bad shape or stride";
    case SMLA_ERR_DTYPE: return "unknown dtype";
    case SMLA_ERR_ALIGN: return "misaligned pointer or stride";
    case SMLA_ERR_INVALID_ARG: return "invalid argument";
    case SMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SMLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sparse_mla_last_error(void) { return g_last_error.c_str(); }

int32_t sparse_mla_abi_version(void) { return SMLA_ABI_VERSION; }

}  // extern "C"
