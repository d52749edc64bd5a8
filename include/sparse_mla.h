/*
 * sparse_mla.h -- C ABI of libsparsemla, the sparse MLA attention forward pass
 * on AMD MI355X (gfx950).
 *
 * The operation (vLLM PR "[ROCm][Perf][GLM-5.3-Flash] Enable AITER sparse MLA
 * on gfx942, including FP8 KV", Overview and Details; vLLM PR "[ROCm][DSv4.1]
 * [Perf] Route gfx942 sparse MLA prefill to AITER pa_prefill_sparse", What
 * changed: one shared KV pool; vLLM PR "[ROCm][MLA][Perf] Fuse decode QK-RoPE
 * + Q-concat + KV-concat + KV-cache write for sparse MLA", Test plan: a cache
 * row is concat(kv_c, RoPE(k_pe)), so V is its first 512 columns):
 *
 *   every query token t has H heads (MQA style: all heads share one latent KV
 *   pool).  Token t attends only to the rows named by its top-k list
 *   topk_idx[t, 0..K-1]; a row is Dqk wide (512 rope-free, or 512 + 64 with
 *   RoPE) and V is its first 512 columns.  For each (t, h):
 *     s_j = sm_scale * <qhat[t,h,:], kv_scale * row_j[0:Dqk]>
 *     lse = ln sum_j exp(s_j)
 *     out = sum_j exp(s_j - lse) * kv_scale * row_j[0:512]
 *   Entries outside [0, N) (N = num_blocks * block_size), e.g. -1 padding,
 *   are never read and contribute nothing; duplicates count once per
 *   occurrence.  A token with no valid entry gets out = +0 and lse = -inf.
 *
 *   qhat = q for bf16 KV.  For OCP fp8-e4m3 KV the QK dots run in fp8 (unless
 *   options select bf16 dots or pass q pre-quantised, see smla_options_t): q is
 *   quantised inside the kernel per tile (the first page, Details: "the
 *   kernel quantizes q per tile"), a tile being heads [64g, min(64g+64, H))
 *   of one token over all Dqk columns:  s_q = amax|q| / 448 (fp32; 1 if the
 *   tile is all zero), code = e4m3_rne(q / s_q) (fp32 division), qhat =
 *   s_q * code.  PV runs in bf16 on exactly dequantised V.
 *
 * Memory: every tensor pointer is a DEVICE pointer owned by the caller; the
 * library allocates nothing and keeps no device memory.  Calls are
 * asynchronous on the given stream; results are valid once the stream reaches
 * them.  On any error status nothing is launched and out/lse are untouched.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 3
#define SMLA_DV 512          /* width of V and of out */
#define SMLA_MAX_SPLITS 64   /* upper bound on the split-K factor */

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL = 1,         /* a required pointer is NULL */
  SMLA_ERR_SHAPE = 2,        /* negative or out-of-range size or stride */
  SMLA_ERR_DTYPE = 3,        /* unknown kv dtype */
  SMLA_ERR_ALIGN = 4,        /* pointer or stride breaks the 16-byte rule */
  SMLA_ERR_INVALID_ARG = 5,  /* non-finite scale, bad option value */
  SMLA_ERR_UNSUPPORTED = 6,  /* well formed but not implemented (reason in last_error) */
  SMLA_ERR_WORKSPACE = 7,    /* workspace missing or too small */
  SMLA_ERR_HIP = 8           /* HIP runtime error (device query or launch) */
} smla_status_t;

typedef enum {
  SMLA_KV_BF16 = 0,          /* kv_pool holds bf16 */
  SMLA_KV_FP8_E4M3 = 1       /* kv_pool holds OCP e4m3 ("e4m3fn") codes */
} smla_kv_dtype_t;

/* Precision of the QK dots for e4m3 KV (options.dot_precision).  For bf16
 * KV the dots are always bf16 and this must be SMLA_DOTS_DEFAULT. */
typedef enum {
  SMLA_DOTS_DEFAULT = 0,     /* e4m3 KV: e4m3 dots with per-tile q quantisation */
  SMLA_DOTS_BF16 = 1         /* e4m3 KV: bf16 dots, q as given, K dequantised exactly
                                (the first page, Details: the dot precision is an
                                optional argument, and bf16 dots carry far less error) */
} smla_dot_precision_t;

typedef struct {
  int32_t num_splits;        /* split-K factor over each top-k list; 0 = automatic,
                                otherwise 1..SMLA_MAX_SPLITS */
  int32_t dot_precision;     /* smla_dot_precision_t */
  void* kernel_events[2];    /* optional instrumentation: two caller-created hipEvent_t
                                that take the start and end timestamps of the main
                                (gather + attention) kernel's own dispatch (not the split
                                combine); NULL = not recorded */
  const float* sinks;        /* optional DEVICE fp32 [H]: per-head attention-sink logit
                                sigma_h, in the units of s_j (finite, or -inf = no sink
                                for that head); NULL = no sinks.  The sink joins the
                                softmax normaliser only, as a key whose value row is zero
                                (the first page, Details, Limitations: sinks are passed
                                through to the kernel):
                                  lse = ln(exp(sigma_h) + sum_j exp(s_j))
                                  out = sum_j exp(s_j - lse) * kv_scale * row_j[0:512]
                                so a token with no valid entry gets out = +0 and
                                lse = sigma_h. */
  float q_scale;             /* 0 = q is bf16 (default).  > 0 (finite): q is already
                                quantised -- it holds OCP e4m3 codes [T, H, Dqk], one byte
                                per element (strides in bytes, multiples of 16), with
                                qhat = q_scale * code for every element (one per-tensor
                                scale; the first page, Details: gfx950 keeps the
                                pre-quantised q).  e4m3 KV with SMLA_DOTS_DEFAULT only; the
                                per-tile quantisation is skipped. */
  int32_t reserved[3];       /* must be zero */
} smla_options_t;

/*
 * sparse_mla_fwd -- the forward pass.
 *
 *   q            bf16 [T, H, Dqk]; element (t,h,d) at q[t*q_stride_t + h*q_stride_h + d].
 *                Strides are in elements, last dimension contiguous.  q, q_stride_t
 *                and q_stride_h must keep every row 16-byte aligned (pointer
 *                16-byte aligned, strides multiples of 8).  Strided (non-packed)
 *                q is computed correctly, never assumed packed.
 *   T, H, Dqk    tokens, heads (multiple of 16), row width (512 or 576).
 *   kv_pool      [num_blocks, block_size, Dqk] packed rows of kv_dtype, 16-byte
 *                aligned.  Viewed as N = num_blocks*block_size flat slots.
 *   topk_idx     int32 [T, K]; entry (t,k) at topk_idx[t*idx_stride_t + k]; each
 *                entry is a flat slot id in [0, N); anything else is padding.
 *   sm_scale     softmax scale (finite), e.g. 1/sqrt(Dqk).
 *   kv_scale     dequantisation multiplier applied to K and V (finite); 1.0 for
 *                bf16 pools, the per-tensor scale for fp8 pools.
 *   out          bf16 [T, H, 512], packed, 16-byte aligned (written).
 *   lse          fp32 [T, H], packed (written), natural log.
 *   workspace    device scratch of at least sparse_mla_workspace_bytes(...) bytes,
 *                16-byte aligned; may be NULL when that size is 0.  Its contents
 *                need no initialisation and are garbage afterwards.  Two calls
 *                that run concurrently must not share a workspace.
 *   stream       hipStream_t to launch on (NULL = default stream).
 *
 * T == 0 is a no-op.  K == 0 makes every token all-padding.
 */
smla_status_t sparse_mla_fwd(const void* q, int64_t T, int64_t H, int64_t Dqk,
                             int64_t q_stride_t, int64_t q_stride_h,
                             const void* kv_pool, int32_t kv_dtype,
                             int64_t num_blocks, int64_t block_size,
                             const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                             float sm_scale, float kv_scale,
                             void* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* Same as sparse_mla_fwd, with options (opts may be NULL = all defaults). */
smla_status_t sparse_mla_fwd_ex(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                int64_t q_stride_t, int64_t q_stride_h,
                                const void* kv_pool, int32_t kv_dtype,
                                int64_t num_blocks, int64_t block_size,
                                const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                                float sm_scale, float kv_scale,
                                void* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                void* stream, const smla_options_t* opts);

/*
 * sparse_mla_fwd_varlen -- the forward pass for a batch whose tokens use lists
 * of different lengths, e.g. decode tokens with full top-k lists next to early
 * prefill rows with short ones (vLLM PR "[ROCm][DSv4.1][Perf] Route gfx942
 * sparse MLA prefill to AITER pa_prefill_sparse", Gating and the review thread
 * after Test plan: a path without a split of the list costs decode-sized calls
 * about nine times more, so rows are routed by size).  Token t uses entries
 * topk_idx[t, 0 .. topk_len[t]) of its row; the rest of the row is never read.
 * The split over each list is chosen per token on the device: a token gets
 * ceil(len / R) units of R entries (R from the batch shape and the CU count,
 * a multiple of 64), and a token with one unit writes out / lse directly; the
 * others are merged by the combine kernel.  A small planning kernel runs
 * first (so the call stays capturable in a HIP graph: nothing comes back to
 * the host).
 *
 *   topk_len   int32 [T] on the device; values are clamped into [0, K].
 *   workspace  at least sparse_mla_workspace_bytes_varlen(T, H, K, Dqk, kv_dtype)
 *              bytes, 16-byte aligned.
 * Everything else as sparse_mla_fwd_ex; options.num_splits must be 0.
 */
smla_status_t sparse_mla_fwd_varlen(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                    int64_t q_stride_t, int64_t q_stride_h,
                                    const void* kv_pool, int32_t kv_dtype,
                                    int64_t num_blocks, int64_t block_size,
                                    const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                                    const int32_t* topk_len,
                                    float sm_scale, float kv_scale,
                                    void* out, float* lse,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream, const smla_options_t* opts);

/*
 * sparse_mla_fwd_noalloc -- sparse_mla_fwd_ex for callers that cannot allocate
 * device memory: code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation.  It takes no
 * workspace: split partials go to a scratch array of SMLA_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device it runs on (from the first call on that
 * device until the process ends).  The call itself allocates nothing.
 *
 * Arguments, results and errors as sparse_mla_fwd_ex.  With options.num_splits
 * = 0 the library's split choice is capped so that its partials
 * (splits * T * H * 1044 bytes; none for one split) fit the scratch; an explicit
 * num_splits whose partials do not fit returns SMLA_ERR_WORKSPACE before
 * anything is launched.  Every call on a device shares that device's scratch:
 * two calls that may overlap on one device (different streams without
 * ordering between them) race and give undefined results; calls ordered on
 * one stream are safe.  The scratch needs no clearing between calls (every
 * partial is written before the merge reads it).
 */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
smla_status_t sparse_mla_fwd_noalloc(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                     int64_t q_stride_t, int64_t q_stride_h,
                                     const void* kv_pool, int32_t kv_dtype,
                                     int64_t num_blocks, int64_t block_size,
                                     const int32_t* topk_idx, int64_t K, int64_t idx_stride_t,
                                     float sm_scale, float kv_scale,
                                     void* out, float* lse,
                                     void* stream, const smla_options_t* opts);

/* Workspace bytes sparse_mla_fwd_varlen needs (queries the current device's
 * CU count).  Returns (size_t)-1 on error. */
size_t sparse_mla_workspace_bytes_varlen(int64_t T, int64_t H, int64_t K, int64_t Dqk,
                                         int32_t kv_dtype);

/*
 * Split-K factor a call with these sizes runs with.  num_splits = 0: the
 * library's choice for the current device (it queries the compute-unit count).
 * num_splits > 0: that request, validated (<= SMLA_MAX_SPLITS) and reduced to
 * what the top-k length allows (every split gets whole 64-entry tiles).
 * Returns 0 on error (see sparse_mla_last_error).
 */
int32_t sparse_mla_num_splits(int64_t T, int64_t H, int64_t K, int64_t Dqk,
                              int32_t kv_dtype, int32_t num_splits);

/*
 * Workspace bytes a call with these sizes needs (num_splits as in
 * smla_options_t; 0 = automatic, which queries the current device).
 * Returns (size_t)-1 on error.
 */
size_t sparse_mla_workspace_bytes(int64_t T, int64_t H, int64_t K, int64_t Dqk,
                                  int32_t kv_dtype, int32_t num_splits);

/*
 * The fp8 per-tile q quantisation step on its own (the same device code the
 * fp8 forward pass runs before its QK dots), for checking it bit by bit.
 *   q       bf16 [T, H, Dqk] with strides as in sparse_mla_fwd.
 *   codes   uint8 [T, H, Dqk] packed (written): OCP e4m3 codes of q / s_q.
 *   scales  fp32 [T, ceil(H/64)] packed (written): s_q per (token, tile).
 */
smla_status_t sparse_mla_quantize_q_fp8(const void* q, int64_t T, int64_t H, int64_t Dqk,
                                        int64_t q_stride_t, int64_t q_stride_h,
                                        uint8_t* codes, float* scales, void* stream);

/*
 * sparse_mla_rope_concat_cache -- the step in front of the forward pass, fused
 * into one kernel (vLLM PR "[ROCm][MLA][Perf] Fuse decode QK-RoPE + Q-concat +
 * KV-concat + KV-cache write for sparse MLA", Summary and Test plan): it turns
 * a layer's absorbed query and new latent KV into the q and the cache rows the
 * forward pass reads.  For every token t and head h:
 *   q_out[t, h, 0:512]   = ql_nope[t, h, :]
 *   q_out[t, h, 512:576] = RoPE(q_pe[t, h, :], positions[t])
 *   cache row slot_mapping[t]: [0:512] = kv_c[t, :], [512:576] = RoPE(k_pe[t, :], positions[t])
 * RoPE rotates the 64 rope columns in pairs with cos_i = cos_sin_cache[p, i],
 * sin_i = cos_sin_cache[p, 32 + i] (i < 32):
 *   is_neox != 0: pairs (i, i + 32) ("rotate halves");  is_neox == 0: pairs (2i, 2i + 1)
 *   (x, y) -> (x cos_i - y sin_i, y cos_i + x sin_i)
 * each output the exact value of that expression rounded once to bf16 (nearest
 * even; the products are exact in fp64 and their sum is rounded to odd before
 * the bf16 step).  Encodings: a bf16
 * output holds that bf16 value; an e4m3 output holds the OCP e4m3 code of
 * value / scale (IEEE fp32 division, magnitudes above 448 saturate to 448,
 * nearest even), with q_scale for q_out and kv_scale for the cache (the
 * scaled-quantisation convention the page's tests check, with non-unit scales).
 *
 *   ql_nope       bf16 [T, H, 512], element (t,h,d) at ql_nope[t*ql_stride_t + h*ql_stride_h + d];
 *                 strided (non-packed) input is read correctly.  q_pe bf16 [T, H, 64] likewise.
 *   kv_c, k_pe    bf16 [T, 512] and [T, 64] with row strides kvc_stride_t, kpe_stride_t.
 *                 Every row of these four inputs must be 16-byte aligned (pointer
 *                 16-byte aligned, strides multiples of 8 elements).
 *   positions     int64 [T]; values outside [0, max_pos) are clamped into it.
 *   cos_sin_cache fp32 [max_pos, 64] packed, 16-byte aligned.
 *   T, H          tokens and heads (H >= 1; T == 0 is a no-op).
 *   q_out         [T, H, 576] packed, 16-byte aligned: bf16 (q_out_dtype 0) or e4m3 codes (1).
 *   slot_mapping  int64 [T]: the flat cache slot of token t's row; a slot outside
 *                 [0, num_blocks*block_size) writes nothing (e.g. -1 for padding tokens).
 *   kv_cache      [num_blocks, block_size, 576] packed, 16-byte aligned, in kv_dtype
 *                 (SMLA_KV_BF16 / SMLA_KV_FP8_E4M3): the pool sparse_mla_fwd reads.
 *   q_scale, kv_scale  positive finite; used only for e4m3 outputs.
 * Two tokens that map to one slot race (one of them wins).  Errors as for
 * sparse_mla_fwd: checked before any launch, nothing written on error.
 */
smla_status_t sparse_mla_rope_concat_cache(const void* ql_nope, int64_t ql_stride_t, int64_t ql_stride_h,
                                           const void* q_pe, int64_t qpe_stride_t, int64_t qpe_stride_h,
                                           const void* kv_c, int64_t kvc_stride_t,
                                           const void* k_pe, int64_t kpe_stride_t,
                                           const int64_t* positions, const float* cos_sin_cache,
                                           int64_t max_pos, int32_t is_neox, int64_t T, int64_t H,
                                           void* q_out, int32_t q_out_dtype, float q_scale,
                                           const int64_t* slot_mapping, void* kv_cache, int32_t kv_dtype,
                                           int64_t num_blocks, int64_t block_size, float kv_scale,
                                           void* stream);

/* Static description of a status code. */
const char* sparse_mla_status_string(smla_status_t status);

/* Detail of the last error returned on this thread ("" if none). */
const char* sparse_mla_last_error(void);

/* SMLA_ABI_VERSION of the built library. */
int32_t sparse_mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_MLA_H */
