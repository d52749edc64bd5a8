/*
 * sparse_mla_oracle.h -- plain fp64 CPU oracle for the sparse MLA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; the two meet only on the bytes of the seeded synthetic inputs.
 *
 * What it computes (sources: vLLM PR "[ROCm][Perf][GLM-5.3-Flash] Enable AITER
 * sparse MLA on gfx942, including FP8 KV", Overview and Details; vLLM PR
 * "[ROCm][DSv4.1][Perf] Route gfx942 sparse MLA prefill to AITER
 * pa_prefill_sparse", What changed ("One KV pool"); vLLM PR "[ROCm][MLA][Perf]
 * Fuse decode QK-RoPE + Q-concat + KV-concat + KV-cache write for sparse MLA",
 * Test plan (cache row = concat(kv_c, RoPE(k_pe)), so V is the kv_c part)):
 *
 *   for every query token t and head h, with J = the valid entries of t's
 *   top-k list (0 <= idx < N; everything else is padding):
 *     s_j   = sm_scale * sum_d qhat[t,h,d] * kv_scale * dec(kv[idx_j, d])   d < Dqk
 *     lse   = log(sum_j exp(s_j))                          (natural log)
 *     out   = sum_j exp(s_j - lse) * kv_scale * dec(kv[idx_j, 0:512])
 *   J empty -> out = 0, lse = -inf.
 *
 *   With attention sinks (same first page, Details, Limitations: sinks are
 *   passed through to the kernel; read here as the usual definition, a
 *   per-head logit sigma_h that joins the normaliser only, as a key whose
 *   value row is zero):
 *     lse   = log(exp(sigma_h) + sum_j exp(s_j)),  out as above with this lse;
 *     J empty -> out = 0, lse = sigma_h.
 *
 *   qhat is q itself (exact) for bf16 KV and in mode ORACLE_Q_EXACT; for fp8
 *   KV in mode ORACLE_Q_TILE_FP8 it is q quantised per tile to OCP e4m3 (the
 *   "FP8 dots" path, where the kernel quantises q per tile):
 *     tile   = heads [64g, min(64g+64, H)) of ONE token, all Dqk columns
 *     amax   = max |q| over the tile (fp32)
 *     s_q    = amax / 448 (fp32 division), or 1 when amax == 0
 *     code_d = e4m3_rne_sat(q_d / s_q)   (fp32 division, then round to the
 *                                         nearest e4m3 value, ties to even,
 *                                         magnitudes above 448 clamp to 448)
 *     qhat_d = s_q * dec(code_d)
 *
 *   In mode ORACLE_Q_GIVEN_FP8 (fp8 KV only) q is already quantised (same first
 *   page, Details: gfx950 keeps the pre-quantised q): the q pointer holds OCP
 *   e4m3 codes, one byte per element with strides in bytes, and
 *   qhat_d = q_scale * dec(code_d) with one per-tensor q_scale.
 *
 * Parity is unpinned for nothing here: every function is pinned by the CPU
 * tests (closed forms, dense attention, library codecs).
 */
#ifndef SPARSE_MLA_ORACLE_H
#define SPARSE_MLA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_KV_BF16 = 0, ORACLE_KV_FP8_E4M3 = 1 };
enum { ORACLE_Q_EXACT = 0, ORACLE_Q_TILE_FP8 = 1, ORACLE_Q_GIVEN_FP8 = 2 };

/* bf16 bit pattern -> value (exact). */
double oracle_bf16_value(uint16_t bits);

/* OCP 8-bit float E4M3 ("e4m3fn") code -> value (exact); NaN for 0x7f/0xff. */
double oracle_e4m3_value(uint8_t code);

/* fp32 value -> nearest OCP E4M3 code, ties to even, |x| > 448 -> +-448.
 * NaN input -> 0x7f. */
uint8_t oracle_e4m3_encode_rne_sat(float x);

/* Per-tile fp8 quantisation of q (see header comment).
 * q: bf16 bits, element (t,h,d) at q[t*q_stride_t + h*q_stride_h + d].
 * codes: uint8 [T, H, Dqk] contiguous.  scales: fp32 [T, ceil(H/64)]. */
void oracle_quantize_q_tiles(const uint16_t* q, int64_t T, int64_t H, int64_t Dqk,
                             int64_t q_stride_t, int64_t q_stride_h,
                             uint8_t* codes, float* scales);

/* The forward pass, fp64 throughout.
 * kv: [N, Dqk] rows of bf16 bits (kv_dtype 0) or e4m3 codes (kv_dtype 1).
 * idx: int32, entry (t,k) at idx[t*idx_stride_t + k].
 * sinks: NULL, or fp64 [H] per-head sink logits (-inf = none for that head); a
 * sink joins the softmax normaliser as a key whose value row is zero.
 * out: fp64 [T, H, 512] contiguous; lse: fp64 [T, H].
 * Returns 0 on success, nonzero on bad arguments. */
int oracle_sparse_mla_fwd(const uint16_t* q, int64_t T, int64_t H, int64_t Dqk,
                          int64_t q_stride_t, int64_t q_stride_h,
                          const void* kv, int kv_dtype, int64_t N,
                          const int32_t* idx, int64_t K, int64_t idx_stride_t,
                          double sm_scale, double kv_scale, int q_mode, double q_scale,
                          const double* sinks, double* out, double* lse);

/* Nearest bf16 (bits) to a real number given exactly as a double, ties to even. */
uint16_t oracle_bf16_round(double v);

/* The fused q-RoPE / q-concat / KV-concat / cache write, element by element
 * (vLLM PR "[ROCm][MLA][Perf] Fuse decode QK-RoPE + Q-concat + KV-concat +
 * KV-cache write for sparse MLA", Summary and Test plan):
 *   q_out[t,h] = concat(ql_nope[t,h], RoPE(q_pe[t,h], positions[t]))   [576]
 *   cache row slot_mapping[t] = concat(kv_c[t], RoPE(k_pe[t], positions[t]))
 * RoPE: 32 pairs, (i, i+32) when is_neox else (2i, 2i+1); pair i turns by the
 * angle with cosine cos_sin[p*64 + i] and sine cos_sin[p*64 + 32 + i]; each
 * result is the exact x cos - y sin / y cos + x sin rounded once to bf16.
 * Positions are clamped into [0, max_pos); slots outside [0, N) write nothing.
 * Outputs: bf16 bits, or (q_fp8 / kv_fp8) the e4m3 code of value / scale with
 * the quotient rounded to binary32, saturated at 448, nearest even.
 * Strides in elements.  Returns 0, or nonzero on bad sizes. */
int oracle_rope_concat_cache(const uint16_t* ql_nope, int64_t ql_st, int64_t ql_sh,
                             const uint16_t* q_pe, int64_t qpe_st, int64_t qpe_sh,
                             const uint16_t* kv_c, int64_t kvc_st,
                             const uint16_t* k_pe, int64_t kpe_st,
                             const int64_t* positions, const float* cos_sin, int64_t max_pos,
                             int is_neox, int64_t T, int64_t H,
                             void* q_out, int q_fp8, double q_scale,
                             const int64_t* slot_mapping, void* kv_cache, int kv_fp8, int64_t N,
                             double kv_scale);

/* Number of OpenMP threads the oracle will use (1 when built without it). */
int oracle_num_threads(void);
/* threads the following calls use (OpenMP; the default is the host's count) */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
