/*
 * sparse_mla_oracle.c -- plain fp64 CPU oracle for the sparse MLA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see sparse_mla_oracle.h).  Deliberately slow and
 * direct: one (token, head) at a time, every element decoded from its bits,
 * every sum in fp64, softmax written out as its definition.  No blocking, no
 * online softmax, no fusion.  OpenMP only distributes independent
 * (token, head) pairs over threads.
 */
#include "sparse_mla_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element codecs --------------------------------------------------- */

double oracle_bf16_value(uint16_t bits) {
  /* bf16 is the upper half of an IEEE binary32 word. */
  uint32_t word = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

double oracle_e4m3_value(uint8_t code) {
  /* OCP 8-bit floating point, E4M3: 1 sign bit, 4 exponent bits (bias 7),
   * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111
   * is NaN; there is no infinity.  Largest finite magnitude: 1.75 * 2^8. */
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);              /* m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

uint8_t oracle_e4m3_encode_rne_sat(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;                 /* saturate at 448 */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: uniform quantum 2^-9; a result of 8 quanta is the
     * smallest normal, whose code (exponent 1, mantissa 0) is also 8. */
    double n = nearbyint(a * 512.0);                  /* ties to even */
    return sign | (uint8_t)n;
  }
  int e2;
  frexp(a, &e2);                     /* a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;                    /* unbiased exponent, -6..8 */
  double n = nearbyint(ldexp(a, 3 - E));   /* significand * 8, in [8, 16] */
  if (n == 16.0) { n = 8.0; E += 1; }
  return sign | (uint8_t)(((E + 7) << 3) | ((int)n - 8));
}

/* ---- per-tile q quantisation (FP8 dots) -------------------------------- */

static float bf16_float(uint16_t bits) { return (float)oracle_bf16_value(bits); }

void oracle_quantize_q_tiles(const uint16_t* q, int64_t T, int64_t H, int64_t Dqk,
                             int64_t q_stride_t, int64_t q_stride_h,
                             uint8_t* codes, float* scales) {
  const int64_t G = (H + 63) / 64;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t g = 0; g < G; ++g) {
      int64_t h0 = 64 * g, h1 = (64 * g + 64 < H) ? 64 * g + 64 : H;
      float amax = 0.0f;
      for (int64_t h = h0; h < h1; ++h)
        for (int64_t d = 0; d < Dqk; ++d) {
          float v = fabsf(bf16_float(q[t * q_stride_t + h * q_stride_h + d]));
          if (v > amax) amax = v;
        }
      float s_q = (amax > 0.0f) ? amax / 448.0f : 1.0f;   /* fp32 division */
      scales[t * G + g] = s_q;
      for (int64_t h = h0; h < h1; ++h)
        for (int64_t d = 0; d < Dqk; ++d) {
          float v = bf16_float(q[t * q_stride_t + h * q_stride_h + d]);
          float x = v / s_q;                                /* fp32 division */
          codes[(t * H + h) * Dqk + d] = oracle_e4m3_encode_rne_sat(x);
        }
    }
  }
}

/* ---- the forward pass --------------------------------------------------- */

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_sparse_mla_fwd(const uint16_t* q, int64_t T, int64_t H, int64_t Dqk,
                          int64_t q_stride_t, int64_t q_stride_h,
                          const void* kv, int kv_dtype, int64_t N,
                          const int32_t* idx, int64_t K, int64_t idx_stride_t,
                          double sm_scale, double kv_scale, int q_mode, double q_scale,
                          const double* sinks, double* out, double* lse) {
  const int64_t DV = 512;
  if (T < 0 || H <= 0 || Dqk < DV || K < 0 || N < 0) return 1;
  if (kv_dtype != ORACLE_KV_BF16 && kv_dtype != ORACLE_KV_FP8_E4M3) return 2;
  if (q_mode != ORACLE_Q_EXACT && q_mode != ORACLE_Q_TILE_FP8 && q_mode != ORACLE_Q_GIVEN_FP8) return 3;
  if (q_mode == ORACLE_Q_GIVEN_FP8 && kv_dtype != ORACLE_KV_FP8_E4M3) return 3;
  if (T == 0) return 0;

  /* Per-tile quantised q, only for FP8 KV with FP8 dots. */
  const int use_q8 = (kv_dtype == ORACLE_KV_FP8_E4M3 && q_mode == ORACLE_Q_TILE_FP8);
  const int64_t G = (H + 63) / 64;
  uint8_t* qcodes = NULL;
  float* qscales = NULL;
  if (use_q8) {
    qcodes = (uint8_t*)malloc((size_t)(T * H * Dqk));
    qscales = (float*)malloc((size_t)(T * G) * sizeof(float));
    if (!qcodes || !qscales) { free(qcodes); free(qscales); return 4; }
    oracle_quantize_q_tiles(q, T, H, Dqk, q_stride_t, q_stride_h, qcodes, qscales);
  }

  /* dec(): element d of slot r, as an exact fp64 value. */
  const uint16_t* kv16 = (const uint16_t*)kv;
  const uint8_t* kv8 = (const uint8_t*)kv;
  double e4m3_table[256];
  for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_value((uint8_t)c);

  int failed = 0;
#pragma omp parallel
  {
    double* qhat = (double*)malloc((size_t)Dqk * sizeof(double));
    double* s = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    int64_t* rows = (int64_t*)malloc((size_t)(K > 0 ? K : 1) * sizeof(int64_t));
    if (!qhat || !s || !rows) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for collapse(2) schedule(dynamic)
      for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
          double* o = out + (t * H + h) * DV;
          /* 1. the valid entries of this token's list, in list order */
          int64_t n = 0;
          for (int64_t k = 0; k < K; ++k) {
            int64_t r = idx[t * idx_stride_t + k];
            if (r >= 0 && r < N) rows[n++] = r;
          }
          /* the head's sink logit (-inf = none): a key with a zero value row */
          const double sig = sinks ? sinks[h] : -INFINITY;
          if (n == 0) {
            for (int64_t d = 0; d < DV; ++d) o[d] = 0.0;
            lse[t * H + h] = sig;
            continue;
          }
          /* 2. the query vector as the dots see it */
          for (int64_t d = 0; d < Dqk; ++d) {
            if (q_mode == ORACLE_Q_GIVEN_FP8)
              qhat[d] = q_scale * e4m3_table[((const uint8_t*)q)[t * q_stride_t + h * q_stride_h + d]];
            else if (use_q8)
              qhat[d] = (double)qscales[t * G + h / 64] *
                        e4m3_table[qcodes[(t * H + h) * Dqk + d]];
            else
              qhat[d] = oracle_bf16_value(q[t * q_stride_t + h * q_stride_h + d]);
          }
          /* 3. scores */
          for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t d = 0; d < Dqk; ++d) {
              double kd = (kv_dtype == ORACLE_KV_BF16)
                              ? oracle_bf16_value(kv16[rows[j] * Dqk + d])
                              : e4m3_table[kv8[rows[j] * Dqk + d]];
              acc += qhat[d] * (kv_scale * kd);
            }
            s[j] = sm_scale * acc;
          }
          /* 4. softmax normaliser, natural log, over the entries and the sink */
          double m = s[0];
          for (int64_t j = 1; j < n; ++j) if (s[j] > m) m = s[j];
          if (sig > m) m = sig;
          double l = exp(sig - m);
          for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
          double L = m + log(l);
          lse[t * H + h] = L;
          /* 5. weighted sum of V = the first 512 columns of the same rows */
          for (int64_t d = 0; d < DV; ++d) o[d] = 0.0;
          for (int64_t j = 0; j < n; ++j) {
            double w = exp(s[j] - L);
            for (int64_t d = 0; d < DV; ++d) {
              double vd = (kv_dtype == ORACLE_KV_BF16)
                              ? oracle_bf16_value(kv16[rows[j] * Dqk + d])
                              : e4m3_table[kv8[rows[j] * Dqk + d]];
              o[d] += w * (kv_scale * vd);
            }
          }
        }
      }
    }
    free(qhat);
    free(s);
    free(rows);
  }
  free(qcodes);
  free(qscales);
  return failed ? 5 : 0;
}

/* ---- the fused q-RoPE / q-concat / KV-concat / cache write --------------- */

/* Nearest bf16 to a real number v (given exactly as a double), ties to even:
 * bf16 keeps 8 significant bits with the binary32 exponent range, so the
 * spacing near |v| in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below the
 * smallest normal 2^-126. */
uint16_t oracle_bf16_round(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);   /* ties to even */
  if (r > 3.3895313892515355e38) return sign | 0x7F80;  /* beyond the largest bf16: inf */
  float f = (float)r;                                   /* exact: r is a bf16 number */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  return sign | (uint16_t)((w >> 16) & 0x7FFF);
}

/* Nearest bf16 to the exact sum a + b of two doubles, ties to even.  The sum
 * is first split exactly into hi + lo (Knuth's TwoSum: hi = the double nearest
 * to a + b, lo the exact remainder, |lo| <= half an ulp of hi).  In units of
 * the bf16 spacing q at |hi|, hi / q = n + f with n an integer and f in [0, 1)
 * (both exact); the exact sum is above the midpoint between n q and (n + 1) q
 * exactly when f - 1/2 + lo / q > 0.  A non-zero f - 1/2 is a multiple of an
 * ulp of hi / q, larger than |lo / q|, so it decides alone; at f = 1/2 the sign
 * of lo decides, and only lo = 0 is a tie.  Rounding hi alone would round
 * twice (fp64, then bf16) and can land on the wrong side of a midpoint. */
static uint16_t bf16_round_sum(double a, double b) {
  const double hi = a + b;
  const double bb = hi - a;
  const double lo = (a - (hi - bb)) + (b - bb);
  if (isnan(hi) || isinf(hi) || lo == 0.0) return oracle_bf16_round(hi);
  const uint16_t sign = signbit(hi) ? 0x8000 : 0x0000;
  const double ahi = fabs(hi), alo = signbit(hi) ? -lo : lo;   /* |a + b| = ahi + alo */
  int e;
  frexp(ahi, &e);
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  const double h = ldexp(ahi, -qexp);
  const double n = floor(h);
  const double f = h - n;
  int up;
  if (f != 0.5) up = f > 0.5;
  else up = alo > 0.0;
  const double r = ldexp(n + (up ? 1.0 : 0.0), qexp);
  return sign | (oracle_bf16_round(r) & 0x7FFF);   /* r is a bf16 number (or past the largest) */
}

/* RoPE of one 64-column bf16 row at one position, as bf16 bits.  Pairs are
 * (i, i + 32) for the rotate-halves ("neox") form and (2i, 2i + 1) for the
 * interleaved form; pair i turns by the angle whose cosine / sine are
 * cs[i] / cs[32 + i]: (x, y) -> (x cos - y sin, y cos + x sin), each output
 * the exact value rounded once to bf16 (the products of a bf16 and an fp32
 * number are exact in fp64, the sum is taken exactly by bf16_round_sum). */
static void rope_row(const uint16_t* x, const float* cs, int is_neox, uint16_t* out) {
  for (int i = 0; i < 32; ++i) {
    const int ix = is_neox ? i : 2 * i;
    const int iy = is_neox ? i + 32 : 2 * i + 1;
    const double c = cs[i], s = cs[32 + i];
    const double xv = oracle_bf16_value(x[ix]), yv = oracle_bf16_value(x[iy]);
    out[ix] = bf16_round_sum(xv * c, -(yv * s));
    out[iy] = bf16_round_sum(yv * c, xv * s);
  }
}

/* one output element: bf16 bits as they are, or the e4m3 code of value / scale
 * (the quotient rounded to binary32 first) */
static void put(void* base, int64_t i, int fp8, double scale, uint16_t bits) {
  if (fp8) {
    float qf = (float)(oracle_bf16_value(bits) / scale);
    ((uint8_t*)base)[i] = oracle_e4m3_encode_rne_sat(qf);
  } else {
    ((uint16_t*)base)[i] = bits;
  }
}

int oracle_rope_concat_cache(const uint16_t* ql_nope, int64_t ql_st, int64_t ql_sh,
                             const uint16_t* q_pe, int64_t qpe_st, int64_t qpe_sh,
                             const uint16_t* kv_c, int64_t kvc_st,
                             const uint16_t* k_pe, int64_t kpe_st,
                             const int64_t* positions, const float* cos_sin, int64_t max_pos,
                             int is_neox, int64_t T, int64_t H,
                             void* q_out, int q_fp8, double q_scale,
                             const int64_t* slot_mapping, void* kv_cache, int kv_fp8, int64_t N,
                             double kv_scale) {
  if (T < 0 || H <= 0 || max_pos <= 0 || N < 0) return 1;
  uint16_t rot[64];
  for (int64_t t = 0; t < T; ++t) {
    int64_t p = positions[t];
    if (p < 0) p = 0;
    if (p >= max_pos) p = max_pos - 1;
    const float* cs = cos_sin + p * 64;
    for (int64_t h = 0; h < H; ++h) {
      const int64_t o = (t * H + h) * 576;
      for (int d = 0; d < 512; ++d) put(q_out, o + d, q_fp8, q_scale, ql_nope[t * ql_st + h * ql_sh + d]);
      rope_row(q_pe + t * qpe_st + h * qpe_sh, cs, is_neox, rot);
      for (int d = 0; d < 64; ++d) put(q_out, o + 512 + d, q_fp8, q_scale, rot[d]);
    }
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= N) continue;
    for (int d = 0; d < 512; ++d) put(kv_cache, slot * 576 + d, kv_fp8, kv_scale, kv_c[t * kvc_st + d]);
    rope_row(k_pe + t * kpe_st, cs, is_neox, rot);
    for (int d = 0; d < 64; ++d) put(kv_cache, slot * 576 + 512 + d, kv_fp8, kv_scale, rot[d]);
  }
  return 0;
}
