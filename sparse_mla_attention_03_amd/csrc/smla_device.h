// smla_device.h -- gfx950 device helpers for libsparsemla: vector types, MFMA
// wrappers, bf16 / OCP-e4m3 conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kE4m3Max = 448.0f;

// ---- MFMA ------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D[m][n] += sum_k A[m][k] B[k][n]; lane l holds
// A row m = l%16, B column n = l%16, 8 k-values each (k-slot l/16), and the
// result D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: as above with 4 k-values per lane (k-slot l/16).
__device__ __forceinline__ f32x4 mfma_bf16_k16(const u32x2& a, const u32x2& b, const f32x4& c) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                   __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x128_f8f6f4 with both operands OCP e4m3 (format code 0):
// same lane roles as above, 32 fp8 k-values per lane.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---- conversions -------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// four OCP e4m3 codes (one dword) -> four bf16 (exact: every e4m3 value is a bf16)
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t codes) {
  // v_cvt_scalef32_pk_bf16_fp8 with scale 1
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// four fp32 -> four OCP e4m3 codes, round to nearest even (v_cvt_pk_fp8_f32).
// Callers keep |x| <= 448 * (1 + 2^-22), which rounds to at most 448.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// low / high bf16 halves of two words -> one word (a's half low, b's half high),
// one v_perm_b32 each: bytes 0-3 select from a, 4-7 from b
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- buffer loads ---------------------------------------------------------------
// Raw buffer: byte offset voffset from the base; offsets at or past
// num_records bytes read zero.
__device__ int raw_load_b32(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.i32");

constexpr int kBufferRsrcWord3 = 0x00020000;   // 32-bit untyped data format

// ---- wavefront reductions (64 lanes) ------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// max / sum over the four lanes l, l^16, l^32, l^48 (the k-slot groups),
// with the gfx950 lane swaps instead of LDS permutes: permlane32_swap(v, v)
// yields {v[l mod 32], v[l mod 32 + 32]} and permlane16_swap(v, v) the same
// for 16-lane rows, so each step pairs lane l with l^32, then with l^16.
__device__ __forceinline__ float xor32_op_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group4_max(float v) {
  v = xor32_op_max(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- per-tile q quantisation (fp8 dots) ---------------------------------------
// amax of |q| over heads [qh0, qh1) of one token, all D columns, by the whole
// workgroup (blockDim.x threads).  red must hold blockDim.x/64 floats of LDS.
template <int D>
__device__ float q_tile_amax(const uint16_t* __restrict__ qtok, int64_t q_sh, int qh0, int qh1,
                             float* red) {
  constexpr int CPR = D / 8;   // 16-byte chunks per head row
  const int n = (qh1 - qh0) * CPR;
  float m = 0.0f;
  // four independent loads per step (indices clamped, so no guard serialises them)
  for (int c0 = threadIdx.x; c0 < n; c0 += 4 * blockDim.x) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = min(c0 + j * (int)blockDim.x, n - 1);
      v[j] = *reinterpret_cast<const u32x4*>(qtok + (int64_t)(qh0 + c / CPR) * q_sh + (c % CPR) * 8);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[j][i])), fabsf(bf16_hi(v[j][i]))));
  }
  m = wave_max(m);
  const int nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// s_q = amax / 448 (IEEE fp32 division), 1 for an all-zero tile
__device__ __forceinline__ float q_scale_from_amax(float amax) {
  return amax > 0.0f ? amax / kE4m3Max : 1.0f;
}

// fp32 quotient x / s (s > 0) from r = RN(1/s): y = RN(x*r) refined once with
// the exact FMA residual x - y*s (Markstein's correction step), in place of
// the IEEE division sequence; copysign gives a zero x's quotient its sign.
// It equals RN(x / s) whenever the residual stays a normal number;
// q_tile_fast_div() gates it to tiles whose amax >= 2^-60, where every case in
// which it could differ has |x / s| < 2^-10, so both quotients round to the
// same signed-zero e4m3 code.  Checked exhaustively over all bf16 (amax, x)
// pairs on the CPU, and bit for bit against the oracle on the GPU.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float y = x * r;
  const float e = __builtin_fmaf(-y, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, y), x);
}

__device__ __forceinline__ bool q_tile_fast_div(float amax) { return amax >= 0x1p-60f; }

// 8 bf16 (one 16-byte chunk) / s_q -> 8 e4m3 codes (two dwords); r = 1/s_q.
// FAST selects the three-op quotient above, otherwise IEEE division.
template <bool FAST>
__device__ __forceinline__ float qdiv(float x, float s, float r) {
  if constexpr (FAST) return div_by_scale(x, s, r);
  else return x / s;
}
template <bool FAST>
__device__ __forceinline__ u32x2 quantize_chunk(const u32x4& v, float s_q, float r) {
  const uint32_t w0 = f32x4_to_e4m3x4(qdiv<FAST>(bf16_lo(v[0]), s_q, r), qdiv<FAST>(bf16_hi(v[0]), s_q, r),
                                      qdiv<FAST>(bf16_lo(v[1]), s_q, r), qdiv<FAST>(bf16_hi(v[1]), s_q, r));
  const uint32_t w1 = f32x4_to_e4m3x4(qdiv<FAST>(bf16_lo(v[2]), s_q, r), qdiv<FAST>(bf16_hi(v[2]), s_q, r),
                                      qdiv<FAST>(bf16_lo(v[3]), s_q, r), qdiv<FAST>(bf16_hi(v[3]), s_q, r));
  return u32x2{w0, w1};
}

}  // namespace smla
