// smla_rope_cache.hip -- the step in front of the forward pass, fused: RoPE on the
// 64 rope columns of q and of the new KV row, the q concat and the KV-cache
// write (vLLM PR "[ROCm][MLA][Perf] Fuse decode QK-RoPE + Q-concat + KV-concat +
// KV-cache write for sparse MLA", Summary and Test plan).
//
// Every token has H q rows (576 outputs each) and one cache row (576
// outputs): R = T (H + 1) rows in all, row r belonging to token r / (H + 1).
// The work is split by wave, so no wave mixes the two kinds of chunk:
//   latent waves copy (or quantise) the 512 latent columns of kLatentRows rows,
//     lane l taking 16-byte chunk l of each (that many 1 KB loads in flight per
//     wave, each contiguous across the lanes);
//   rope waves rotate the 64 rope columns of eight rows, eight lanes per row.
// On large calls consecutive waves come in groups of two latent waves and one
// rope wave (the rows of the two kinds in the same ratio), so that the
// arithmetic of the rope waves runs beside the latent waves' streaming on every
// CU instead of after it; calls whose waves the device holds at once keep all
// latent waves first (measured on MI355X: interleaving costs up to 9 % at
// 8K - 33K rows and saves 6 - 8 % from 70K rows).  The rotation:
//   (x, y) -> (x cos - y sin, y cos + x sin)
// with the pairs (i, i + 32) (rotate-halves, "neox") or (2i, 2i + 1)
// (interleaved).  Each output is the exact value rounded once to bf16: both
// products are exact in fp64 for a bf16 times an fp32, their sum is rounded
// to fp64 with round-to-odd (the exact error of the nearest-rounded sum, from
// TwoSum, moves an even result one step toward the exact value), and the
// round-to-odd fp64 value, with 45 bits more than bf16, rounds to nearest even
// as the exact value would.  The bf16 step works on the fp64 bits; a chunk
// with an output outside the range of normal bf16 numbers (zero, subnormal,
// non-finite) takes a two-step conversion instead (to fp32 with round-to-odd,
// then to bf16).  e4m3 outputs encode value / scale (the
// correctly rounded fp32 quotient, saturated to +-448, round to nearest even)
// of the bf16 value.
#include <hip/hip_runtime.h>

#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kRopeCols = 64;
constexpr int kLatentRows = 4;   // rows per latent wave
constexpr uint32_t kGroup = 8 / kLatentRows + 1;   // waves per group: latent ones, then one rope wave
constexpr int64_t kInterleaveRows = 49152;          // rows from which the wave kinds interleave
static_assert(8 % kLatentRows == 0, "a group covers the eight rows of its rope wave");

// a + b for two fp64 values whose exact sum is wanted, rounded to odd: the
// nearest sum s and its exact error (Knuth's TwoSum, six additions; a and b
// are exact products, so contracting one of them into an addition rounds the
// same way); a non-zero error on
// an s with an even last bit moves s one ulp toward the exact sum (up in
// magnitude when the error has s's sign), which is the round-to-odd result.
__device__ __forceinline__ double add_round_odd(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double err = (a - (s - bb)) + (b - bb);
  uint64_t u = (uint64_t)__double_as_longlong(s);
  if (err != 0.0 && (u & 1u) == 0u) u += ((err > 0.0) == (s > 0.0)) ? 1u : ~(uint64_t)0;
  return __longlong_as_double((long long)u);
}

// fp64 -> bf16 bits, round to nearest even, in two steps that round once: to
// fp32 toward zero with the sticky "inexact" bit folded into the last place
// (round to odd), then fp32 -> bf16 to nearest even.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  float f = __double2float_rz(d);
  uint32_t b = __float_as_uint(f);
  if ((double)f != d) b |= 1u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// The same rounding with integer operations on the fp64 bits, for
// 2^-126 <= |d| < 2^128: bf16 keeps the 7 mantissa bits 45..51 of d, bit 44 is
// the half and bits 0..43 are discarded.  The low word is folded into bit 0 of
// the high word as a sticky bit (round to odd, which cannot move the high word
// across the half), then adding 2^12 - 1 and the kept last bit rounds to
// nearest even (a carry out of the mantissa steps the exponent, to infinity
// past 2^128).  Then the exponent is rebased from fp64's 1023 to bf16's 127.
// `ok` is cleared when d is out of that range (the result is then not used).
__device__ __forceinline__ uint32_t f64_to_bf16_rne_normal(double d, bool& ok) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint32_t hi = (uint32_t)(u >> 32) | ((uint32_t)u != 0u ? 1u : 0u);
  const uint32_t e = (hi >> 20) & 0x7ffu;
  ok = ok && e - (1023u - 126u) <= 127u + 126u;
  const uint32_t t = hi + 0xfffu + ((hi >> 13) & 1u);
  return ((t >> 16) & 0x8000u) | (((t >> 13) & 0x3ffffu) - ((1023u - 127u) << 7));
}

// v / s rounded to nearest fp32 without a division per value, given
// r = RN(1 / s) with 2^-64 <= s <= 2^64: q0 = RN(v r) lies within an ulp of
// the quotient, so the residual v - q0 s is exact in one fma and one more fma
// q0 + residual * r rounds to RN(v / s) (Markstein's correction step), while
// no intermediate underflows -- which holds wherever the e4m3 code depends on
// the exact quotient (|v / s| >= 2^-11, so |v| >= 2^-75).  Smaller quotients
// only need their sign and to stay below 2^-10 (code +-0), which the
// copysign keeps for zeros too; when q0 is past 1024 (or infinite) it is used
// as it is, since it saturates like the quotient.
__device__ __forceinline__ float quotient_rn(float v, float s, float r) {
  const float q0 = v * r;
  const float e = __builtin_fmaf(-q0, s, v);
  const float q1 = __builtin_fmaf(e, r, q0);
  return __builtin_copysignf(fabsf(q0) > 1024.0f ? q0 : q1, v);
}

// eight outputs (as fp32 values of bf16 numbers) -> their encoding at dst
template <bool E4M3>
__device__ __forceinline__ void store8(uint8_t* dst, const float (&v)[8], float scale) {
  if constexpr (!E4M3) {
    *reinterpret_cast<u32x4*>(dst) =
        u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
  } else {
    float y[8];
    if (scale >= 0x1p-64f && scale <= 0x1p64f) {   // uniform
      const float r = 1.0f / scale;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = quotient_rn(v[i], scale, r);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = v[i] / scale;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(y[i], -kE4m3Max), kE4m3Max);
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{f32x4_to_e4m3x4(y[0], y[1], y[2], y[3]), f32x4_to_e4m3x4(y[4], y[5], y[6], y[7])};
  }
}

__device__ __forceinline__ void unpack8(const u32x4& w, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

// chunk j (rope columns 8j .. 8j+7) of RoPE(x) for one 64-column bf16 row x
template <bool NEOX>
__device__ __forceinline__ void rope8(const uint16_t* x, const float* cs, int j, float (&v)[8]) {
  float own[8];
  double d[8];
  unpack8(*reinterpret_cast<const u32x4*>(x + 8 * j), own);
  if constexpr (NEOX) {
    // column i pairs with i ^ 32; both halves use frequency i mod 32
    float other[8];
    unpack8(*reinterpret_cast<const u32x4*>(x + 8 * (j ^ 4)), other);
    const int f0 = 8 * (j & 3);
    const bool first = j < 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double c = cs[f0 + i], s = cs[32 + f0 + i];
      const double a = own[i], b = other[i];
      d[i] = add_round_odd(a * c, first ? -(b * s) : b * s);
    }
  } else {
    // pairs (2m, 2m + 1), frequency m
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * j + i;
      const double c = cs[m], s = cs[32 + m];
      const double a = own[2 * i], b = own[2 * i + 1];
      d[2 * i] = add_round_odd(a * c, -(b * s));
      d[2 * i + 1] = add_round_odd(b * c, a * s);
    }
  }
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(f64_to_bf16_rne_normal(d[i], ok) << 16);
  if (__builtin_expect(!ok, 0)) {
    // a zero, subnormal or non-finite output somewhere in the chunk
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(f64_to_bf16_rne(d[i]) << 16);
  }
}

// destination of output column 8k of row r, or null when the row is a cache
// row whose slot is out of range
template <bool Q8, bool KV8>
__device__ __forceinline__ uint8_t* row_dst(const RopeCacheParams& p, int t, int h, int k) {
  if (h < p.H) return p.q_out + (((int64_t)t * p.H + h) * (kDV + kRopeCols) + 8 * k) * (Q8 ? 1 : 2);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.N) return nullptr;
  return p.kv_cache + (slot * (kDV + kRopeCols) + 8 * k) * (KV8 ? 1 : 2);
}

template <bool NEOX, bool Q8, bool KV8>
__global__ __launch_bounds__(kThreads) void smla_rope_cache_kernel(RopeCacheParams p, uint32_t latent_waves, bool interleave) {
  const uint32_t g = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  // latent wave w, or rope wave k
  uint32_t w = g, k = g - latent_waves;
  bool latent = g < latent_waves;
  if (interleave) {
    k = g / kGroup;
    const uint32_t m = g - k * kGroup;
    latent = m + 1 < kGroup;
    w = (kGroup - 1) * k + m;
  }
  const int lane = threadIdx.x & 63;
  const uint32_t rows = (uint32_t)p.H + 1;
  const uint32_t R = (uint32_t)p.T * rows;
  if (latent) {
    if (w >= latent_waves) return;
    // ---- latent columns of rows LW w .. LW w + LW - 1, lane = 16-byte chunk
    constexpr int LW = kLatentRows;
    float v[LW][8];
    int tt[LW], hh[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const uint32_t r = min(LW * w + i, R - 1);   // clamped; rows past R are not stored
      tt[i] = (int)(r / rows);
      hh[i] = (int)(r - (uint32_t)tt[i] * rows);
      const uint16_t* src = (hh[i] < p.H) ? p.ql_nope + tt[i] * p.ql_st + hh[i] * p.ql_sh
                                          : p.kv_c + tt[i] * p.kvc_st;
      unpack8(*reinterpret_cast<const u32x4*>(src + 8 * lane), v[i]);
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      if (LW * w + i >= R) break;
      if (hh[i] < p.H) {
        store8<Q8>(row_dst<Q8, KV8>(p, tt[i], hh[i], lane), v[i], p.q_scale);
      } else {
        uint8_t* d = row_dst<Q8, KV8>(p, tt[i], hh[i], lane);
        if (d) store8<KV8>(d, v[i], p.kv_scale);
      }
    }
  } else {
    // ---- rope columns of rows 8w' .. 8w' + 7, eight lanes per row
    const uint32_t r = k * 8 + (lane >> 3);   // rope wave k
    if (r >= R) return;
    const int j = lane & 7;
    const int t = (int)(r / rows);
    const int h = (int)(r - (uint32_t)t * rows);
    const int64_t pos = min(max(p.positions[t], (int64_t)0), p.max_pos - 1);
    const float* cs = p.cos_sin + pos * kRopeCols;
    float v[8];
    if (h < p.H) {
      rope8<NEOX>(p.q_pe + t * p.qpe_st + h * p.qpe_sh, cs, j, v);
      store8<Q8>(row_dst<Q8, KV8>(p, t, h, kDV / 8 + j), v, p.q_scale);
    } else {
      uint8_t* d = row_dst<Q8, KV8>(p, t, h, kDV / 8 + j);
      if (d == nullptr) return;
      rope8<NEOX>(p.k_pe + t * p.kpe_st, cs, j, v);
      store8<KV8>(d, v, p.kv_scale);
    }
  }
}

template <bool NEOX, bool Q8>
hipError_t launch_rc2(const RopeCacheParams& p, bool kv8, hipStream_t stream) {
  const int64_t R = (int64_t)p.T * (p.H + 1);
  const uint32_t latent_waves = (uint32_t)((R + kLatentRows - 1) / kLatentRows);
  const bool interleave = R >= kInterleaveRows;
  const int64_t waves = interleave ? kGroup * ((R + 7) / 8) : latent_waves + (R + 7) / 8;
  const dim3 gd((unsigned)((waves + 3) / 4)), bd(kThreads);
  if (kv8)
    hipLaunchKernelGGL((smla_rope_cache_kernel<NEOX, Q8, true>), gd, bd, 0, stream, p, latent_waves, interleave);
  else
    hipLaunchKernelGGL((smla_rope_cache_kernel<NEOX, Q8, false>), gd, bd, 0, stream, p, latent_waves, interleave);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_cache(const RopeCacheParams& p, bool neox, bool q8, bool kv8, hipStream_t stream) {
  if (neox) return q8 ? launch_rc2<true, true>(p, kv8, stream) : launch_rc2<true, false>(p, kv8, stream);
  return q8 ? launch_rc2<false, true>(p, kv8, stream) : launch_rc2<false, false>(p, kv8, stream);
}

}  // namespace smla
