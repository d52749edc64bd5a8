// smla_kernels.hip -- gfx950 kernels of libsparsemla.
//
// One workgroup (4 wavefronts) owns one unit of work: a query token t, a head
// group of HT heads (16, 32 or 64) and a split s, i.e. a contiguous range of
// t's top-k list.  It walks that range in tiles of 64 entries:
//
//   gather   every wave fetches 16 of the tile's rows with 16-byte loads (one
//            64-lane load covers a whole 1 KiB bf16 row) into registers, then
//            writes them to an LDS stage whose 16-byte chunks are rotated by
//            the row number (conflict-free column reads).  Invalid entries
//            (padding, out of range, past the split) read a zero row instead of
//            the pool.  Two LDS stages plus one tile in flight in registers.
//   QK^T     v_mfma_f32_16x16x32_bf16 (bf16 KV) or v_mfma_f32_16x16x128_f8f6f4
//            (e4m3 KV, q quantised per tile), rows x heads, fp32 accumulation.
//   softmax  online, in registers, log2 domain; each lane owns one head and 16
//            of the tile's rows, so the only cross-lane steps are a max over
//            four lanes per tile and the final sum.
//   PV       V = the first 512 columns of the same LDS rows, read 8 rows x 8
//            columns per lane and transposed in registers into the MFMA
//            operand; O^T[dim][head] accumulates in fp32.
//   epilogue S == 1: out = bf16(O * kv_scale / l), lse = ln(sum exp).  S > 1:
//            normalised fp32 partials + lse per split, merged by the combine
//            kernel (log-sum-exp weights).
//
// Waves of a head group split the work two ways: with WD = 4 / (HT/16) waves
// per 16-head tile, each wave computes QK for 64/WD rows (exchanged through
// LDS) and PV for 512/WD output columns.
#include <type_traits>

#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

// Stand-in for the rows of invalid top-k entries: all zero, never written.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[2048];

template <bool KV8, int DQK>
struct Geom {
  static constexpr int ELEM = KV8 ? 1 : 2;
  static constexpr int ROW = DQK * ELEM;           // bytes of a pool row
  static constexpr int MAIN = kDV * ELEM;          // bytes of its V part
  static constexpr int TAIL = (DQK - kDV) * ELEM;  // bytes of its RoPE part (0 if rope-free)
  static constexpr int MCH = MAIN / 16;            // 16-byte chunks in MAIN (64 or 32)
  static constexpr int TCH = TAIL / 16;            // ... in TAIL (8, 4 or 0)
  static constexpr int STAGE_MAIN = kBK * MAIN;
  static constexpr int STAGE = kBK * (MAIN + TAIL);
  static constexpr int NLD_MAIN = KV8 ? 8 : 16;    // 64-lane loads per wave per tile (16 rows)
  static constexpr int NLD_TAIL = (16 * TCH) / 64; // 2 (bf16/576), 1 (fp8/576), 0
  static constexpr int NLD = NLD_MAIN + NLD_TAIL;
  static constexpr int NKB = KV8 ? (DQK + 127) / 128 : DQK / 32;   // QK k-steps
};

// LDS byte offset of 16-byte chunk c of tile row r, main part / RoPE part.
template <class G>
__device__ __forceinline__ int lds_main(int r, int c) {
  return r * G::MAIN + 16 * ((c + r) & (G::MCH - 1));
}
template <class G>
__device__ __forceinline__ int lds_tail(int r, int c) {
  return G::STAGE_MAIN + r * G::TAIL + 16 * ((c + r) & (G::TCH - 1));
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 lds_read8(const uint8_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

template <bool KV8, int DQK, int HT>
__global__ __launch_bounds__(kThreads, 1) void smla_fwd_kernel(FwdParams p) {
  using G = Geom<KV8, DQK>;
  constexpr int WH = HT / 16;          // 16-head tiles per workgroup
  constexpr int WD = 4 / WH;           // waves per head tile
  constexpr int DPW = kDV / WD;        // output columns per wave
  constexpr int NSLOT = DPW / 128;     // 8-column chunks per lane (x16 lanes x8 = 128 cols)
  constexpr int NBLK = kBK / 16;       // 16-row blocks per tile
  constexpr int BPW = NBLK / WD;       // QK row blocks per wave
  constexpr int NSTAGE = 2;
  constexpr int SX = (WD > 1) ? WH * NBLK * 16 * 16 * 4 : 0;   // score exchange bytes
  constexpr int QLDS = KV8 ? HT * DQK : 0;                     // quantised q (prologue only)
  constexpr int RING = NSTAGE * G::STAGE;
  static_assert(QLDS <= RING, "q staging must fit in the ring");

  __shared__ __attribute__((aligned(16))) uint8_t smem[RING + SX];
  __shared__ uint32_t s_mask[NSTAGE][4];
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;
  const int ht = wave / WD;
  const int dp = wave % WD;

  // Workgroup -> (token, split, head group).  Consecutive workgroup ids go to
  // different XCDs; the head groups of one (token, split) are 8 ids apart so
  // they share an XCD (and its L2) for the rows they both gather.
  const int HG = p.H / HT;
  const int L = blockIdx.x;
  const int hg = (L >> 3) % HG;
  const int u = ((L >> 3) / HG) * 8 + (L & 7);
  if (u >= p.T * p.S) return;
  const int t = u / p.S;
  const int s = u - t * p.S;
  const int h0 = hg * HT;
  const int kbeg = s * p.rps;
  const int kend = min(kbeg + p.rps, p.K);
  const int ntiles = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

  const int head = h0 + ht * 16 + m16;
  const uint16_t* qtok = p.q + (int64_t)t * p.q_st;
  const uint16_t* qrow = qtok + (int64_t)head * p.q_sh;
  const int32_t* idx_t = p.idx + (int64_t)t * p.idx_st;

  // ---- q operand (B of QK^T): lane (m16 = head, g) holds 8 (bf16) or 32 (fp8)
  // columns per k-step; column d of the row maps to the same (k-step, g, slot)
  // in the K fragments below.
  u32x4 qf[KV8 ? 1 : G::NKB];
  i32x8 q8[KV8 ? G::NKB : 1];
  float c2;   // logit multiplier, log2 domain
  if constexpr (!KV8) {
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
      qf[kb] = *reinterpret_cast<const u32x4*>(qrow + kb * 32 + 8 * g);
    c2 = p.sm_scale * p.kv_scale * kLog2e;
  } else {
    // per-tile q quantisation: tile = heads [64*floor(h/64), +64) of token t
    const int qt0 = (h0 / 64) * 64;
    const int qt1 = min(qt0 + 64, p.H);
    const float amax = q_tile_amax<DQK>(qtok, p.q_sh, qt0, qt1, s_red);
    const float s_q = q_scale_from_amax(amax);
    const float r_q = 1.0f / s_q;
    // quantise this group's HT heads once, into LDS
    constexpr int CPR = DQK / 8;
    auto quantize_into_lds = [&](auto fast) {
      for (int c = tid; c < HT * CPR; c += kThreads) {
        const int hh = c / CPR, cc = c - hh * CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(qtok + (int64_t)(h0 + hh) * p.q_sh + cc * 8);
        *reinterpret_cast<u32x2*>(smem + hh * DQK + cc * 8) = quantize_chunk<decltype(fast)::value>(v, s_q, r_q);
      }
    };
    if (q_tile_fast_div(amax)) quantize_into_lds(std::true_type{});
    else quantize_into_lds(std::false_type{});
    __syncthreads();
    const uint8_t* qs = smem + (ht * 16 + m16) * DQK;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
      const int d0 = kb * 128 + 32 * g;
      u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (d0 < DQK) { a = lds_read16(qs + d0); b = lds_read16(qs + d0 + 16); }
      q8[kb] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                     (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    __syncthreads();   // the ring is reused by the gather below
    c2 = p.sm_scale * p.kv_scale * s_q * kLog2e;
  }

  // ---- gather: wave w fetches tile rows 16w .. 16w+15 -----------------------
  u32x4 ld[G::NLD];
  uint32_t ld_mask = 0;
  const uint8_t* zero_row = g_zero_row;

  auto issue = [&](int tile) {
    const int k0 = kbeg + tile * kBK + 16 * wave;
    const uint8_t* rp[16];
    uint32_t vm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = k0 + j;
      const int64_t slot = (k < kend) ? (int64_t)idx_t[k] : -1;
      const bool ok = slot >= 0 && slot < p.N;
      rp[j] = ok ? p.kv + slot * G::ROW : zero_row;
      vm |= ok ? (1u << j) : 0u;
    }
    ld_mask = vm;
    if constexpr (!KV8) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        ld[j] = *reinterpret_cast<const u32x4*>(rp[j] + 16 * lane);
    } else {
      // two rows per load: lanes 0-31 row 2j, lanes 32-63 row 2j+1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint8_t* b = (lane < 32) ? rp[2 * j] : rp[2 * j + 1];
        ld[j] = *reinterpret_cast<const u32x4*>(b + 16 * (lane & 31));
      }
    }
    if constexpr (G::NLD_TAIL > 0) {
      // RoPE columns: each load covers 64/TCH rows x TCH chunks
      constexpr int RPL = 64 / G::TCH;
#pragma unroll
      for (int j = 0; j < G::NLD_TAIL; ++j) {
        const int rl = j * RPL + lane / G::TCH;
        const uint8_t* b = rp[0];
#pragma unroll
        for (int x = 1; x < 16; ++x) b = (rl == x) ? rp[x] : b;
        ld[G::NLD_MAIN + j] = *reinterpret_cast<const u32x4*>(b + G::MAIN + 16 * (lane % G::TCH));
      }
    }
  };

  auto commit = [&](int stage) {
    uint8_t* st = smem + stage * G::STAGE;
    const int r0 = 16 * wave;
    if constexpr (!KV8) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *reinterpret_cast<u32x4*>(st + lds_main<G>(r0 + j, lane)) = ld[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x4*>(st + lds_main<G>(r0 + 2 * j + (lane >> 5), lane & 31)) = ld[j];
    }
    if constexpr (G::NLD_TAIL > 0) {
      constexpr int RPL = 64 / G::TCH;
#pragma unroll
      for (int j = 0; j < G::NLD_TAIL; ++j)
        *reinterpret_cast<u32x4*>(st + lds_tail<G>(r0 + j * RPL + lane / G::TCH, lane % G::TCH)) =
            ld[G::NLD_MAIN + j];
    }
    if (lane == 0) s_mask[stage][wave] = ld_mask;
  };

  // ---- running state --------------------------------------------------------
  f32x4 O[NSLOT][8];
#pragma unroll
  for (int a = 0; a < NSLOT; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[a][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of the logits (log2 domain), per head
  float l_run = 0.0f;        // this lane's share of the running denominator

  float* sx = reinterpret_cast<float*>(smem + RING);

  if (ntiles > 0) { issue(0); commit(0); }
  if (ntiles > 1) issue(1);

  for (int it = 0; it < ntiles; ++it) {
    const int stage = it & 1;
    __syncthreads();   // stage `it` gathered by every wave
    const uint8_t* st = smem + stage * G::STAGE;
    const uint64_t tmask = (uint64_t)s_mask[stage][0] | ((uint64_t)s_mask[stage][1] << 16) |
                           ((uint64_t)s_mask[stage][2] << 32) | ((uint64_t)s_mask[stage][3] << 48);

    // ---- QK^T for this wave's row blocks: S^T[row][head]
    f32x4 sacc[BPW];
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int r = 16 * (bi * WD + dp) + m16;   // tile row this lane feeds
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!KV8) {
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb) {
          const int c = 4 * kb + g;   // 16-byte chunk: columns 32kb + 8g .. +8
          const u32x4 a = (kb < G::MCH / 4) ? lds_read16(st + lds_main<G>(r, c))
                                            : lds_read16(st + lds_tail<G>(r, c - G::MCH));
          acc = mfma_bf16(a, qf[kb], acc);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb) {
          const int c = 8 * kb + 2 * g;   // two chunks: columns 128kb + 32g .. +32
          u32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
          if (kb < G::MCH / 8) {
            a0 = lds_read16(st + lds_main<G>(r, c));
            a1 = lds_read16(st + lds_main<G>(r, c + 1));
          } else if (2 * g < G::TCH) {   // RoPE columns 512 .. Dqk-1; the rest is zero
            a0 = lds_read16(st + lds_tail<G>(r, c - G::MCH));
            a1 = lds_read16(st + lds_tail<G>(r, c - G::MCH + 1));
          }
          const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                           (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          acc = mfma_fp8(a, q8[kb], acc);
        }
      }
      sacc[bi] = acc;
    }

    // ---- all NBLK blocks of scores for this lane's head: rows 16b + 4g + i
    float sv[NBLK][4];
    if constexpr (WD == 1) {
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[b][i] = sacc[b][i];
    } else {
#pragma unroll
      for (int bi = 0; bi < BPW; ++bi) {
        const int b = bi * WD + dp;
        *reinterpret_cast<f32x4*>(sx + ((ht * NBLK + b) * 16 + m16) * 16 + 4 * g) = sacc[bi];
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(sx + ((ht * NBLK + b) * 16 + m16) * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[b][i] = v[i];
      }
    }

    // ---- online softmax
    float mt = -INFINITY;
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * b + 4 * g + i;
        const float x = ((tmask >> row) & 1ull) ? sv[b][i] * c2 : -INFINITY;
        sv[b][i] = x;
        mt = fmaxf(mt, x);
      }
    mt = group4_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    uint32_t pk[NBLK][2];
    float psum = 0.0f;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const float e0 = __builtin_amdgcn_exp2f(sv[b][0] - m_use);
      const float e1 = __builtin_amdgcn_exp2f(sv[b][1] - m_use);
      const float e2 = __builtin_amdgcn_exp2f(sv[b][2] - m_use);
      const float e3 = __builtin_amdgcn_exp2f(sv[b][3] - m_use);
      pk[b][0] = pack_bf16(e0, e1);
      pk[b][1] = pack_bf16(e2, e3);
      // the denominator sums exactly the bf16 weights PV multiplies by
      psum += (bf16_lo(pk[b][0]) + bf16_hi(pk[b][0])) + (bf16_lo(pk[b][1]) + bf16_hi(pk[b][1]));
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int a = 0; a < NSLOT; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[a][e] *= alpha;

    // ---- PV: O^T[dim][head] += V^T[dim][row] * P^T[row][head]
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      // k-slot i' of lane group g <-> tile row 16*(2ks + i'/4) + 4g + i'%4
      const u32x4 pf = {pk[2 * ks][0], pk[2 * ks][1], pk[2 * ks + 1][0], pk[2 * ks + 1][1]};
#pragma unroll
      for (int a = 0; a < NSLOT; ++a) {
        const int c = dp * (DPW / 8) + m16 + 16 * a;   // 8-column chunk of this lane
        u32x4 R[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 16 * (2 * ks + (i >> 2)) + 4 * g + (i & 3);
          if constexpr (!KV8) {
            R[i] = lds_read16(st + lds_main<G>(row, c));
          } else {
            const u32x2 raw = lds_read8(st + lds_main<G>(row, c >> 1) + 8 * (c & 1));
            const u32x2 lo = e4m3x4_to_bf16x4(raw[0]);
            const u32x2 hi = e4m3x4_to_bf16x4(raw[1]);
            R[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
        // 8 rows x 8 columns of bf16 -> per column e: 8 rows, as an A operand
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x4 A;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t lo = R[2 * x][w], hi = R[2 * x + 1][w];
            A[x] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          O[a][e] = mfma_bf16(A, pf, O[a][e]);
        }
      }
    }

    // ---- refill: tile it+1 -> the other stage (free since the barrier above),
    // then start fetching tile it+2 into registers
    if (it + 1 < ntiles) commit(stage ^ 1);
    if (it + 2 < ntiles) issue(it + 2);
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l = group4_sum(l_run);
  const bool any = l > 0.0f;
  const float scale = any ? p.kv_scale / l : 0.0f;
  const float lse_nat = any ? (m_run + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  const int64_t th = (int64_t)t * p.H + head;
#pragma unroll
  for (int a = 0; a < NSLOT; ++a) {
    const int d0 = dp * DPW + 128 * a + 32 * g;   // 32 contiguous columns of this lane
    if (p.S == 1) {
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int j0 = 2 * k, j1 = 2 * k + 1;   // column offset 8i + e
        w[k] = pack_bf16(O[a][j0 & 7][j0 >> 3] * scale, O[a][j1 & 7][j1 >> 3] * scale);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(p.out + th * kDV + d0);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(p.part_o + ((int64_t)s * p.T * p.H + th) * kDV + d0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        f32x4 v;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int j = 4 * k + x;
          v[x] = O[a][j & 7][j >> 3] * scale;
        }
        dst[k] = v;
      }
    }
  }
  if (g == 0 && dp == 0) {
    if (p.S == 1) p.lse[th] = lse_nat;
    else p.part_lse[(int64_t)s * p.T * p.H + th] = lse_nat;
  }
}

// ---- split merge: out = sum_s w_s * O_s / sum_s w_s, w_s = exp(lse_s - max) ----
__global__ __launch_bounds__(kThreads) void smla_combine_kernel(FwdParams p) {
  const int64_t TH = (int64_t)p.T * p.H;
  const int64_t pair = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  if (pair >= TH) return;
  const int d4 = (threadIdx.x & 127) * 4;
  float M = -INFINITY;
  for (int s = 0; s < p.S; ++s) M = fmaxf(M, p.part_lse[s * TH + pair]);
  u32x2* dst = reinterpret_cast<u32x2*>(p.out + pair * kDV + d4);
  if (M == -INFINITY) {
    *dst = u32x2{0u, 0u};
    if (d4 == 0) p.lse[pair] = -INFINITY;
    return;
  }
  float W = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.S; ++s) {
    const float ls = p.part_lse[s * TH + pair];
    if (ls == -INFINITY) continue;   // empty split: its partial is not read
    const float w = __builtin_amdgcn_exp2f((ls - M) * kLog2e);
    W += w;
    acc += w * *reinterpret_cast<const f32x4*>(p.part_o + (s * TH + pair) * kDV + d4);
  }
  const float inv = 1.0f / W;
  *dst = u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  if (d4 == 0) p.lse[pair] = M + __builtin_amdgcn_logf(W) * kLn2;
}

// ---- the per-tile q quantisation alone: one workgroup per (token, 64-head tile)
template <int DQK>
__global__ __launch_bounds__(kThreads) void smla_quantize_q_kernel(const uint16_t* q, int64_t q_st,
                                                                   int64_t q_sh, int32_t H,
                                                                   uint8_t* codes, float* scales) {
  __shared__ float s_red[4];
  const int G = (H + 63) / 64;
  const int t = blockIdx.x / G, gq = blockIdx.x % G;
  const int qt0 = gq * 64, qt1 = min(qt0 + 64, H);
  const uint16_t* qtok = q + (int64_t)t * q_st;
  const float amax = q_tile_amax<DQK>(qtok, q_sh, qt0, qt1, s_red);
  const float s_q = q_scale_from_amax(amax);
  const float r_q = 1.0f / s_q;
  constexpr int CPR = DQK / 8;
  auto quantize_out = [&](auto fast) {
    for (int c = threadIdx.x; c < (qt1 - qt0) * CPR; c += blockDim.x) {
      const int hh = qt0 + c / CPR, cc = c % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(qtok + (int64_t)hh * q_sh + cc * 8);
      *reinterpret_cast<u32x2*>(codes + ((int64_t)t * H + hh) * DQK + cc * 8) =
          quantize_chunk<decltype(fast)::value>(v, s_q, r_q);
    }
  };
  if (q_tile_fast_div(amax)) quantize_out(std::true_type{});
  else quantize_out(std::false_type{});
  if (threadIdx.x == 0) scales[(int64_t)t * G + gq] = s_q;
}

// ---- launch wrappers ----------------------------------------------------------------
template <bool KV8, int DQK>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const int HT = heads_per_workgroup(p.H);
  const int HG = p.H / HT;
  const int64_t units = (int64_t)p.T * p.S;
  const int64_t grid = ((units + 7) / 8) * 8 * HG;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(kThreads);
  switch (HT) {
    case 16: hipLaunchKernelGGL((smla_fwd_kernel<KV8, DQK, 16>), gd, bd, 0, stream, p); break;
    case 32: hipLaunchKernelGGL((smla_fwd_kernel<KV8, DQK, 32>), gd, bd, 0, stream, p); break;
    default: hipLaunchKernelGGL((smla_fwd_kernel<KV8, DQK, 64>), gd, bd, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, bool kv_fp8, int dqk, hipStream_t stream) {
  if (kv_fp8) return dqk == 576 ? launch_fwd_t<true, 576>(p, stream) : launch_fwd_t<true, 512>(p, stream);
  return dqk == 576 ? launch_fwd_t<false, 576>(p, stream) : launch_fwd_t<false, 512>(p, stream);
}

hipError_t launch_combine(const FwdParams& p, hipStream_t stream) {
  const int64_t TH = (int64_t)p.T * p.H;
  const dim3 gd((unsigned)((TH + 1) / 2)), bd(kThreads);
  hipLaunchKernelGGL(smla_combine_kernel, gd, bd, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quantize_q(const uint16_t* q, int64_t q_st, int64_t q_sh, int32_t T, int32_t H,
                             int dqk, uint8_t* codes, float* scales, hipStream_t stream) {
  const int G = (H + 63) / 64;
  const dim3 gd((unsigned)((int64_t)T * G)), bd(kThreads);
  if (dqk == 576)
    hipLaunchKernelGGL(smla_quantize_q_kernel<576>, gd, bd, 0, stream, q, q_st, q_sh, H, codes, scales);
  else
    hipLaunchKernelGGL(smla_quantize_q_kernel<512>, gd, bd, 0, stream, q, q_st, q_sh, H, codes, scales);
  return hipGetLastError();
}

}  // namespace smla
