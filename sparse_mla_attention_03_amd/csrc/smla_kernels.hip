// smla_kernels.hip -- gfx950 kernels of libsparsemla.
//
// A workgroup owns one unit of work: a query token t, a group of heads and a
// split s (a contiguous range of t's top-k list).  Three kernels, by heads per
// workgroup:
//
//   smla_rows_kernel   16 heads (H not a multiple of 32).  Four waves; each
//                      streams its own 32-row tiles (16 for bf16 with RoPE) of
//                      the split through a private LDS slot, one tile in
//                      flight in registers, no barrier in the loop; the waves
//                      merge their (max, sum, O) once at the end.
//   smla_heads_kernel  64 heads (H a multiple of 64).  Eight waves: four score
//                      waves gather the shared tiles, run QK^T and the softmax
//                      and write P to LDS; four output waves hold O^T for 128
//                      columns of all 64 heads and run PV one tile behind.
//   smla_tiles_kernel  32 heads (H = 32 mod 64).  Four waves share each 64-row
//                      tile in LDS, one barrier per tile.
//
// Per gathered row they run the same steps:
//   gather   16-byte buffer loads by slot id into registers (out-of-range
//            ids, padding and entries past the split read zeros, never the
//            pool), then into LDS with 16-byte chunks permuted by the row
//            number (conflict-free row and column reads).
//   QK^T     v_mfma_f32_16x16x32_bf16 (bf16 KV) or v_mfma_f32_16x16x128_f8f6f4
//            (e4m3 KV, q quantised per 64-head tile), fp32 accumulation.
//   softmax  online, in registers, log2 domain; a lane owns one head and a
//            few rows, so the only cross-lane step is a max over 4 lanes.
//   PV       V = the first 512 columns of the same LDS rows as the MFMA
//            operand next to P (bf16); O^T[dim][head] accumulates in fp32.
//   epilogue S == 1: out = bf16(O * kv_scale / l), lse = ln(sum exp).  S > 1:
//            normalised fp32 partials + lse per split, merged by the combine
//            kernel (log-sum-exp weights).
#include <type_traits>

#include <hip/hip_ext.h>

#include "smla_common.h"

namespace smla {

template <bool KV8, int DQK, int HT, bool QB = false>
__global__ __launch_bounds__(kThreads, 1) void smla_tiles_kernel(FwdParams p) {
  using G = Geom<KV8, DQK>;
  // QB: e4m3 KV with bf16 QK dots (q as given, K dequantised exactly);
  // F8: e4m3 dots on the per-tile quantised q
  constexpr bool F8 = KV8 && !QB;
  constexpr int NKQ = F8 ? G::NKB : DQK / 32;   // QK k-steps
  constexpr int WH = HT / 16;          // 16-head tiles per workgroup
  constexpr int WD = 4 / WH;           // waves per head tile
  constexpr int DPW = kDV / WD;        // output columns per wave
  constexpr int NSLOT = DPW / 128;     // 8-column chunks per lane (x16 lanes x8 = 128 cols)
  constexpr int NBLK = kBK / 16;       // 16-row blocks per tile
  constexpr int BPW = NBLK / WD;       // QK row blocks per wave
  constexpr int NSTAGE = 2;
  constexpr int SX = (WD > 1) ? WH * NBLK * 16 * 16 * 4 : 0;   // score exchange bytes
  constexpr int QLDS = F8 ? HT * DQK : 0;                      // quantised q (prologue only)
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
  Unit wu;
  if (!unit_of(p, u, wu)) return;
  const int t = wu.t;
  const int h0 = hg * HT;
  const int kbeg = wu.kbeg;
  const int kend = wu.kend;
  const int ntiles = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

  const int head = h0 + ht * 16 + m16;
  const uint16_t* qtok = p.q + (int64_t)t * p.q_st;
  const uint16_t* qrow = qtok + (int64_t)head * p.q_sh;
  const int32_t* idx_t = p.idx + (int64_t)t * p.idx_st;

  // ---- q operand (B of QK^T): lane (m16 = head, g) holds 8 (bf16) or 32 (fp8)
  // columns per k-step; column d of the row maps to the same (k-step, g, slot)
  // in the K fragments below.
  u32x4 qf[F8 ? 1 : NKQ];
  i32x8 q8[F8 ? G::NKB : 1];
  float c2;   // logit multiplier, log2 domain
  if constexpr (!F8) {
#pragma unroll
    for (int kb = 0; kb < NKQ; ++kb)
      qf[kb] = *reinterpret_cast<const u32x4*>(qrow + kb * 32 + 8 * g);
    c2 = p.sm_scale * p.kv_scale * kLog2e;
  } else {
    float s_q;
    if (p.q_scale > 0.0f) {
      // q given as e4m3 codes with one per-tensor scale: copy this group's rows
      constexpr int CPC = DQK / 16;
      const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)t * p.q_st;
      for (int c = tid; c < HT * CPC; c += kThreads) {
        const int hh = c / CPC, cc = c - hh * CPC;
        *reinterpret_cast<u32x4*>(smem + hh * DQK + cc * 16) =
            *reinterpret_cast<const u32x4*>(qb + (int64_t)(h0 + hh) * p.q_sh + cc * 16);
      }
      s_q = p.q_scale;
    } else {
      // per-tile q quantisation: tile = heads [64*floor(h/64), +64) of token t
      const int qt0 = (h0 / 64) * 64;
      const int qt1 = min(qt0 + 64, p.H);
      const float amax = q_tile_amax<DQK>(qtok, p.q_sh, qt0, qt1, s_red);
      s_q = q_scale_from_amax(amax);
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
    }
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

  auto tile_k0 = [&](int tile) { return kbeg + tile * kBK + 16 * wave; };
  auto issue = [&](int vidx) {
    const uint8_t* rp[16];
    ld_mask = tile_rows<G::ROW>(vidx, p.kv, p.N, zero_row, rp);
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

  // slot ids run two tiles ahead of the row loads that use them
  int vidx_next = load_tile_idx(idx_t, tile_k0(0), kend, lane);
  int vidx_next2 = load_tile_idx(idx_t, tile_k0(1), kend, lane);
  if (ntiles > 0) { issue(vidx_next); commit(0); }
  vidx_next = vidx_next2;
  vidx_next2 = load_tile_idx(idx_t, tile_k0(2), kend, lane);
  if (ntiles > 1) issue(vidx_next);
  vidx_next = vidx_next2;

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
      } else if constexpr (QB) {
#pragma unroll
        for (int kb = 0; kb < NKQ; ++kb) {
          // e4m3 columns 32kb + 8g .. +8: half of 16-byte chunk 2kb + g/2, widened exactly
          const int c = 2 * kb + (g >> 1);
          const int o = (c < G::MCH) ? lds_main<G>(r, c) : lds_tail<G>(r, c - G::MCH);
          const u32x2 raw = lds_read8(st + o + 8 * (g & 1));
          const u32x2 lo = e4m3x4_to_bf16x4(raw[0]);
          const u32x2 hi = e4m3x4_to_bf16x4(raw[1]);
          acc = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, qf[kb], acc);
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
      psum += (e0 + e1) + (e2 + e3);   // fp32 weights: the denominator and lse stay fp32-accurate
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
    const int vidx_after = load_tile_idx(idx_t, tile_k0(it + 3), kend, lane);
    if (it + 2 < ntiles) issue(vidx_next);
    vidx_next = vidx_after;
  }

  // ---- epilogue ---------------------------------------------------------------
  const UnitTail wt = unit_tail(p, u);
  const float2 nz = finish_row(m_run, group4_sum(l_run), sink_log2(p, head, wt.direct), p.kv_scale);
  const float scale = nz.x;
  const float lse_nat = nz.y;
  const int64_t th = (int64_t)t * p.H + head;
#pragma unroll
  for (int a = 0; a < NSLOT; ++a) {
    const int d0 = dp * DPW + 128 * a + 32 * g;   // 32 contiguous columns of this lane
    if (wt.direct) {
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
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(O[a][j & 7][j >> 3]));
      const int e = part_exp(quarter_max(amax * scale));   // rounding is monotonic
      u32x2* dst = reinterpret_cast<u32x2*>(p.part_o) + part_chunk(p, wt.prow, head, d0 / 4);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        f32x4 v;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int j = 4 * k + x;
          v[x] = O[a][j & 7][j >> 3] * scale;
        }
        part_store(dst + 16 * k, part_encode(v, e));
      }
      if (g == 0) part_store_scale(p, wt.prow, head, (dp * DPW + 128 * a) / 128, e);
    }
  }
  if (g == 0 && dp == 0) {
    if (wt.direct) p.lse[th] = lse_nat;
    else part_store_f32(p.part_lse + (int64_t)wt.prow * p.H + head, lse_nat);
  }
}

// ---- 16-head groups: every wave streams its own tiles ---------------------------


template <bool KV8, int DQK, int TR, bool QB = false>
__global__ __launch_bounds__(kThreads, 1) void smla_rows_kernel(FwdParams p) {
  using G = Geom<KV8, DQK>;
  // QB: e4m3 KV with bf16 QK dots (q as given, K dequantised exactly);
  // F8: e4m3 dots on the per-tile quantised q
  constexpr bool F8 = KV8 && !QB;
  constexpr int NKQ = F8 ? G::NKB : DQK / 32;             // QK k-steps
  static_assert(TR == 16 || TR == 32, "a wave tile is one or two 16-row blocks");
  constexpr int NB = TR / 16;                             // 16-row blocks per tile
  constexpr int WMAIN = TR * G::MAIN;
  constexpr int WSLOT = TR * (G::MAIN + G::TAIL);         // a wave's LDS slot
  // Gather layout: one 64-lane load covers 8 rows x 128 bytes (8 lanes per full
  // cache line); lane l takes row 8*grp + (l >> 3), chunk (l & 7) + 8*i.
  constexpr int NGRP = TR / 8;                            // 8-row groups per tile
  constexpr int NCI = G::MCH / 8;                         // 128-byte pieces of a row's V part
  constexpr int NLDM = NGRP * NCI;                        // main loads per tile
  constexpr int TROWS = (G::TCH == 8) ? 8 : 16;           // RoPE part: rows per load
  constexpr int NLDT = G::TCH ? TR / TROWS : 0;           // RoPE loads per tile
  constexpr int NLD = NLDM + NLDT;
  constexpr int QROW = DQK * (F8 ? 1 : 2) + 16;           // padded q row (no bank conflicts)
  constexpr int QBYTES = 16 * QROW;                       // the group's q (B operand of QK^T)
  constexpr int OPAD = kDV + 4;                           // padded fp32 row of the merge buffer
  constexpr int MERGE = 4 * 16 * OPAD * 4;                // the four waves' O (after the loop)
  constexpr int SMEM = (4 * WSLOT + QBYTES > MERGE) ? 4 * WSLOT + QBYTES : MERGE;

  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;

  // workgroup -> (token, split, 16-head group), head groups of a unit 8 ids apart
  const int HG = p.H / 16;
  const int L = blockIdx.x;
  const int hg = (L >> 3) % HG;
  const int u = ((L >> 3) / HG) * 8 + (L & 7);
  Unit wu;
  if (!unit_of(p, u, wu)) return;
  const int t = wu.t;
  const int h0 = hg * 16;
  const int kbeg = wu.kbeg;
  const int kend = wu.kend;
  const int ntile = kend > kbeg ? (kend - kbeg + TR - 1) / TR : 0;
  const int nt = ntile > wave ? (ntile - wave + 3) / 4 : 0;   // this wave's tiles: wave + 4i

  const int head = h0 + m16;
  const uint16_t* qtok = p.q + (int64_t)t * p.q_st;
  const int32_t* idx_t = p.idx + (int64_t)t * p.idx_st;

  uint8_t* slot = smem + wave * WSLOT;   // this wave's tile, rows 0 .. TR-1
  // 16-byte chunk c of tile row r sits at chunk position c ^ row_key(r) (V
  // part) or c ^ (r & (TCH-1)) (RoPE part): conflict-free row and column accesses.
  auto off_main = [](int r, int c) { return r * G::MAIN + 16 * (c ^ row_key(r)); };
  auto off_tail = [](int r, int c) { return WMAIN + r * G::TAIL + 16 * (c ^ (r & (G::TCH - 1))); };

  // ---- slot ids of a tile: lane j < TR holds entry k0 + j of the list, or -1
  // (padding, out of range, past the split: all read zeros).  Returns the
  // record index every lane gathers for each 8-row group via ds_bpermute.
  auto tile_k0 = [&](int i) { return kbeg + TR * (wave + 4 * i); };
  auto load_idx = [&](int i) -> int {
    const int k = tile_k0(i) + (lane & (TR - 1));
    return (lane < TR && k < kend) ? idx_t[k] : -1;
  };
  auto issue = [&](u32x4 (&ld)[NLD], uint32_t& vmask, int vslot) {
    const bool ok = lane < TR && vslot >= 0 && (int64_t)vslot < p.N;
    vmask = (uint32_t)__ballot(ok);
    const int rec = ok ? vslot : -1;   // -1: the zero row
#pragma unroll
    for (int grp = 0; grp < NGRP; ++grp) {
      const uint8_t* rp = pool_row(p.kv, __shfl(rec, 8 * grp + (lane >> 3)), G::ROW) + 16 * (lane & 7);
#pragma unroll
      for (int i = 0; i < NCI; ++i) ld[grp * NCI + i] = load16(rp + 128 * i);
    }
    if constexpr (NLDT > 0) {
      // RoPE part: 8 rows x 8 chunks (bf16) or 16 rows x 4 chunks (e4m3) per load
#pragma unroll
      for (int j = 0; j < NLDT; ++j) {
        const uint8_t* rp = pool_row(p.kv, __shfl(rec, TROWS * j + lane / G::TCH), G::ROW);
        ld[NLDM + j] = load16(rp + G::MAIN + 16 * (lane % G::TCH));
      }
    }
  };

  // lane bases of the commit: lane l writes row 8grp + h (h = l >> 3), whose
  // key is 8 (h & 1) + 4 (grp & 1) + (h >> 1), so chunk (l & 7) + 8i lands at
  // 8 (i ^ (h & 1)) + ((l & 7) ^ (4 (grp & 1) + (h >> 1))): one base per
  // parity of grp and of i
  int cm_base[2][2];
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      const int h = lane >> 3;
      cm_base[gp][ip] = h * G::MAIN + 128 * (ip ^ (h & 1)) + 16 * ((lane & 7) ^ (4 * gp + (h >> 1)));
    }
  auto commit = [&](const u32x4 (&ld)[NLD]) {
#pragma unroll
    for (int grp = 0; grp < NGRP; ++grp)
#pragma unroll
      for (int i = 0; i < NCI; ++i)
        *reinterpret_cast<u32x4*>(slot + cm_base[grp & 1][i & 1] + 8 * grp * G::MAIN + 256 * (i >> 1)) =
            ld[grp * NCI + i];
    if constexpr (NLDT > 0) {
#pragma unroll
      for (int j = 0; j < NLDT; ++j)
        *reinterpret_cast<u32x4*>(slot + off_tail(TROWS * j + lane / G::TCH, lane % G::TCH)) = ld[NLDM + j];
    }
  };

  // ---- slot ids of the first two tiles, then the group's 16 q rows (every
  // thread loads its chunks at once; indices clamped instead of guarded, so all
  // loads are in flight together), then the first tile's rows: the row
  // requests wait only for the ids, and the q staging below overlaps them
  int vidx_next = load_idx(0);
  int vidx_next2 = load_idx(1);
  constexpr int CPR = DQK / 8;                              // 16-byte chunks per head row
  constexpr int NQ = (16 * CPR + kThreads - 1) / kThreads;  // chunks per thread
  constexpr int CPC = DQK / 16;                             // ... per row of e4m3 codes
  constexpr int NQC = (16 * CPC + kThreads - 1) / kThreads;
  const bool qpre = F8 && p.q_scale > 0.0f;                 // q given as e4m3 codes
  u32x4 qv[NQ];
  if (!qpre) {
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      const int c = min(tid + r * kThreads, 16 * CPR - 1), hh = c / CPR, cc = c - hh * CPR;
      qv[r] = *reinterpret_cast<const u32x4*>(qtok + (int64_t)(h0 + hh) * p.q_sh + cc * 8);
    }
  } else {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)t * p.q_st;
#pragma unroll
    for (int r = 0; r < NQC; ++r) {
      const int c = min(tid + r * kThreads, 16 * CPC - 1), hh = c / CPC, cc = c - hh * CPC;
      qv[r] = *reinterpret_cast<const u32x4*>(qb + (int64_t)(h0 + hh) * p.q_sh + cc * 16);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 ldA[NLD];
  uint32_t vmA = 0;
  issue(ldA, vmA, vidx_next);   // unconditional: past the split every row reads as zero
  vidx_next = vidx_next2;

  // ---- q operand (B of QK^T), staged once in LDS for the four waves: bf16 rows,
  // or e4m3 codes of the per-tile quantised q
  uint8_t* qs = smem + 4 * WSLOT;
  float c2;
  if constexpr (!F8) {
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      const int c = tid + r * kThreads, hh = c / CPR, cc = c - hh * CPR;
      if (c < 16 * CPR) *reinterpret_cast<u32x4*>(qs + hh * QROW + cc * 16) = qv[r];
    }
    c2 = p.sm_scale * p.kv_scale * kLog2e;
  } else if (qpre) {
    // codes as given, one per-tensor scale
#pragma unroll
    for (int r = 0; r < NQC; ++r) {
      const int c = tid + r * kThreads, hh = c / CPC, cc = c - hh * CPC;
      if (c < 16 * CPC) *reinterpret_cast<u32x4*>(qs + hh * QROW + cc * 16) = qv[r];
    }
    c2 = p.sm_scale * p.kv_scale * p.q_scale * kLog2e;
  } else {
    const int qt0 = (h0 / 64) * 64;
    const int qt1 = min(qt0 + 64, p.H);
    float amax;
    if (qt1 - qt0 == 16) {
      // the quantisation tile is exactly this head group: amax from the registers
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < NQ; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m = fmaxf(m, fmaxf(fabsf(bf16_lo(qv[r][i])), fabsf(bf16_hi(qv[r][i]))));
      m = wave_max(m);
      if (lane == 0) s_red[wave] = m;
      __syncthreads();
      amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    } else {
      amax = q_tile_amax<DQK>(qtok, p.q_sh, qt0, qt1, s_red);
    }
    const float s_q = q_scale_from_amax(amax);
    const float r_q = 1.0f / s_q;
    auto quantize_into_lds = [&](auto fast) {
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        const int c = tid + r * kThreads, hh = c / CPR, cc = c - hh * CPR;
        if (c < 16 * CPR)
          *reinterpret_cast<u32x2*>(qs + hh * QROW + cc * 8) = quantize_chunk<decltype(fast)::value>(qv[r], s_q, r_q);
      }
    };
    if (q_tile_fast_div(amax)) quantize_into_lds(std::true_type{});
    else quantize_into_lds(std::false_type{});
    c2 = p.sm_scale * p.kv_scale * s_q * kLog2e;
  }
  __syncthreads();
  // lane (head = m16, g): bf16 columns 32kb + 8g .. +8, or e4m3 columns 128kb + 32g .. +32
  const uint8_t* qlane = qs + m16 * QROW;

  // QK reads: row 16b + m16 has key k = row_key(m16), so chunk 4kb + g lands
  // at 4 (kb ^ (k >> 2)) + (g ^ (k & 3)): four lane bases, one per kb mod 4
  int qk_base[4];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int k = row_key(m16);
    qk_base[r4] = m16 * G::MAIN + 64 * (r4 ^ (k >> 2)) + 16 * (g ^ (k & 3));
  }
  // PV reads (bf16): row 16b + 4g + i, chunk m16 + 16a lands at
  // 16a + (m16 ^ row_key(4g + i))
  int pv_base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pv_base[i] = (4 * g + i) * G::MAIN + 16 * (m16 ^ row_key(4 * g + i));
  // bf16 V through transposed LDS reads: in k-slot group g, lane k = m16 of the
  // group reads row 16b + 4g + (k >> 2) (key kr), 4 columns from
  // 128a + 32 (k & 3) + 4e; 16-byte chunk 16a + 4 (k & 3) + (e >> 1) of that
  // row lands at 16a + ((4 (k & 3) + (e >> 1)) ^ kr), half e & 1 of it.  So
  // lane (m16, g) receives column 128a + 32 (m16 >> 2) + 4e + (m16 & 3) of
  // rows 16b + 4g .. + 3, the A operand whose output lane (head, g) holds
  // columns 128a + 32g + 4e + i in O[a][e][i].
  // 32-row tiles: lanes with k & 2 set read the other 8-byte half of each
  // 16-byte chunk (columns from 4 (e ^ 1)): lanes (k & 3, row) and
  // (k & 3 ^ 2, row ^ 1) of a group land on the same 16-byte bank slot of the
  // swizzle and so use different halves of it (a third of the bank-conflict
  // cycles on prefill; the 16-row decode tiles keep the plain order, where the
  // extra lane arithmetic costs more than the conflicts).  O[a][e] of output
  // lane group g then holds columns 128a + 32g + 4 (e ^ ((g >> 1) & 1)).
  constexpr bool FLIP = !KV8 && TR == 32;
  int pvt_base[NB][4][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = 16 * b + 4 * g + (m16 >> 2);
    const int fl = FLIP ? 8 * ((m16 >> 1) & 1) : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int base = r * G::MAIN + 16 * ((4 * (m16 & 3) + h) ^ row_key(r));
      pvt_base[b][h][0] = base + fl;
      pvt_base[b][h][1] = base + 8 - fl;
    }
  }

  f32x4 O[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[a][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // ---- QK^T of the wave's tile: S^T[row][head] per 16-row block b, lane
  // (head = m16, g) receives rows 16b + 4g .. 16b + 4g + 3.  k-step outer,
  // blocks inner, so each q fragment feeds NB MFMAs; two partial sums per
  // block (even / odd k-steps) keep back-to-back MFMAs independent, and the
  // fragments of the next DEPTH k-steps are read ahead of their MFMAs.
  using KFrag = std::conditional_t<F8, i32x8, u32x4>;
  auto kfrag = [&](int b, int kb) -> KFrag {
    if constexpr (QB) {
      // e4m3 columns 32kb + 8g .. +8 (8 bytes of a 16-byte chunk), widened to
      // bf16 exactly; RoPE columns come from the tail part
      const int r = 16 * b + m16;
      const int c = 2 * kb + (g >> 1);
      const int o = (c < G::MCH) ? off_main(r, c) : off_tail(r, c - G::MCH);
      const u32x2 raw = lds_read8(slot + o + 8 * (g & 1));
      const u32x2 lo = e4m3x4_to_bf16x4(raw[0]);
      const u32x2 hi = e4m3x4_to_bf16x4(raw[1]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else if constexpr (!KV8) {
      return (kb < G::MCH / 4) ? lds_read16(slot + 16 * b * G::MAIN + qk_base[kb & 3] + 256 * (kb >> 2))
                               : lds_read16(slot + off_tail(16 * b + m16, 4 * kb + g - G::MCH));
    } else {
      const int c = 8 * kb + 2 * g;
      u32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      if (kb < G::MCH / 8) {
        a0 = lds_read16(slot + off_main(16 * b + m16, c));
        a1 = lds_read16(slot + off_main(16 * b + m16, c + 1));
      } else if (2 * g < G::TCH) {   // RoPE columns; the rest of the k-step is zero
        a0 = lds_read16(slot + off_tail(16 * b + m16, c - G::MCH));
        a1 = lds_read16(slot + off_tail(16 * b + m16, c - G::MCH + 1));
      }
      return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    }
  };
  auto qfrag = [&](int kb) -> KFrag {
    if constexpr (!F8) {
      return lds_read16(qlane + (kb * 32 + 8 * g) * 2);
    } else {
      const int c = 8 * kb + 2 * g;
      u32x4 b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
      if (kb < G::MCH / 8 || 2 * g < G::TCH) {
        b0 = lds_read16(qlane + 16 * c);
        b1 = lds_read16(qlane + 16 * c + 16);
      }
      return i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    }
  };
  constexpr int DEPTH = 3;
  auto qk = [&](f32x4 (&acc)[NB]) {
    if constexpr (F8) {
      // e4m3: few, wide k-steps (128 columns); the NB blocks are the
      // independent chains
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < G::NKB; ++kb) {
        const KFrag bq = qfrag(kb);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_fp8(kfrag(b, kb), bq, acc[b]);
      }
      return;
    }
    f32x4 ac[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b) ac[b][0] = ac[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    KFrag ra[DEPTH][NB], rq[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      rq[d] = qfrag(d);
#pragma unroll
      for (int b = 0; b < NB; ++b) ra[d][b] = kfrag(b, d);
    }
#pragma unroll
    for (int kb = 0; kb < NKQ; ++kb) {
      const KFrag bq = rq[kb % DEPTH];
      KFrag a[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) a[b] = ra[kb % DEPTH][b];
      if (kb + DEPTH < NKQ) {
        rq[kb % DEPTH] = qfrag(kb + DEPTH);
#pragma unroll
        for (int b = 0; b < NB; ++b) ra[kb % DEPTH][b] = kfrag(b, kb + DEPTH);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (!F8) ac[b][kb & 1] = mfma_bf16(a[b], bq, ac[b][kb & 1]);
        else ac[b][kb & 1] = mfma_fp8(a[b], bq, ac[b][kb & 1]);
      }
    }
    if constexpr (!F8) {
      // issue order: DEPTH k-steps of reads, then per k-step NB MFMAs and the
      // NB + 1 reads of k-step kb + DEPTH
      constexpr int RPK = NB + 1;
      __builtin_amdgcn_sched_group_barrier(0x100, DEPTH * RPK, 0);
#pragma unroll
      for (int kb = 0; kb < NKQ; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
        if (kb + DEPTH < NKQ) __builtin_amdgcn_sched_group_barrier(0x100, RPK, 0);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = ac[b][0] + ac[b][1];
  };

  // ---- scores of the tile in log2 units (masked rows -inf) and their max
  float sv[NB][4];
  float mt = -INFINITY;
  auto score = [&](uint32_t vm) {
    f32x4 acc[NB];
    qk(acc);
    mt = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[b][i] = ((vm >> (16 * b + 4 * g + i)) & 1u) ? acc[b][i] * c2 : -INFINITY;
        mt = fmaxf(mt, sv[b][i]);
      }
    mt = group4_max(mt);
  };

  // ---- P = exp2(s - m_run) and O^T[dim][head] += V^T[dim][row] P^T[row][head];
  // k-slot g holds rows 16b + 4g + i for every block b (i = 0..3), in the same
  // order on both sides
  auto accumulate = [&]() {
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    uint32_t pk[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float e0 = __builtin_amdgcn_exp2f(sv[b][0] - m_use);
      const float e1 = __builtin_amdgcn_exp2f(sv[b][1] - m_use);
      const float e2 = __builtin_amdgcn_exp2f(sv[b][2] - m_use);
      const float e3 = __builtin_amdgcn_exp2f(sv[b][3] - m_use);
      l_run += (e0 + e1) + (e2 + e3);
      pk[b][0] = pack_bf16(e0, e1);
      pk[b][1] = pack_bf16(e2, e3);
    }
    if constexpr (!KV8) {
      // 128-column chunk a + 1's transposed reads interleaved with chunk a's MFMAs
      u32x2 A[2][8][NB];
      auto load_a = [&](int a) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int b = 0; b < NB; ++b) A[a & 1][e][b] = lds_read_tr16(slot + pvt_base[b][e >> 1][e & 1] + 256 * a);
      };
      load_a(0);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (a + 1 < 4) load_a(a + 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (NB == 1) {
            O[a][e] = mfma_bf16_k16(A[a & 1][e][0], u32x2{pk[0][0], pk[0][1]}, O[a][e]);
          } else {
            O[a][e] = mfma_bf16(u32x4{A[a & 1][e][0][0], A[a & 1][e][0][1], A[a & 1][e][1][0], A[a & 1][e][1][1]},
                                u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]}, O[a][e]);
          }
        }
      }
      // issue order: chunk 0's reads, then per chunk its MFMAs with the next chunk's reads between them
      __builtin_amdgcn_sched_group_barrier(0x100, 8 * NB, 0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (a + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);
        }
      return;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c = m16 + 16 * a;   // 8-column chunk of this lane
      u32x4 R[4 * NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * b + 4 * g + i;
          if constexpr (!KV8) {
            R[4 * b + i] = lds_read16(slot + pv_base[i] + 16 * b * G::MAIN + 256 * a);
          } else {
            const u32x2 raw = lds_read8(slot + off_main(row, c >> 1) + 8 * (c & 1));
            const u32x2 lo = e4m3x4_to_bf16x4(raw[0]);
            const u32x2 hi = e4m3x4_to_bf16x4(raw[1]);
            R[4 * b + i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        if constexpr (NB == 1) {
          const u32x2 pf = {pk[0][0], pk[0][1]};
          const u32x2 A = (e & 1) ? u32x2{pack_hi(R[0][w], R[1][w]), pack_hi(R[2][w], R[3][w])}
                                  : u32x2{pack_lo(R[0][w], R[1][w]), pack_lo(R[2][w], R[3][w])};
          O[a][e] = mfma_bf16_k16(A, pf, O[a][e]);
        } else {
          const u32x4 pf = {pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
          u32x4 A;
#pragma unroll
          for (int x = 0; x < 4; ++x)
            A[x] = (e & 1) ? pack_hi(R[2 * x][w], R[2 * x + 1][w]) : pack_lo(R[2 * x][w], R[2 * x + 1][w]);
          O[a][e] = mfma_bf16(A, pf, O[a][e]);
        }
      }
    }
  };

  // ---- main loop: one tile in flight in registers while the previous one
  // computes from LDS; slot ids run two tiles ahead of the loads that use them.
  // m_run is a reference max that may lag the true one by up to kSlack, so
  // exponents stay <= 2^kSlack.  A head with no valid entry yet simply takes
  // the tile's max (its O is still zero).  Only when a head's scores outgrow a
  // finite reference must O be rescaled; that leaves the inner loop for the
  // outer one, so the inner loop touches O by MFMAs alone.
  int i = 0;
  for (;;) {
    for (; i < nt; ++i) {
      commit(ldA);
      const uint32_t va = vmA;
      const int vidx_after = load_idx(i + 2);
      if (i + 1 < nt) issue(ldA, vmA, vidx_next);   // none past the end: the merge barrier would wait for it
      vidx_next = vidx_after;
      score(va);
      if (__ballot(m_run != -INFINITY && mt > m_run + kSlack) != 0) break;
      m_run = (m_run == -INFINITY) ? mt : m_run;
      accumulate();
    }
    if (i >= nt) break;
    // tile i is scored and outgrows a reference: rescale, accumulate, go on
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[a][e] *= alpha;
    accumulate();
    ++i;
  }

  // ---- merge the four waves: each writes its raw O (straight from the
  // accumulators) and (max, sum) to LDS; wave w then combines columns
  // [128w, 128w + 128) of all four in a fixed order and writes them out.
  // Quarter a of O (columns 128a ..) is O[a]; for split partials a wave keeps
  // its own quarter in registers, so only the other three go through LDS.
  // quad k of this lane's head in quarter a: columns 128a + 32g + 4 (k ^ fq)
  // .. + 3; one accumulator with bf16 V (transposed reads), spread over four
  // with e4m3 V (column 8c + e of chunk c in O[a][e]; fq = 0)
  const int fq = FLIP ? ((g >> 1) & 1) : 0;
  auto o_quad = [&](int a, int k) -> f32x4 {
    if constexpr (!KV8) {
      return O[a][k];
    } else {
      f32x4 v;
#pragma unroll
      for (int x = 0; x < 4; ++x) { const int j = 4 * k + x; v[x] = O[a][j & 7][j >> 3]; }
      return v;
    }
  };
  const float l_w = group4_sum(l_run);
  const UnitTail wt = unit_tail(p, u);
  __syncthreads();   // every wave is done with its slot; the merge reuses them
  float* ob = reinterpret_cast<float*>(smem);
  {
    float* row = ob + (wave * 16 + m16) * OPAD;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (a == wave && !wt.direct) continue;
        *reinterpret_cast<f32x4*>(row + 128 * a + 32 * g + 4 * (k ^ fq)) = o_quad(a, k);
      }
  }
  if (g == 0) { s_m[wave][m16] = m_run; s_l[wave][m16] = l_w; }
  __syncthreads();
  // weights of the four waves for head m16
  float M = s_m[0][m16];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][m16]);
  float f[4], Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][m16] - M);
    Lsum += f[w] * s_l[w][m16];
  }
  const float2 nz = finish_row(M, Lsum, sink_log2(p, head, wt.direct), p.kv_scale);
  const float scale = nz.x;
  if (!wt.direct) {
    // lane (m16, g) merges columns 128 wave + 32 g + 4 (k ^ fq) .. + 4 (k < 8) of
    // head m16 -- the columns its own accumulators hold -- and stores them as
    // chunks 32 wave + 8 g + (k ^ fq): each store writes four whole 128-byte lines
    f32x4 vv[8];
    float amax = 0.0f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a != wave) continue;   // uniform: the quarter index stays a constant
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          f32x4 o;
          if (w == a) {
            o = o_quad(a, k);
          } else {
            o = *reinterpret_cast<const f32x4*>(ob + (w * 16 + m16) * OPAD + 128 * a + 32 * g + 4 * (k ^ fq));
          }
          v += f[w] * o;
        }
        vv[k] = v * scale;
        amax = fmaxf(fmaxf(amax, fmaxf(fabsf(vv[k][0]), fabsf(vv[k][1]))), fmaxf(fabsf(vv[k][2]), fabsf(vv[k][3])));
      }
    }
    const int e = part_exp(quarter_max(amax));   // this wave's columns are quarter `wave`
    u32x2* dst = reinterpret_cast<u32x2*>(p.part_o) + part_chunk(p, wt.prow, head, 32 * wave + 8 * g);
#pragma unroll
    for (int k = 0; k < 8; ++k) part_store(dst + 16 * (k ^ fq), part_encode(vv[k], e));
    if (g == 0) part_store_scale(p, wt.prow, head, wave, e);
  } else {
    // 16 heads x 16 chunks of 8 columns, 4 per lane: store k takes head 4k + g,
    // columns 128 wave + 8 m16 .. + 8, so 16 lanes write a head's 256 bytes;
    // the weights of head 4k + g come from lane 4k + g
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int hh = 4 * k + g;
      float fk[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) fk[w] = __shfl(f[w], hh);
      const float sk = __shfl(scale, hh);
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* src = ob + (w * 16 + hh) * OPAD + 128 * wave + 8 * m16;
        v0 += fk[w] * *reinterpret_cast<const f32x4*>(src);
        v1 += fk[w] * *reinterpret_cast<const f32x4*>(src + 4);
      }
      *reinterpret_cast<u32x4*>(p.out + ((int64_t)t * p.H + h0 + hh) * kDV + 128 * wave + 8 * m16) =
          u32x4{pack_bf16(v0[0] * sk, v0[1] * sk), pack_bf16(v0[2] * sk, v0[3] * sk),
                pack_bf16(v1[0] * sk, v1[1] * sk), pack_bf16(v1[2] * sk, v1[3] * sk)};
    }
  }
  if (wave == 0 && g == 0) {
    const int64_t th = (int64_t)t * p.H + head;
    if (wt.direct) p.lse[th] = nz.y;
    else part_store_f32(p.part_lse + (int64_t)wt.prow * p.H + head, nz.y);
  }
}

// ---- 64-head groups: score waves and output waves ---------------------------------
// Eight waves.  Waves 0-3 (score waves) gather the tiles and own 16 heads each:
// q stays in their registers as the B operand of QK^T, and they keep the online
// softmax state and write P (bf16) to LDS.  Waves 4-7 (output waves) own 128
// output columns of all 64 heads: O^T[128][64] in accumulators, with every V
// fragment read from LDS feeding four head blocks.  Scoring runs one tile ahead
// of PV, so each SIMD interleaves one score wave's and one output wave's MFMAs;
// three LDS stages hold the tile being scored, the tile being multiplied and
// the tile being filled, and one barrier per tile separates the phases.
template <bool KV8, int DQK, bool VL = false, bool QB = false>
__global__ __launch_bounds__(2 * kThreads) void smla_heads_kernel(FwdParams p) {
  using G = Geom<KV8, DQK>;
  // QB: e4m3 KV with bf16 QK dots (q as given, K widened to bf16 exactly);
  // F8: e4m3 dots on the quantised q
  static_assert(!QB || KV8, "bf16 dots are an e4m3-KV variant");
  constexpr bool F8 = KV8 && !QB;
  constexpr int NKQ = F8 ? G::NKB : DQK / 32;   // QK k-steps
  // rows per tile: 36 KiB for Dqk = 576 with e4m3 dots or bf16 KV; 32 rows (18 KiB) for bf16
  // dots on e4m3 KV, whose score waves hold q as bf16 and have no registers for more
  constexpr int TR = (KV8 && !QB) ? 64 : 32;
  constexpr int NB = TR / 16;              // 16-row QK blocks per tile
  constexpr int NKS = TR / 32;             // 32-row PV k-steps per tile
  constexpr int RPW = TR / 4;              // rows each score wave gathers (8 or 16)
  constexpr int NGRP = RPW / 8;            // 8-row load groups
  constexpr int NCI = G::MAIN / 128;       // 128-byte pieces of a row's V part
  constexpr int NLDM = NGRP * NCI;
  constexpr int TROWS = (G::TCH == 8 || RPW < 16) ? 8 : 16;   // RoPE part: rows per load
  constexpr int NLDT = G::TCH ? RPW / TROWS : 0;
  constexpr int NLD = NLDM + NLDT;
  constexpr int TMAIN = TR * G::MAIN;
  constexpr int STAGE = TR * G::ROW;
  constexpr int PBUF = NKS * 4 * 64 * 16;  // P^T operands of one tile, lane order
  static_assert(RPW % 8 == 0 && (G::TCH == 0 || RPW % TROWS == 0), "gather shape");

  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * STAGE + 2 * PBUF];
  __shared__ uint32_t s_mask[3][4];        // validity bits of each score wave's rows, per stage
  __shared__ float s_alpha[2][64];         // rescale factor of O per head (when flagged)
  __shared__ int s_flag[2][4];             // score wave w moved its heads' reference max
  __shared__ float s_lfin[64];             // final multipliers of O (kv_scale / denominator)
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;

  // workgroup -> (token, split, 64-head group); the head groups of one
  // (token, split) are 8 ids apart, on one XCD, so the second gather of a row
  // is served by that XCD's L2
  const int HG = p.H / 64;
  const int L = blockIdx.x;
  const int hg = (L >> 3) % HG;
  const int u = ((L >> 3) / HG) * 8 + (L & 7);
  // VL: the per-token plan's table (a separate instantiation: the 64-head
  // kernel has no registers to spare for a branch between the two)
  int t, s, kbeg, kend;
  if constexpr (!VL) {
    if (u >= p.T * p.S) return;
    t = u / p.S;
    s = u - t * p.S;
    kbeg = s * p.rps;
    kend = min(kbeg + p.rps, p.K);
  } else {
    if (u >= __builtin_amdgcn_readfirstlane(*p.num_units)) return;
    const int4 e = p.units[u];
    t = __builtin_amdgcn_readfirstlane(e.x);
    s = 0;
    kbeg = __builtin_amdgcn_readfirstlane(e.y);
    kend = __builtin_amdgcn_readfirstlane(e.z);
  }
  const int h0 = hg * 64;
  // tiles, rounded up to even: the score waves run two phases per trip with
  // no exit in between (an odd count gets one all-padding tile, which adds 0)
  const int nt = kend > kbeg ? (((kend - kbeg + TR - 1) / TR + 1) & ~1) : 0;
  const uint16_t* qtok = p.q + (int64_t)t * p.q_st;
  uint8_t* pbuf = smem + 3 * STAGE;

  // 16-byte chunk c of tile row r sits at chunk position c ^ row_key(r) (V
  // part) or c ^ (r & (TCH-1)) (RoPE part)
  auto off_main = [](int r, int c) { return r * G::MAIN + 16 * (c ^ row_key(r)); };
  auto off_tail = [](int r, int c) { return TMAIN + r * G::TAIL + 16 * (c ^ (r & (G::TCH - 1))); };

  if (wave < 4) {
    // =============================== score waves ===============================
    const int qw = wave;                   // heads h0 + 16 qw + m16; gathers tile rows RPW*qw ..
    const int head = h0 + 16 * qw + m16;
    const uint16_t* qrow = qtok + (int64_t)head * p.q_sh;
    const int32_t* idx_t = p.idx + (int64_t)t * p.idx_st;

    // slot ids through a raw buffer over this split's entries: the load is
    // issued for every lane (out of range reads zero), then masked to -1
    const __amdgpu_buffer_rsrc_t ids = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(idx_t + kbeg), (short)0, (int)(4 * (kend > kbeg ? kend - kbeg : 0)), kBufferRsrcWord3);
    auto load_idx = [&](int j) -> int {
      return raw_load_b32(ids, 4 * (TR * j + RPW * qw + (lane & (RPW - 1))), 0, 0);
    };
    // rows of this wave's share of tile j: 8 rows x 128 bytes per load (lane l:
    // row l >> 3, chunk l & 7 of a 128-byte piece); padding, entries past the
    // split and lanes >= RPW read zeros.  The range test is made here, not at
    // the slot id load, so nothing waits on that load before it is needed.
    auto issue = [&](u32x4 (&ld)[NLD], uint32_t& vm, int vslot, int j) {
      const int k = kbeg + TR * j + RPW * qw + (lane & (RPW - 1));
      const bool ok = lane < RPW && k < kend && vslot >= 0 && (int64_t)vslot < p.N;
      vm = (uint32_t)__ballot(ok);
      const int rec = ok ? vslot : -1;   // -1: the zero row
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        const uint8_t* rp = pool_row(p.kv, __shfl(rec, 8 * grp + (lane >> 3)), G::ROW) + 16 * (lane & 7);
#pragma unroll
        for (int i = 0; i < NCI; ++i) ld[grp * NCI + i] = load16(rp + 128 * i);
      }
      if constexpr (NLDT > 0) {
#pragma unroll
        for (int j = 0; j < NLDT; ++j) {
          const uint8_t* rp = pool_row(p.kv, __shfl(rec, TROWS * j + lane / G::TCH), G::ROW);
          ld[NLDM + j] = load16(rp + G::MAIN + 16 * (lane % G::TCH));
        }
      }
    };
    // row rb + h (h = l >> 3, rb a multiple of 8) has key 8 (h & 1) + 4x +
    // (h >> 1), x = (rb >> 3) & 1, so chunk (l & 7) + 8i lands at
    // 8 (i ^ (h & 1)) + ((l & 7) ^ (4x + (h >> 1)))
    const int hl = lane >> 3;
    const int cm_par[2] = {128 * (hl & 1), -128 * (hl & 1)};   // 128 (i ^ (h&1)) - 128 i, by i parity
    auto commit = [&](int stage, const u32x4 (&ld)[NLD], uint32_t vm) {
      uint8_t* st = smem + stage * STAGE;
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        const int rb = RPW * qw + 8 * grp;
        const int x = (rb >> 3) & 1;
        uint8_t* base = st + (rb + hl) * G::MAIN + 16 * ((lane & 7) ^ (4 * x + (hl >> 1)));
#pragma unroll
        for (int i = 0; i < NCI; ++i)
          *reinterpret_cast<u32x4*>(base + 128 * i + cm_par[i & 1]) = ld[grp * NCI + i];
      }
      if constexpr (NLDT > 0) {
#pragma unroll
        for (int j = 0; j < NLDT; ++j)
          if (lane / G::TCH < TROWS)   // e4m3 parts of 8 rows: lanes 32-63 load zeros and store nothing
            *reinterpret_cast<u32x4*>(st + off_tail(RPW * qw + TROWS * j + lane / G::TCH, lane % G::TCH)) =
                ld[NLDM + j];
      }
      if (lane == 0) s_mask[stage][qw] = vm;
    };

    // slot ids of the first two tiles, then q, then the first tile's rows: all
    // in flight together, and the q loads complete before the loop (the wait
    // for tile 0 covers them), so the loop never waits on them
    u32x4 ldA[NLD], ldB[NLD];              // two tiles in flight: odd tiles in A, even in B
    uint32_t vmA = 0, vmB = 0;
    int vA = load_idx(0);
    const int vB = load_idx(1);
    const int vC = load_idx(2);

    // ---- q operand (B of QK^T): lane (head m16, g) holds bf16 columns
    // 32kb + 8g .. +8, or e4m3 codes of columns 128kb + 32g .. +32
    u32x4 qf[F8 ? 1 : NKQ];
    i32x8 q8[F8 ? G::NKB : 1];
    u32x4 qv[F8 ? G::NKB : 1][4];
    const bool qpre = F8 && p.q_scale > 0.0f;   // q given as e4m3 codes
    if constexpr (!F8) {
#pragma unroll
      for (int kb = 0; kb < NKQ; ++kb)
        qf[kb] = *reinterpret_cast<const u32x4*>(qrow + kb * 32 + 8 * g);
    } else if (qpre) {
      // e4m3 codes of columns 128kb + 32g .. +32 (the B fragment as it is) in
      // the first two chunks of the staging registers
      const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)t * p.q_st + (int64_t)head * p.q_sh;
#pragma unroll
      for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int col = 128 * kb + 32 * g + 16 * jj;
          const u32x4 v = *reinterpret_cast<const u32x4*>(qb + min(col, DQK - 16));
          qv[kb][jj] = (col < DQK) ? v : u32x4{0u, 0u, 0u, 0u};
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int col = 128 * kb + 32 * g + 8 * jj;
          // columns past Dqk (the last k-step of Dqk = 576) are zero; the load
          // address is clamped so every load issues unconditionally
          const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + min(col, DQK - 8));
          qv[kb][jj] = (col < DQK) ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // bf16: keep every q load ahead of the row loads, so the wait for tile 0
    // retires them and the loop never waits on them.  e4m3: the rows are
    // requested once q is quantised (fewer registers live at once).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!F8) issue(ldA, vmA, vA, 0);

    float c2;
    if constexpr (!F8) {
      // QB (e4m3 KV): q needs no quantisation, but the output waves still
      // meet the score waves at the q amax exchange barrier
      if constexpr (KV8) __syncthreads();
      c2 = p.sm_scale * p.kv_scale * kLog2e;
    } else if (qpre) {
      __syncthreads();   // the output waves' barrier of the q amax exchange
#pragma unroll
      for (int kb = 0; kb < G::NKB; ++kb)
        q8[kb] = i32x8{(int)qv[kb][0][0], (int)qv[kb][0][1], (int)qv[kb][0][2], (int)qv[kb][0][3],
                       (int)qv[kb][1][0], (int)qv[kb][1][1], (int)qv[kb][1][2], (int)qv[kb][1][3]};
      c2 = p.sm_scale * p.kv_scale * p.q_scale * kLog2e;
      issue(ldA, vmA, vA, 0);
    } else {
      // the 64 heads are exactly one quantisation tile: amax over the four
      // score waves' registers, then s_q = amax / 448 and codes in registers
      float am = 0.0f;
#pragma unroll
      for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            am = fmaxf(am, fmaxf(fabsf(bf16_lo(qv[kb][jj][i])), fabsf(bf16_hi(qv[kb][jj][i]))));
      am = wave_max(am);
      if (lane == 0) s_red[qw] = am;
      __syncthreads();
      const float amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      const float s_q = q_scale_from_amax(amax);
      const float r_q = 1.0f / s_q;
      auto quantize = [&](auto fast) {
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const u32x2 c = quantize_chunk<decltype(fast)::value>(qv[kb][jj], s_q, r_q);
            q8[kb][2 * jj] = (int)c[0];
            q8[kb][2 * jj + 1] = (int)c[1];
          }
      };
      if (q_tile_fast_div(amax)) quantize(std::true_type{});
      else quantize(std::false_type{});
      c2 = p.sm_scale * p.kv_scale * s_q * kLog2e;
      issue(ldA, vmA, vA, 0);
    }

    commit(0, ldA, vmA);                   // tile 0 -> stage 0
    // The order of these loads is what the loop's waits count on (set A and
    // its ids strictly before set B and its ids); sched_barrier pins it.
    issue(ldA, vmA, vB, 1);                // tiles 1 and 2 in flight (zeros past the split)
    vA = load_idx(3);
    __builtin_amdgcn_sched_barrier(0);
    issue(ldB, vmB, vC, 2);
    int vD = load_idx(4);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

    // QK reads (bf16): row 16b + m16 has key k = row_key(m16), so chunk
    // 4kb + g lands at 4 (kb ^ (k >> 2)) + (g ^ (k & 3)): one lane base per kb mod 4
    int qk_base[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int k = row_key(m16);
      qk_base[r4] = m16 * G::MAIN + 64 * (r4 ^ (k >> 2)) + 16 * (g ^ (k & 3));
    }

    float m_run = -INFINITY;   // reference max (log2 domain) of this lane's head; may lag by kSlack
    float l_run = 0.0f;        // this lane's share of the denominator

    // One QK^T A fragment: rows 16b .. 16b + 15 of the tile, bf16 columns
    // 32kb + 8g .. +8 (one 16-byte read) or e4m3 columns 128kb + 32g .. +32
    // (two reads; zeros past Dqk)
    using Frag = std::conditional_t<F8, i32x8, u32x4>;
    auto frag = [&](const uint8_t* st, int b, int kb) -> Frag {
      const int r = 16 * b + m16;
      if constexpr (QB) {
        // e4m3 columns 32kb + 8g .. +8 (half a 16-byte chunk; RoPE columns from
        // the tail part), widened to bf16 exactly
        const int c = 2 * kb + (g >> 1);
        const int o = (c < G::MCH) ? off_main(r, c) : off_tail(r, c - G::MCH);
        const u32x2 raw = lds_read8(st + o + 8 * (g & 1));
        const u32x2 lo = e4m3x4_to_bf16x4(raw[0]);
        const u32x2 hi = e4m3x4_to_bf16x4(raw[1]);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else if constexpr (!KV8) {
        return (kb < G::MCH / 4) ? lds_read16(st + 16 * b * G::MAIN + qk_base[kb & 3] + 256 * (kb >> 2))
                                 : lds_read16(st + off_tail(r, 4 * kb + g - G::MCH));
      } else {
        const int c = 8 * kb + 2 * g;
        u32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
        if (kb < G::MCH / 8) {
          a0 = lds_read16(st + off_main(r, c));
          a1 = lds_read16(st + off_main(r, c + 1));
        } else if (2 * g < G::TCH) {   // RoPE columns; the rest of the k-step is zero
          a0 = lds_read16(st + off_tail(r, c - G::MCH));
          a1 = lds_read16(st + off_tail(r, c - G::MCH + 1));
        }
        return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      }
    };
    // S^T[row][head] of the tile's NB row blocks.  bf16: fragments are read
    // DEPTH k-steps ahead of their MFMA (LDS latency) and each block keeps two
    // partial sums (even / odd k-steps), so back-to-back MFMAs are
    // independent.  e4m3: the four blocks already are.
    // QB: one partial sum per row block (its bf16 q takes the registers of the
    // second); with 32-row tiles its two blocks alternate
    constexpr int DEPTH = 3;
    constexpr int NACC = QB ? 1 : 2;
    auto qk = [&](const uint8_t* st, f32x4 (&acc)[NB]) {
      if constexpr (F8) {
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[b] = mfma_fp8(frag(st, b, kb), q8[kb], acc[b]);
      } else {
        f32x4 ac[NB][NACC];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int h = 0; h < NACC; ++h) ac[b][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        Frag ring[DEPTH][NB];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
#pragma unroll
          for (int b = 0; b < NB; ++b) ring[d][b] = frag(st, b, d);
#pragma unroll
        for (int kb = 0; kb < NKQ; ++kb) {
          Frag cur[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) cur[b] = ring[kb % DEPTH][b];
          if (kb + DEPTH < NKQ) {
#pragma unroll
            for (int b = 0; b < NB; ++b) ring[kb % DEPTH][b] = frag(st, b, kb + DEPTH);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) ac[b][kb % NACC] = mfma_bf16(cur[b], qf[kb], ac[b][kb % NACC]);
        }
        // issue order: DEPTH k-steps of reads, then one MFMA per read, so
        // NB * DEPTH reads stay in flight (the default schedule keeps ~2)
        constexpr int NR = NB * NKQ, PRE = NB * DEPTH;
        __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
        for (int i = 0; i < NR - PRE; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc[b] = ac[b][0];
#pragma unroll
          for (int h = 1; h < NACC; ++h) acc[b] += ac[b][h];
        }
      }
    };

    // scores, softmax and P of the tile in stage sq, into P buffer PB
    auto score_tile = [&](int sq, auto pb_sel) {
      constexpr int PB = decltype(pb_sel)::value;
      uint64_t tm = 0;   // validity of the tile's rows (read before the MFMAs)
#pragma unroll
      for (int w = 0; w < 4; ++w) tm |= (uint64_t)s_mask[sq][w] << (RPW * w);
      f32x4 acc[NB];
      qk(smem + sq * STAGE, acc);

      // ---- online softmax with a lazily moved reference max
      float sv[NB][4];
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[b][i] = ((tm >> (16 * b + 4 * g + i)) & 1ull) ? acc[b][i] * c2 : -INFINITY;
          mt = fmaxf(mt, sv[b][i]);
        }
      mt = group4_max(mt);
      int moved = 0;
      if (__ballot(mt > m_run + kSlack) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        if (g == 0) s_alpha[PB][16 * qw + m16] = alpha;
        moved = 1;
      }
      if (lane == 0) s_flag[PB][qw] = moved;
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      uint32_t pk[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float e0 = __builtin_amdgcn_exp2f(sv[b][0] - m_use);
        const float e1 = __builtin_amdgcn_exp2f(sv[b][1] - m_use);
        const float e2 = __builtin_amdgcn_exp2f(sv[b][2] - m_use);
        const float e3 = __builtin_amdgcn_exp2f(sv[b][3] - m_use);
        l_run += (e0 + e1) + (e2 + e3);
        pk[b][0] = pack_bf16(e0, e1);
        pk[b][1] = pack_bf16(e2, e3);
      }
      // P^T operand of k-step ks, head block qw: k-slots = rows 32ks + {4g+i, 16+4g+i}
      uint8_t* pb = pbuf + PB * PBUF;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        *reinterpret_cast<u32x4*>(pb + ((ks * 4 + qw) * 64 + lane) * 16) =
            u32x4{pk[2 * ks][0], pk[2 * ks][1], pk[2 * ks + 1][0], pk[2 * ks + 1][1]};
    };

    // Two phases per trip, so each register set has fixed code: tile j + 1
    // goes to LDS and tile j + 3 takes its registers.  Loads and commits are
    // unconditional (past the split they read zeros into a free stage), and
    // each set's slot ids are fetched right after its rows, a trip ahead: so
    // no wait for one set or its ids ever covers the other set's loads.
    int sq = 0;                // stage of tile j
    for (int j = 0; j < nt; j += 2) {
      int sc = (sq == 2) ? 0 : sq + 1;
      score_tile(sq, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
      commit(sc, ldA, vmA);                  // tile j + 1, after the MFMAs are under way
      issue(ldA, vmA, vA, j + 3);
      vA = load_idx(j + 5);
      __builtin_amdgcn_sched_barrier(0);
      sq = sc;
      __syncthreads();
      sc = (sq == 2) ? 0 : sq + 1;
      score_tile(sq, std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
      commit(sc, ldB, vmB);                  // tile j + 2
      issue(ldB, vmB, vD, j + 4);
      vD = load_idx(j + 6);
      __builtin_amdgcn_sched_barrier(0);
      sq = sc;
      __syncthreads();
    }

    // ---- the output waves need the denominators; this wave writes lse
    const UnitTail wt = VL ? unit_tail(p, u) : UnitTail{s * p.T + t, p.S == 1};
    const float2 nz = finish_row(m_run, group4_sum(l_run), sink_log2(p, head, wt.direct), p.kv_scale);
    if (g == 0) s_lfin[16 * qw + m16] = nz.x;
    __syncthreads();   // pairs with the output waves' last PV phase
    if (g == 0) {
      const int64_t th = (int64_t)t * p.H + head;
      if (wt.direct) p.lse[th] = nz.y;
      else part_store_f32(p.part_lse + (int64_t)wt.prow * p.H + head, nz.y);
    }
  } else {
    // =============================== output waves ==============================
    const int pw = wave - 4;               // output columns 128 pw .. 128 pw + 127
    if constexpr (KV8) __syncthreads();    // q amax exchange of the score waves
    __syncthreads();                       // tile 0 in LDS

    // PV reads (bf16): row 16h + 4g + i (key row_key(4g + i)), chunk 16pw + m16
    // lands at 16pw + (m16 ^ row_key(4g + i))
    int pv_base[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv_base[i] = (4 * g + i) * G::MAIN + 16 * (16 * pw + (m16 ^ row_key(4 * g + i)));

    f32x4 O[8][4];   // [column e of the lane's 8-column chunks][head block]
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) O[e][hb] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();   // phase 0: the score waves score tile 0

    // V fragments of a tile (rows 32ks + {4g + i, 16 + 4g + i}, the lane's 8
    // columns 8 (16pw + m16) ..), read one phase ahead of their MFMAs: tile j
    // is in LDS from the start of phase j, its PV runs in phase j + 1
    u32x4 Rv[NKS][8];
    auto pv_load = [&](int sp) {
      const uint8_t* st = smem + sp * STAGE;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 32 * ks + 16 * h + 4 * g + i;
            if constexpr (!KV8) {
              Rv[ks][4 * h + i] = lds_read16(st + pv_base[i] + (32 * ks + 16 * h) * G::MAIN);
            } else {
              const int c = 16 * pw + m16;   // 8-column chunk = half of a 16-byte e4m3 chunk
              const u32x2 raw = lds_read8(st + off_main(row, c >> 1) + 8 * (c & 1));
              Rv[ks][4 * h + i] = u32x4{raw[0], raw[1], 0u, 0u};
            }
          }
    };
    // O^T[col][head] += V^T[col][row] P^T[row][head] for tile jj from Rv
    auto pv = [&](int jj) {
      const uint8_t* pb = pbuf + (jj & 1) * PBUF;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 B[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          B[hb] = *reinterpret_cast<const u32x4*>(pb + ((ks * 4 + hb) * 64 + lane) * 16);
        u32x4 R[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if constexpr (!KV8) {
            R[r] = Rv[ks][r];
          } else {   // e4m3 -> bf16, exact
            const u32x2 lo = e4m3x4_to_bf16x4(Rv[ks][r][0]);
            const u32x2 hi = e4m3x4_to_bf16x4(Rv[ks][r][1]);
            R[r] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x4 A;
#pragma unroll
          for (int x = 0; x < 4; ++x)
            A[x] = (e & 1) ? pack_hi(R[2 * x][w], R[2 * x + 1][w]) : pack_lo(R[2 * x][w], R[2 * x + 1][w]);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) O[e][hb] = mfma_bf16(A, B[hb], O[e][hb]);
        }
      }
    };

    // Phase j multiplies tile j - 1.  The rescale of O (rare: the first valid
    // tile, then only when a head's max outgrows the reference by 2^kSlack)
    // sits in the outer loop, so the inner loop touches O only through MFMAs.
    pv_load(0);
    int j = 1;
    int sp = 0;          // stage of tile j - 1
    bool rescaled = false;
    for (;;) {
      for (; j <= nt; ++j) {
        const int fb = (j - 1) & 1;
        const int fl = __builtin_amdgcn_readfirstlane(s_flag[fb][0] | s_flag[fb][1] | s_flag[fb][2] | s_flag[fb][3]);
        if (fl != 0 && !rescaled) break;
        rescaled = false;
        pv(j - 1);
        sp = (sp == 2) ? 0 : sp + 1;
        pv_load(sp);     // tile j (past the last tile: a stale stage, never used)
        __syncthreads();
      }
      if (j > nt) break;
      const int fb = (j - 1) & 1;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float a = s_flag[fb][hb] ? s_alpha[fb][16 * hb + m16] : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) O[e][hb] *= a;
      }
      rescaled = true;
    }

    // ---- epilogue: lane (m16, g) holds columns 128pw + 32g + 8i + e of head
    // 16hb + m16 in O[e][hb][i]
    const UnitTail wt = VL ? unit_tail(p, u) : UnitTail{s * p.T + t, p.S == 1};
    const int d0 = 128 * pw + 32 * g;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float scale = s_lfin[16 * hb + m16];
      const int64_t th = (int64_t)t * p.H + h0 + 16 * hb + m16;
      if (wt.direct) {
        u32x4* dst = reinterpret_cast<u32x4*>(p.out + th * kDV + d0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t w4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int j0 = 8 * k + 2 * x, j1 = j0 + 1;   // column offset 8i + e
            w4[x] = pack_bf16(O[j0 & 7][hb][j0 >> 3] * scale, O[j1 & 7][hb][j1 >> 3] * scale);
          }
          dst[k] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
      } else {
        float amax = 0.0f;
#pragma unroll
        for (int jx = 0; jx < 32; ++jx) amax = fmaxf(amax, fabsf(O[jx & 7][hb][jx >> 3]));
        const int e = part_exp(quarter_max(amax * scale));   // rounding is monotonic
        u32x2* dst = reinterpret_cast<u32x2*>(p.part_o) + part_chunk(p, wt.prow, h0 + 16 * hb + m16, d0 / 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          f32x4 v;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int jx = 4 * k + x;
            v[x] = O[jx & 7][hb][jx >> 3] * scale;
          }
          part_store(dst + 16 * k, part_encode(v, e));
        }
        if (g == 0) part_store_scale(p, wt.prow, h0 + 16 * hb + m16, pw, e);
      }
    }
  }
}

// ---- split merge: out = sum_s w_s * O_s / sum_s w_s, w_s = exp(lse_s - max) ----
// One workgroup per (token, 16-head group, slice of 64 CPT columns): thread
// (column cl = tid >> 4, head tid & 15) merges chunks cl + 16 k (k < CPT) of the
// slice, so each split's partials of the workgroup arrive as whole lines.  The
// lse and partial loads of B splits are issued together (B CPT of 8 - 16 bytes
// in flight per lane; loads past the token's count are skipped and their
// weight selects zero).  CPT grows with the batch (tokens x head groups) while
// the grid keeps at least 512 workgroups: a short batch gets 8 narrow slices
// per row, a long one fewer, longer-lived workgroups with more loads in
// flight.  The bf16 result goes through LDS so that whole rows are stored.
template <bool VL, int CPT>
__global__ __launch_bounds__(kThreads) void smla_combine_kernel(FwdParams p) {
  constexpr int NSL = 8 / CPT;                  // slices per (token, head group)
  constexpr int B = CPT >= 4 ? 2 : 8 / CPT;     // splits per batch
  constexpr int SROW = 64 * CPT + 8;            // padded LDS row (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t s_out[16][SROW];
  const int HG = p.H / 16;
  const int slice = blockIdx.x % NSL;
  const int unit = blockIdx.x / NSL;
  const int t = unit / HG, grp = unit - t * HG;
  const int hl = threadIdx.x & 15, cl = threadIdx.x >> 4;
  const int head = 16 * grp + hl;
  // the token's partial rows: fr, fr + rs, ... (cnt of them)
  int fr = t, rs = p.T, cnt = p.S;
  if constexpr (VL) {
    // one token per workgroup: keep its values in scalar registers
    fr = __builtin_amdgcn_readfirstlane(p.tok_first[t]);
    rs = 1;
    cnt = __builtin_amdgcn_readfirstlane(p.tok_count[t]);
    if (__builtin_amdgcn_readfirstlane(p.num_units[1]) != 0) {
      // the plan dropped units (its bounds exclude this): every output of the
      // call becomes NaN rather than whatever the buffers held
      for (int i = threadIdx.x; i < 128 * CPT; i += kThreads) {
        const int h = i / (8 * CPT), k8 = i - h * (8 * CPT);
        *reinterpret_cast<u32x4*>(p.out + ((int64_t)t * p.H + 16 * grp + h) * kDV + 64 * CPT * slice + 8 * k8) =
            u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
      }
      if (slice == 0 && cl == 0) p.lse[(int64_t)t * p.H + head] = __builtin_nanf("");
      return;
    }
    if (cnt == 1) return;   // the token's only unit wrote out / lse itself
    cnt = max(0, min(cnt, p.max_prows - fr));
  }
  constexpr int NQ = (CPT + 1) / 2;             // quarters the lane's chunks fall in
  const float* pl = p.part_lse + (int64_t)fr * p.H + head;
  const float* pc = p.part_scale + ((int64_t)fr * p.H + head) * 4 + CPT * slice / 2;
  const u32x2* po = reinterpret_cast<const u32x2*>(p.part_o) + part_chunk(p, fr, head, 16 * CPT * slice + cl);
  const int64_t lstride = (int64_t)rs * p.H;                 // between partial rows: lse,
  const int64_t cstride = 4 * lstride;                       // quarter scales
  const int64_t sstride = (int64_t)rs * p.H * (kDV / 4);     // and chunks
  // a sink enters as one more split whose partial is zero: weight exp(sink - M)
  float M = p.sinks ? p.sinks[head] : -INFINITY;
  float W = (M == -INFINITY) ? 0.0f : 1.0f;
  f32x4 acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < cnt; s0 += B) {
    float ls[B], cs[B][NQ];
    u32x2 v[B][CPT];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      ls[j] = -INFINITY;
#pragma unroll
      for (int k = 0; k < NQ; ++k) cs[j][k] = 0.0f;
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[j][k] = u32x2{0u, 0u};
      if (s0 + j < cnt) {   // uniform
        ls[j] = pl[(s0 + j) * lstride];
#pragma unroll
        for (int k = 0; k < NQ; ++k) cs[j][k] = pc[(s0 + j) * cstride + k];
#pragma unroll
        for (int k = 0; k < CPT; ++k) v[j][k] = po[(s0 + j) * sstride + 256 * k];   // chunk + 16 k
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < B; ++j) mb = fmaxf(mb, ls[j]);
    if (mb == -INFINITY) continue;
    // rescale what was accumulated so far to the new running max
    const float r = __builtin_amdgcn_exp2f((M - mb) * kLog2e);
    W *= r;
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[k] *= r;
    M = mb;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const bool live = ls[j] != -INFINITY;
      const float w = live ? __builtin_amdgcn_exp2f((ls[j] - M) * kLog2e) : 0.0f;
      W += w;
#pragma unroll
      for (int k = 0; k < CPT; ++k)   // chunk cl + 16 k lies in quarter CPT slice / 2 + k / 2
        acc[k] += live ? (w * cs[j][k / 2]) * part_decode(v[j][k]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const float inv = (M == -INFINITY) ? 0.0f : 1.0f / W;   // all splits empty: +0
#pragma unroll
  for (int k = 0; k < CPT; ++k)
    *reinterpret_cast<u32x2*>(&s_out[hl][4 * (cl + 16 * k)]) =
        u32x2{pack_bf16(acc[k][0] * inv, acc[k][1] * inv), pack_bf16(acc[k][2] * inv, acc[k][3] * inv)};
  if (slice == 0 && cl == 0)
    p.lse[(int64_t)t * p.H + head] = (M == -INFINITY) ? -INFINITY : M + __builtin_amdgcn_logf(W) * kLn2;
  __syncthreads();
  // 16 rows of 128 CPT bytes, in 16-byte pieces
  for (int i = threadIdx.x; i < 128 * CPT; i += kThreads) {
    const int h = i / (8 * CPT), k8 = i - h * (8 * CPT);
    *reinterpret_cast<u32x4*>(p.out + ((int64_t)t * p.H + 16 * grp + h) * kDV + 64 * CPT * slice + 8 * k8) =
        *reinterpret_cast<const u32x4*>(&s_out[h][8 * k8]);
  }
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

// ---- the per-token split plan: one workgroup scans the list lengths ---------------
// With W = the batch's tiles (64 entries each, summed over tokens), units are
// R = 64 max(4, ceil(W HG / CUs)) entries long, so the batch's units about fill
// the device once; token t gets count_t = max(1, ceil(len_t / R)) of them.
// Units are numbered token by token; the units of split tokens (count > 1) get
// consecutive partial rows, a token's only unit gets -1 (it writes out / lse
// itself).  Bounds: count_t <= 1 + tiles_t / rt, so units <= T + W / rt <=
// T + CUs / HG; a split token has tiles_t > rt, so count_t <= 2 tiles_t / rt
// and partial rows <= 2 W / rt <= 2 CUs / HG.  The host sizes the tables one
// past these.  Every write is still checked against the table sizes; a unit
// that would not fit is dropped with all units after it, and num_units[1] is
// set, on which the combine kernel writes NaN to every output of the call.
__device__ __forceinline__ int block_sum_1024(int v, int* s_part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) s_part[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < 16; ++w) t += s_part[w];
  return t;
}

__global__ __launch_bounds__(1024) void smla_plan_kernel(PlanParams q) {
  __shared__ int32_t s_part[16], s_part2[16];
  __shared__ int32_t s_carry[2];
  __shared__ int32_t s_cut;   // first unit past a bound (none expected): no unit from it on runs
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // pass 1: the batch's tiles
  int tiles = 0;
  for (int t = tid; t < q.T; t += 1024) tiles += (min(max(q.lens[t], 0), q.K) + 63) / 64;
  const int W = block_sum_1024(tiles, s_part);
  const int rt = max(4, (int)(((int64_t)W * q.HG + q.cus - 1) / q.cus));
  const int R = 64 * rt;
  if (tid == 0) { s_carry[0] = 0; s_carry[1] = 0; s_cut = 0x7fffffff; }
  __syncthreads();
  // pass 2: units and partial rows, two scans at once
  for (int base = 0; base < q.T; base += 1024) {
    const int t = base + tid;
    const int len = (t < q.T) ? min(max(q.lens[t], 0), q.K) : 0;
    const int cnt = (t < q.T) ? max(1, (len + R - 1) / R) : 0;
    const int sp = cnt > 1 ? cnt : 0;
    int x = cnt, y = sp;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int xo = __shfl_up(x, o), yo = __shfl_up(y, o);
      if (lane >= o) { x += xo; y += yo; }
    }
    if (lane == 63) { s_part[wave] = x; s_part2[wave] = y; }
    __syncthreads();
    int bu = s_carry[0], bp = s_carry[1];
    for (int w = 0; w < wave; ++w) { bu += s_part[w]; bp += s_part2[w]; }
    const int fu = bu + x - cnt, fp = bp + y - sp;
    if (t < q.T) {
      q.tok_first[t] = fp;
      q.tok_count[t] = cnt;
      for (int j = 0; j < cnt; ++j) {
        const int pr = (cnt > 1) ? fp + j : -1;
        if (fu + j < q.max_units && pr < q.max_prows)
          q.units[fu + j] = int4{t, j * R, min((j + 1) * R, len), pr};
        else
          atomicMin(&s_cut, fu + j);
      }
    }
    __syncthreads();
    if (tid == 1023) { s_carry[0] = fu + cnt; s_carry[1] = fp + sp; }
    __syncthreads();
  }
  __syncthreads();
  if (tid == 0) {
    *q.num_units = min(min(s_carry[0], q.max_units), s_cut);
    q.num_units[1] = s_cut != 0x7fffffff ? 1 : 0;   // read by the combine kernel
  }
}

hipError_t launch_plan(const PlanParams& q, hipStream_t stream) {
  hipLaunchKernelGGL(smla_plan_kernel, dim3(1), dim3(1024), 0, stream, q);
  return hipGetLastError();
}

// ---- launch wrappers ----------------------------------------------------------------
template <bool KV8, int DQK, bool QB>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int HT = heads_per_workgroup(p.H);
  const int HG = p.H / HT;
  const int64_t units = p.units ? (int64_t)p.max_units : (int64_t)p.T * p.S;
  const int64_t grid = ((units + 7) / 8) * 8 * HG;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(kThreads);
  // hipExtLaunchKernelGGL: the optional events take the kernel's own start and
  // end timestamps (no marker packets around it)
  switch (HT) {
    case 16:
      // Split lists (decode: few rows per workgroup, bound by gather latency)
      // take 16-row wave tiles -- more, shorter pipeline stages and a shorter
      // tail after the last gather.  Whole lists (prefill, bound by LDS
      // bandwidth) take 32-row tiles where four of them plus q fit in LDS: one
      // q fragment read then feeds two 16-row blocks -- unless the list is so
      // short that each wave would get a single 32-row tile, with nothing to
      // overlap its gather (K <= 128: 16-row tiles measured 2 - 3 % faster).
      if constexpr (!KV8 && DQK == 512) {
        if (p.prefill16) return launch_prefill(p, gd, stream, ev0, ev1);
      }
      if constexpr (KV8 || DQK == 512) {
        if (p.S > 1 || p.units != nullptr || p.K <= 4 * 32)
          hipExtLaunchKernelGGL((smla_rows_kernel<KV8, DQK, 16, QB>), gd, bd, 0, stream, ev0, ev1, 0, p);
        else
          hipExtLaunchKernelGGL((smla_rows_kernel<KV8, DQK, 32, QB>), gd, bd, 0, stream, ev0, ev1, 0, p);
      } else {
        hipExtLaunchKernelGGL((smla_rows_kernel<KV8, DQK, 16, QB>), gd, bd, 0, stream, ev0, ev1, 0, p);
      }
      break;
    case 32:
      hipExtLaunchKernelGGL((smla_tiles_kernel<KV8, DQK, 32, QB>), gd, bd, 0, stream, ev0, ev1, 0, p);
      break;
    default:
      if (p.units != nullptr)
        hipExtLaunchKernelGGL((smla_heads_kernel<KV8, DQK, true, QB>), gd, dim3(2 * kThreads), 0, stream, ev0, ev1, 0, p);
      else
        hipExtLaunchKernelGGL((smla_heads_kernel<KV8, DQK, false, QB>), gd, dim3(2 * kThreads), 0, stream, ev0, ev1, 0, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, bool kv_fp8, bool bf16_dots, int dqk, hipStream_t stream,
                      hipEvent_t ev0, hipEvent_t ev1) {
  if (kv_fp8 && bf16_dots)
    return dqk == 576 ? launch_fwd_t<true, 576, true>(p, stream, ev0, ev1)
                      : launch_fwd_t<true, 512, true>(p, stream, ev0, ev1);
  if (kv_fp8)
    return dqk == 576 ? launch_fwd_t<true, 576, false>(p, stream, ev0, ev1)
                      : launch_fwd_t<true, 512, false>(p, stream, ev0, ev1);
  return dqk == 576 ? launch_fwd_t<false, 576, false>(p, stream, ev0, ev1)
                    : launch_fwd_t<false, 512, false>(p, stream, ev0, ev1);
}

template <int CPT>
static void launch_combine_t(const FwdParams& p, int64_t rows, hipStream_t stream) {
  const dim3 gd((unsigned)(rows * (8 / CPT))), bd(kThreads);
  if (p.tok_first != nullptr)
    hipLaunchKernelGGL((smla_combine_kernel<true, CPT>), gd, bd, 0, stream, p);
  else
    hipLaunchKernelGGL((smla_combine_kernel<false, CPT>), gd, bd, 0, stream, p);
}

hipError_t launch_combine(const FwdParams& p, hipStream_t stream) {
  // (token, head group) rows; the widest slices that leave >= 512 workgroups
  const int64_t rows = (int64_t)p.T * (p.H / 16);
  int cpt = 1;
  while (cpt < 8 && rows * (8 / (2 * cpt)) >= 512) cpt *= 2;
  switch (cpt) {
    case 1: launch_combine_t<1>(p, rows, stream); break;
    case 2: launch_combine_t<2>(p, rows, stream); break;
    case 4: launch_combine_t<4>(p, rows, stream); break;
    default: launch_combine_t<8>(p, rows, stream); break;
  }
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
