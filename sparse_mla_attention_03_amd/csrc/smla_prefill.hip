// smla_prefill.hip -- 16-head groups on whole long lists (prefill) of bf16 rows
// 512 wide.
//
// Each wave takes every fourth 16-entry tile of its token's list (tiles wave,
// wave + 4, ...) and streams them through a private LDS slot with no barrier
// in the loop.  Three things set this kernel apart from the 16-head kernel of
// smla_kernels.hip:
//
// * Entry order.  Many query rows of one sequence select overlapping rows of
//   a pool a few MiB large, so whether a gathered row is still in L2 depends
//   on when the waves of an XCD read it.  Before its loop each wave orders its
//   share of the list (up to 512 entries per round) by slot range: a stable
//   split on three bits of the slot id (eight ranges over the pool) and a
//   fourth split that moves invalid entries (padding, ids outside the pool)
//   past the valid ones, where they are dropped.  All resident waves then
//   sweep the pool from low to high slots at about the same pace, and a
//   range of the pool is read by all of them while it is in L2.  The order is
//   a function of the list alone (equal keys keep their list order), so the
//   result is deterministic; softmax does not depend on the order.
//   The sorted ids stay in registers (8 per lane); each tile's ids reach the
//   lanes that need them by one cross-lane permute per 8 rows.
// * Copies.  Rows go from the pool straight into LDS by global_load_lds_dwordx4,
//   8 rows x 128 bytes per copy (lane l: row l >> 3, one 16-byte chunk), so a
//   64-bit lane address is formed once per 8 rows and the eight copies of
//   those rows differ only in their immediate offset; per copy only M0 is
//   set.  In the slot, chunk c of row r sits at byte
//   8192 (r >> 3) + 1024 (c >> 3) + 128 (r & 7) + 16 ((c & 7) ^ kx(r)),
//   kx(r) = (r >> 1) & 7: every copy fills 1 KiB lane-linearly, and 16 rows
//   read at one chunk hit 16 different 16-byte bank groups.
// * Two workgroups per compute unit (two waves per SIMD): LDS per workgroup is
//   exactly 80 KiB, four 16 KiB slots and q (16 rows of 1 KiB, read by all
//   four waves as the B operand of QK^T).
//
// Per tile: QK^T on 16x16x32 bf16 MFMAs (S^T[row][head], fragments read three
// k-steps ahead), the online softmax with a lazily moved reference max, and PV
// on 16x16x16 bf16 MFMAs with V through transposed LDS reads.  At the end the
// four waves merge (max, sum, O) through LDS in two rounds of two 128-column
// quarters and store out / lse (the kernel runs whole lists only: no split).
#include <hip/hip_ext.h>

#include "smla_common.h"

namespace smla {

namespace {

// global_load_lds_dwordx4 from a per-lane 64-bit address plus the immediate
// OFF.  The immediate offsets the LDS destination as well, so M0 is set to
// the wanted destination minus OFF (M0 needs one wait state after it is
// written).  The add that forms M0 writes SCC: declared, so that no compare
// the compiler keeps in SCC lives across a copy.
template <int OFF, int LDS>
__device__ __forceinline__ void copy_v_off(const uint8_t* src, uint32_t slot_lds) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3" ::"v"(src),
               "s"(slot_lds), "i"(LDS - OFF), "i"(OFF)
               : "memory", "m0", "scc");
}

// lanes below this one with their bit set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

}  // namespace

__global__ __launch_bounds__(kThreads, 2) void smla_prefill_kernel(FwdParams p) {
  using G = Geom<false, 512>;
  constexpr int TR = 16;                       // rows per tile
  constexpr int SLOT = TR * G::MAIN;           // 16 KiB
  constexpr int QOFF = 4 * SLOT;               // q: 16 rows of 1 KiB
  constexpr int LDS = QOFF + 16 * G::MAIN;     // 80 KiB: two workgroups per compute unit
  constexpr int NKQ = 16;                      // QK k-steps (32 columns each)
  constexpr int OP = 256 + 4;                  // merge row: two quarters of fp32, padded
  constexpr int NREG = 8;                      // a wave's entries per round: NREG x 64 (32 tiles)
  constexpr int RTILES = NREG * 64 / TR;
  static_assert(4 * 16 * OP * 4 + 2 * 64 * 4 <= LDS, "merge buffer fits");
  static_assert(NREG * 64 * 4 <= SLOT, "the sort scratch fits in a slot");

  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;

  // workgroup -> (token, 16-head group), head groups of a token 8 ids apart
  const int HG = p.H / 16;
  const int L = blockIdx.x;
  const int hg = (L >> 3) % HG;
  const int u = ((L >> 3) / HG) * 8 + (L & 7);
  Unit wu;
  if (!unit_of(p, u, wu)) return;
  const int t = wu.t;
  const int h0 = hg * 16;
  const int len = wu.kend > wu.kbeg ? wu.kend - wu.kbeg : 0;
  const int ntile = (len + TR - 1) / TR;
  const int ntw = ntile > wave ? (ntile - wave + 3) / 4 : 0;   // this wave's tiles: wave + 4i
  const int nround = (ntw + RTILES - 1) / RTILES;
  const int head = h0 + m16;

  uint8_t* slot = smem + wave * SLOT;
  const uint32_t slot_lds = lds_addr(slot);
  const uint8_t* qs = smem + QOFF;
  int32_t* sscr = reinterpret_cast<int32_t*>(slot);   // sort scratch (before a round's copies)

  // ---- the wave's share of round rd: entry j = 64k + l (register k, lane l) is
  // row j & 15 of wave tile 32 rd + (j >> 4), i.e. list position
  // 16 (wave + 4 (32 rd + (j >> 4))) + (j & 15); -1 past the list
  const __amdgpu_buffer_rsrc_t ids_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.idx + (int64_t)t * p.idx_st + wu.kbeg), (short)0, (int)(4 * len), kBufferRsrcWord3);
  // a slot id is valid when 0 <= id < N: one unsigned compare against min(N, 2^31)
  const uint32_t n_lim = (uint32_t)min(p.N, (int64_t)0x80000000LL);
  // slot ranges: the top three bits of the smallest power of two >= N
  const int lg = n_lim > 1 ? 32 - __builtin_clz(n_lim - 1) : 0;
  const int rsh = lg > 3 ? lg - 3 : 0;
  int32_t sid[NREG];
  auto load_round = [&](int rd) {
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const int pos = TR * (wave + 4 * (RTILES * rd + 4 * k + (lane >> 4))) + m16;
      const int v = raw_load_b32(ids_rsrc, 4 * pos, 0, 0);
      sid[k] = pos < len ? v : -1;
    }
  };
  // stable split of the NREG x 64 entries (in order j) on bit b of their key
  // (bits 0-2: slot range, bit 3: invalid) through the wave's LDS scratch;
  // returns the number of entries whose bit is clear
  auto split = [&](int b) -> int {
    uint64_t ones[NREG];
    bool one[NREG];
    int before[NREG];
    int n1 = 0;
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const uint32_t id = (uint32_t)sid[k];
      const uint32_t key = id < n_lim ? ((id >> rsh) & 7u) : 8u;
      one[k] = (key >> b) & 1u;
      ones[k] = __ballot(one[k]);
      before[k] = n1;
      n1 += __popcll(ones[k]);
    }
    const int n0 = NREG * 64 - n1;
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const int o = lanes_below(ones[k]);
      const int pos = one[k] ? n0 + before[k] + o : 64 * k - before[k] + lane - o;
      sscr[pos] = sid[k];
    }
#pragma unroll
    for (int k = 0; k < NREG; ++k) sid[k] = sscr[64 * k + lane];
    return n0;
  };
  auto sort_round = [&]() -> int {
    split(0);
    split(1);
    split(2);
    const int nvalid = split(3);
    wait_lgkmcnt0();   // the scratch reads are done before copies land in the slot
    return nvalid;
  };

  // ---- copies of tile i (of the round): lane l copies row 8 gr + (l >> 3) for
  // gr = 0, 1, its 16-byte chunk (l & 7) ^ kx(row) of each 128-byte piece j
  // into slot byte 1024 (8 gr + j) + 16 l
  const uint32_t key16[2] = {16u * (uint32_t)((lane & 7) ^ (lane >> 4)),
                             16u * (uint32_t)((lane & 7) ^ (4 + (lane >> 4)))};
  const uint8_t* zero_row = g_zero_row;
  // the ids of tile i's copy rows (sid[0] holds tiles 4 (i >> 2) .. + 3 then)
  auto fetch = [&](int i, int32_t (&cid)[2]) {
    cid[0] = __shfl(sid[0], 16 * (i & 3) + (lane >> 3));
    cid[1] = __shfl(sid[0], 16 * (i & 3) + 8 + (lane >> 3));
  };
  auto rotate = [&]() {
#pragma unroll
    for (int k = 0; k + 1 < NREG; ++k) sid[k] = sid[k + 1];
  };
  int nvalid = 0;
  auto issue = [&](int i, const int32_t (&cid)[2]) -> uint32_t {
    static_for<0, 2>([&](auto gc) {
      constexpr int gr = decltype(gc)::value;
      // rows past the valid ones read the zero row; the id test keeps every
      // address inside the pool whatever the permutes delivered
      const bool ok = TR * i + 8 * gr + (lane >> 3) < nvalid && (uint32_t)cid[gr] < n_lim;
      const uint8_t* rp = (ok ? p.kv + (uint64_t)(uint32_t)cid[gr] * G::ROW : zero_row) + key16[gr];
      static_for<0, 8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        copy_v_off<128 * j, 1024 * (8 * gr + j)>(rp, slot_lds);
      });
    });
    const int nv = nvalid - TR * i;   // valid rows of the tile
    return nv >= TR ? 0xffffu : (1u << nv) - 1u;
  };

  // ---- q: wave w copies heads 4w .. 4w + 3 (row h, chunk c at c ^ row_key(h));
  // then the first round's ids, its order, and its first tile
  {
    const uint8_t* qtok = reinterpret_cast<const uint8_t*>(p.q + (int64_t)t * p.q_st);
    const uint32_t lane16 = 16 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * wave + i;
      copy_s(qtok + (int64_t)(h0 + hh) * p.q_sh * 2, lane16 ^ (16 * row_key(hh)), lds_addr(qs) + hh * G::MAIN);
    }
  }
  int nt = 0;                     // tiles of the current round
  int32_t cid[2];
  uint32_t vm_cur = 0;
  auto start_round = [&](int rd) {
    load_round(rd);
    nvalid = sort_round();
    nt = (nvalid + TR - 1) / TR;
    if (nt > 0) {
      fetch(0, cid);
      vm_cur = issue(0, cid);
      fetch(1, cid);
    }
  };
  if (nround > 0) start_round(0);
  wait_vmcnt<0>();
  __syncthreads();   // every wave's q rows are in LDS
  const float c2 = p.sm_scale * p.kv_scale * kLog2e;   // logit multiplier, log2 domain

  // QK reads: lane (m16, g) at k-step kb takes chunk 4 kb + g of row m16 of the
  // tile and of q (head m16).  Tile: byte 8192 (m16 >> 3) + 128 (m16 & 7) +
  // 1024 (kb >> 1) + 16 ((4 (kb & 1) + g) ^ kx(m16)), two lane bases by kb & 1;
  // q (row-major, key row_key(m16)): chunk 4kb + g at 4 (kb ^ (k >> 2)) +
  // (g ^ (k & 3)), four lane bases by kb mod 4
  int kq_base[2];
  {
    const int kx = (m16 >> 1) & 7;
#pragma unroll
    for (int b = 0; b < 2; ++b) kq_base[b] = 8192 * (m16 >> 3) + 128 * (m16 & 7) + 16 * ((4 * b + g) ^ kx);
  }
  int qk_base[4];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int k = row_key(m16);
    qk_base[r4] = m16 * G::MAIN + 64 * (r4 ^ (k >> 2)) + 16 * (g ^ (k & 3));
  }
  // PV (transposed reads): in k-slot group g, lane k = m16 reads row
  // r = 4g + (k >> 2), columns 128a + 32 (k & 3) + 4e .. +4, i.e. half e & 1 of
  // chunk 16a + 4 (k & 3) + (e >> 1), at byte 8192 (r >> 3) + 2048 a +
  // 1024 ((k >> 1) & 1) + 128 (r & 7) + 16 ((4 (k & 1) + (e >> 1)) ^ kx(r)) +
  // 8 (e & 1); lane (m16, g) then receives column 128a + 32 (m16 >> 2) + 4e +
  // (m16 & 3) of rows 4g .. 4g + 3, and the output lane (head, g) holds columns
  // 128a + 32g + 4e + i in O[a][e][i]
  int pvt_base[4];
  {
    const int r = 4 * g + (m16 >> 2);
    const int kx = (r >> 1) & 7;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      pvt_base[h] = 8192 * (r >> 3) + 1024 * ((m16 >> 1) & 1) + 128 * (r & 7) + 16 * ((4 * (m16 & 1) + h) ^ kx);
  }

  f32x4 O[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[a][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // reference max (log2 units), may lag the true max by kSlack
  float l_run = 0.0f;        // this lane's share of the denominator

  // ---- S^T[row][head] of the tile: lane (head m16, g) receives rows 4g .. 4g + 3;
  // fragments read DEPTH k-steps ahead, two partial sums (even / odd k-steps)
  constexpr int DEPTH = 3;
  float sv[4];
  float mt = -INFINITY;
  auto score = [&](uint32_t vm) {
    f32x4 ac[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 ra[DEPTH], rq[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      ra[d] = lds_read16(slot + kq_base[d & 1] + 1024 * (d >> 1));
      rq[d] = lds_read16(qs + qk_base[d & 3] + 256 * (d >> 2));
    }
#pragma unroll
    for (int kb = 0; kb < NKQ; ++kb) {
      const u32x4 a = ra[kb % DEPTH], b = rq[kb % DEPTH];
      if (kb + DEPTH < NKQ) {
        const int kn = kb + DEPTH;
        ra[kb % DEPTH] = lds_read16(slot + kq_base[kn & 1] + 1024 * (kn >> 1));
        rq[kb % DEPTH] = lds_read16(qs + qk_base[kn & 3] + 256 * (kn >> 2));
      }
      ac[kb & 1] = mfma_bf16(a, b, ac[kb & 1]);
    }
    // issue order: DEPTH k-steps of reads, then per k-step its MFMA and the two
    // reads of k-step kb + DEPTH
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * DEPTH, 0);
#pragma unroll
    for (int kb = 0; kb < NKQ; ++kb) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (kb + DEPTH < NKQ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    const f32x4 acc = ac[0] + ac[1];
    mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((vm >> (4 * g + i)) & 1u) ? acc[i] * c2 : -INFINITY;
      mt = fmaxf(mt, sv[i]);
    }
    mt = group4_max(mt);
  };

  // ---- P = exp2(s - m_run) and O^T[col][head] += V^T[col][row] P^T[row][head]
  auto accumulate = [&]() {
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    const float e0 = __builtin_amdgcn_exp2f(sv[0] - m_use);
    const float e1 = __builtin_amdgcn_exp2f(sv[1] - m_use);
    const float e2 = __builtin_amdgcn_exp2f(sv[2] - m_use);
    const float e3 = __builtin_amdgcn_exp2f(sv[3] - m_use);
    l_run += (e0 + e1) + (e2 + e3);
    const u32x2 pf = {pack_bf16(e0, e1), pack_bf16(e2, e3)};
    // quarter a + 1's transposed reads interleaved with quarter a's MFMAs
    u32x2 A[2][8];
    auto load_a = [&](int a) {
#pragma unroll
      for (int e = 0; e < 8; ++e) A[a & 1][e] = lds_read_tr16(slot + pvt_base[e >> 1] + 8 * (e & 1) + 2048 * a);
    };
    load_a(0);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a + 1 < 4) load_a(a + 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) O[a][e] = mfma_bf16_k16(A[a & 1][e], pf, O[a][e]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (a + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
  };

  // ---- the next tile goes into the slot once every read of this one is done;
  // then the ids of the tile after it are fetched (sid[0] moves on every 4 tiles)
  auto next = [&](int i) {
    wait_lgkmcnt0();
    if (i + 1 < nt) {
      vm_cur = issue(i + 1, cid);
      if (((i + 2) & 3) == 0) rotate();
      fetch(i + 2, cid);
    }
  };

  // ---- main loop, by rounds of up to RTILES tiles per wave.  m_run is a
  // reference max that may lag the true one by up to kSlack, so exponents stay
  // <= 2^kSlack; a head with no valid entry yet takes the tile's max (its O is
  // still zero).  Only when a head's scores outgrow a finite reference is O
  // rescaled (a uniform branch, rarely taken).
  for (int rd = 0; rd < nround;) {
    for (int i = 0; i < nt; ++i) {
      wait_vmcnt<0>();   // tile i's copies (the only vector memory operations in flight)
      score(vm_cur);
      if (__ballot(m_run != -INFINITY && mt > m_run + kSlack) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 8; ++e) O[a][e] *= alpha;
      }
      m_run = (m_run == -INFINITY) ? mt : m_run;
      accumulate();
      next(i);
    }
    if (++rd < nround) start_round(rd);
  }

  // ---- merge the four waves through LDS: (max, sum) of every wave, then two
  // rounds of two 128-column quarters: every wave writes its quarters 2r, 2r + 1,
  // and waves 2r, 2r + 1 combine quarter `wave` of all four and store it
  const float l_w = group4_sum(l_run);
  float* ob = reinterpret_cast<float*>(smem);
  float* s_m = ob + 4 * 16 * OP;
  float* s_l = s_m + 64;
  __syncthreads();   // every wave is done with its slot and with q
  if (g == 0) {
    s_m[16 * wave + m16] = m_run;
    s_l[16 * wave + m16] = l_w;
  }
  float f[4] = {0.f, 0.f, 0.f, 0.f};
  float scale = 0.0f, lse_nat = -INFINITY;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    {
      float* row = ob + (wave * 16 + m16) * OP;
#pragma unroll
      for (int qa = 0; qa < 2; ++qa)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<f32x4*>(row + 128 * qa + 32 * g + 4 * e) = O[2 * r + qa][e];
    }
    __syncthreads();
    if (r == 0) {
      // weights of the four waves for head m16
      float M = s_m[m16];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[16 * w + m16]);
      float Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[16 * w + m16] - M);
        Ls += f[w] * s_l[16 * w + m16];
      }
      const float2 nz = finish_row(M, Ls, sink_log2(p, head, true), p.kv_scale);
      scale = nz.x;
      lse_nat = nz.y;
    }
    if ((wave >> 1) == r) {
      const int qa = wave & 1;   // quarter `wave`, at column 128 qa of the buffer rows
      // 16 heads x 16 chunks of 8 columns, 4 per lane: store k takes head 4k + g,
      // columns 128 wave + 8 m16 .. + 8 (16 lanes write a head's 256 bytes);
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
          const float* src = ob + (w * 16 + hh) * OP + 128 * qa + 8 * m16;
          v0 += fk[w] * *reinterpret_cast<const f32x4*>(src);
          v1 += fk[w] * *reinterpret_cast<const f32x4*>(src + 4);
        }
        *reinterpret_cast<u32x4*>(p.out + ((int64_t)t * p.H + h0 + hh) * kDV + 128 * wave + 8 * m16) =
            u32x4{pack_bf16(v0[0] * sk, v0[1] * sk), pack_bf16(v0[2] * sk, v0[3] * sk),
                  pack_bf16(v1[0] * sk, v1[1] * sk), pack_bf16(v1[2] * sk, v1[3] * sk)};
      }
    }
    if (r == 0) __syncthreads();   // round 1 overwrites the buffer
  }
  if (wave == 0 && g == 0) p.lse[(int64_t)t * p.H + head] = lse_nat;
}

hipError_t launch_prefill(const FwdParams& p, dim3 grid, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipExtLaunchKernelGGL(smla_prefill_kernel, grid, dim3(kThreads), 0, stream, ev0, ev1, 0, p);
  return hipGetLastError();
}

}  // namespace smla
