// smla_prefill.hip -- 16-head groups on whole long lists (prefill) of bf16 rows
// 512 wide.
//
// Each wave streams its own 16-row tiles (tiles wave, wave + 4, ...) through a
// private LDS slot, with no barrier in the loop, as the 16-head kernel of
// smla_kernels.hip does; the difference is how rows reach LDS.  Every row is
// copied from the pool straight into the slot by one global_load_lds_dwordx4
// (64 lanes x 16 bytes, its 16-byte chunks permuted by the row number through
// the lane offsets), with the slot ids of a tile coming in by one scalar
// buffer load, so a tile in flight holds no registers and needs no ds_write.
// That frees enough registers for two workgroups per compute unit (two waves
// per SIMD): while one wave waits for its next tile, the other computes.  LDS
// per workgroup is exactly 80 KiB: four 16 KiB slots and q (16 rows of 1 KiB,
// read by all four waves as the B operand of QK^T).
//
// Per tile: QK^T on 16x16x32 bf16 MFMAs (S^T[row][head], fragments read three
// k-steps ahead), the online softmax with a lazily moved reference max, and PV
// on 16x16x16 bf16 MFMAs with V through transposed LDS reads.  At the end the
// four waves merge (max, sum, O) through LDS in two rounds of two 128-column
// quarters and store out / lse (the kernel runs whole lists only: no split).
#include <hip/hip_ext.h>

#include "smla_common.h"

namespace smla {

__global__ __launch_bounds__(kThreads, 2) void smla_prefill_kernel(FwdParams p) {
  using G = Geom<false, 512>;
  constexpr int TR = 16;                       // rows per tile
  constexpr int SLOT = TR * G::MAIN;           // 16 KiB
  constexpr int QOFF = 4 * SLOT;               // q: 16 rows of 1 KiB
  constexpr int LDS = QOFF + 16 * G::MAIN;     // 80 KiB: two workgroups per compute unit
  constexpr int NKQ = 16;                      // QK k-steps (32 columns each)
  constexpr int OP = 256 + 4;                  // merge row: two quarters of fp32, padded
  static_assert(4 * 16 * OP * 4 + 2 * 64 * 4 <= LDS, "merge buffer fits");

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
  const int kbeg = wu.kbeg;
  const int kend = wu.kend;
  const int ntile = kend > kbeg ? (kend - kbeg + TR - 1) / TR : 0;
  const int nt = ntile > wave ? (ntile - wave + 3) / 4 : 0;   // this wave's tiles: wave + 4i
  const int head = h0 + m16;

  uint8_t* slot = smem + wave * SLOT;
  const uint32_t slot_lds = lds_addr(slot);
  const uint8_t* qs = smem + QOFF;

  // ---- slot ids of this wave's tile i (16 entries) through the scalar unit
  const i32x4 ids_rsrc = scalar_rsrc(p.idx + (int64_t)t * p.idx_st + kbeg, 4 * (kend - kbeg));
  auto load_ids = [&](int i) -> i32x16 { return sbuf_load_x16(ids_rsrc, 4 * TR * (wave + 4 * i), 0); };
  // a slot id is valid when 0 <= id < N: one unsigned compare against min(N, 2^31)
  const uint32_t n_lim = (uint32_t)min(p.N, (int64_t)0x80000000LL);
  const uint8_t* zero_row = g_zero_row;
  // 16 copies: row r of tile i into slot row r, lane l fetching chunk l ^ row_key(r);
  // returns the validity bits of the tile's rows
  const uint32_t lane16 = 16 * lane;
  auto issue = [&](int i, const i32x16& ids) -> uint32_t {
    const int k0 = kbeg + TR * (wave + 4 * i);
    uint32_t vm = 0;
    static_for<0, TR>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const bool ok = (uint32_t)ids[r] < n_lim && k0 + r < kend;
      vm |= ok ? (1u << r) : 0u;
      const uint8_t* b = ok ? p.kv + (uint64_t)(uint32_t)ids[r] * G::ROW : zero_row;
      copy_sx<16 * row_key(r)>(b, lane16, slot_lds + r * G::MAIN);
    });
    return vm;
  };

  // ---- q: wave w copies heads 4w .. 4w + 3 (row h, chunk c at c ^ row_key(h)),
  // then the first tile; q has landed once only the tile's copies are outstanding
  {
    const uint8_t* qtok = reinterpret_cast<const uint8_t*>(p.q + (int64_t)t * p.q_st);
    // rows 4w + i have keys ((i & 1) << 3) | (2w + (i >> 1)): the wave's part as a scalar
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * wave + i;
      copy_s(qtok + (int64_t)(h0 + hh) * p.q_sh * 2, lane16 ^ (16 * row_key(hh)), lds_addr(qs) + hh * G::MAIN);
    }
  }
  i32x16 ids = load_ids(0);
  uint32_t vm_cur = 0;
  if (nt > 0) {
    vm_cur = issue(0, ids);
    wait_vmcnt<TR>();
  } else {
    wait_vmcnt<0>();
  }
  ids = load_ids(1);
  __syncthreads();   // every wave's q rows are in LDS
  const float c2 = p.sm_scale * p.kv_scale * kLog2e;   // logit multiplier, log2 domain

  // QK reads: row m16 (key k = row_key(m16)), chunk 4kb + g lands at
  // 4 (kb ^ (k >> 2)) + (g ^ (k & 3)): one lane base per kb mod 4, the same
  // for the K rows of the slot and the q rows (head m16)
  int qk_base[4];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int k = row_key(m16);
    qk_base[r4] = m16 * G::MAIN + 64 * (r4 ^ (k >> 2)) + 16 * (g ^ (k & 3));
  }
  // PV (transposed reads): in k-slot group g, lane k = m16 reads row
  // 4g + (k >> 2), columns 128a + 32 (k & 3) + 4e .. +4, i.e. half e & 1 of
  // chunk 16a + 4 (k & 3) + (e >> 1); lane (m16, g) then receives column
  // 128a + 32 (m16 >> 2) + 4e + (m16 & 3) of rows 4g .. 4g + 3, and the output
  // lane (head, g) holds columns 128a + 32g + 4e + i in O[a][e][i]
  int pvt_base[4];
  {
    const int r = 4 * g + (m16 >> 2);
#pragma unroll
    for (int h = 0; h < 4; ++h) pvt_base[h] = r * G::MAIN + 16 * ((4 * (m16 & 3) + h) ^ row_key(r));
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
      ra[d] = lds_read16(slot + qk_base[d & 3] + 256 * (d >> 2));
      rq[d] = lds_read16(qs + qk_base[d & 3] + 256 * (d >> 2));
    }
#pragma unroll
    for (int kb = 0; kb < NKQ; ++kb) {
      const u32x4 a = ra[kb % DEPTH], b = rq[kb % DEPTH];
      if (kb + DEPTH < NKQ) {
        const int kn = kb + DEPTH;
        ra[kb % DEPTH] = lds_read16(slot + qk_base[kn & 3] + 256 * (kn >> 2));
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
      for (int e = 0; e < 8; ++e) A[a & 1][e] = lds_read_tr16(slot + pvt_base[e >> 1] + 8 * (e & 1) + 256 * a);
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

  // ---- the next tile goes into the slot once every read of this one is done
  auto next = [&](int i) {
    wait_lgkmcnt0();
    if (i + 1 < nt) {
      vm_cur = issue(i + 1, ids);
      ids = load_ids(i + 2);
    }
  };

  // ---- main loop.  m_run is a reference max that may lag the true one by up
  // to kSlack, so exponents stay <= 2^kSlack; a head with no valid entry yet
  // takes the tile's max (its O is still zero).  Only when a head's scores
  // outgrow a finite reference is O rescaled (a uniform branch, rarely taken).
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
