// smla_common.h -- device helpers shared by the forward kernels of libsparsemla:
// the split-partial format, work units, the final normalisation, pool row
// addresses, tile geometry and LDS access helpers.
#pragma once

#include <type_traits>

#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

// Split partials are chunks of 4 columns; chunk c (columns 4c .. 4c+3) of the
// 16 heads of a group sit side by side, so the 16 lanes that hold one chunk of
// 16 consecutive heads store contiguous bytes.  Index in chunks (8 bytes).
// Partial row pr holds one unit's partials (uniform plan: pr = s T + t).
__device__ __forceinline__ int64_t part_chunk(const FwdParams& p, int64_t pr, int head, int c) {
  return (pr * p.H + (head & ~15)) * (kDV / 4) + 16 * c + (head & 15);
}

// A chunk is stored as four fp16 numbers against a power-of-two scale 2^e per
// (partial row, head, 128-column quarter), e the binary exponent of the
// quarter's largest magnitude: every stored number lies in (-2, 2), so it keeps
// 11 significant bits relative to that largest value, over fp32's whole
// exponent range, in half the bytes of fp32.  Zero and subnormal maxima take
// e = -126; inf / nan take e = 0 and are stored as they are.
__device__ __forceinline__ int part_exp(float amax) {
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xff);
  return eb == 0xff ? 0 : max(eb, 1) - 127;
}
// the largest magnitude over the four lanes m16 + 16 g that hold one quarter
__device__ __forceinline__ float quarter_max(float a) {
  a = fmaxf(a, __shfl_xor(a, 16));
  return fmaxf(a, __shfl_xor(a, 32));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;   // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ u32x2 part_encode(const f32x4& v, int e) {
  return u32x2{pack_f16(ldexpf(v[0], -e), ldexpf(v[1], -e)), pack_f16(ldexpf(v[2], -e), ldexpf(v[3], -e))};
}
__device__ __forceinline__ f32x4 part_decode(const u32x2& w) {
  return f32x4{(float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xffffu)),
               (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16)),
               (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xffffu)),
               (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16))};
}
// Partial rows are written through to memory (device-scope relaxed atomic
// stores: the L2 does not keep them dirty).  They are read only by the merge
// kernel that follows, so the L2 write-back at the end of the forward kernel
// has nothing of them left to write: 1.6 - 1.9 % less time per call than
// write-back stores in every split decode workload.
__device__ __forceinline__ void part_store(u32x2* dst, const u32x2& w) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), (uint64_t)w[0] | ((uint64_t)w[1] << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void part_store_f32(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void part_store_scale(const FwdParams& p, int64_t pr, int head, int quarter, int e) {
  part_store_f32(p.part_scale + (pr * p.H + head) * 4 + quarter, ldexpf(1.0f, e));
}

// A workgroup's unit of work: token t, entries [kbeg, kend) of its list, the
// partial row of its result, and whether it is the token's only unit (then it
// writes out / lse itself).  Uniform plan: S splits of rps entries per token;
// per-token plan: a table the planner wrote.  False past the last unit.
// The kernels decode (t, kbeg, kend) at entry and (prow, direct) only in the
// epilogue, so the second pair is not held through the main loop.
struct Unit {
  int t, kbeg, kend;
};
__device__ __forceinline__ bool unit_of(const FwdParams& p, int u, Unit& w) {
  if (p.units == nullptr) {
    if (u >= p.T * p.S) return false;
    w.t = u / p.S;
    const int s = u - w.t * p.S;
    w.kbeg = s * p.rps;
    w.kend = min(w.kbeg + p.rps, p.K);
    return true;
  }
  // the table entries are workgroup-uniform: keep them in scalar registers
  if (u >= __builtin_amdgcn_readfirstlane(*p.num_units)) return false;
  const int4 e = p.units[u];
  w.t = __builtin_amdgcn_readfirstlane(e.x);
  w.kbeg = __builtin_amdgcn_readfirstlane(e.y);
  w.kend = __builtin_amdgcn_readfirstlane(e.z);
  return true;
}
struct UnitTail {
  int prow;
  bool direct;
};
__device__ __forceinline__ UnitTail unit_tail(const FwdParams& p, int u) {
  if (p.units == nullptr) {
    const int t = u / p.S;
    return UnitTail{(u - t * p.S) * p.T + t, p.S == 1};
  }
  const int pr = __builtin_amdgcn_readfirstlane(__atomic_load_n(&p.units[u].w, __ATOMIC_RELAXED));
  return UnitTail{pr, pr < 0};   // a token's only unit has no partial row
}

// Sink logit of a head in log2 units; only a unit that writes out itself takes
// it (with splits the combine does).  -inf = no sink.
__device__ __forceinline__ float sink_log2(const FwdParams& p, int head, bool direct) {
  return (direct && p.sinks != nullptr) ? p.sinks[head] * kLog2e : -INFINITY;
}

// Final normalisation of one (token, head): m = the running max and l = the
// sum of exp2(s - m) over the valid entries (log2 units; m = -inf if there is
// none), s2 = the sink logit (log2 units, -inf = none), which joins the
// normaliser as a key whose value row is zero.  Returns {multiplier of the
// accumulated O, including kv_scale; natural-log lse}; {0, -inf} when there
// is neither a valid entry nor a sink.
__device__ __forceinline__ float2 finish_row(float m, float l, float s2, float kv_scale) {
  const float M = fmaxf(m, s2);
  if (M == -INFINITY) return float2{0.0f, -INFINITY};
  const float a = __builtin_amdgcn_exp2f(m - M);   // 1 without a sink, 0 without entries
  const float L = l * a + __builtin_amdgcn_exp2f(s2 - M);
  return float2{kv_scale * a / L, (M + __builtin_amdgcn_logf(L)) * kLn2};
}

// Stand-in for the rows of invalid top-k entries: all zero, never written (one
// copy per translation unit).
static __device__ __attribute__((aligned(16))) uint8_t g_zero_row[2048];

// Address of pool row `rec` (rec < 0: the zero row).  The byte offset is
// formed in 64 bits: a structured buffer (record index x stride) wraps its
// offset at 2^32 bytes, which would silently gather the wrong rows of a pool
// larger than 4 GiB.
__device__ __forceinline__ const uint8_t* pool_row(const uint8_t* kv, int rec, int row_bytes) {
  return rec >= 0 ? kv + (int64_t)rec * row_bytes : g_zero_row;
}
__device__ __forceinline__ u32x4 load16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

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
// ds_read_b64_tr_b16: within each group of 16 lanes, lane k reads 4 consecutive
// 16-bit values D_k[0..3] at its address, and lane 4a + b receives
// D_{a + 4j}[b] for j = 0..3 (a 16 x 4 block read row-wise, delivered
// column-wise).  With lane k of a group reading row k / 4 of a 4-row block at
// column offset c_{k % 4}, lane i gets column c_{i / 4} + i % 4 of all 4 rows:
// the k-major MFMA operand of a row-major tile.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_read8(const uint8_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Slot ids of an n-row tile: lane j (j < n) loads entry k0 + j of the list,
// -1 past the end of the split.  One vector load per tile, issued ahead of use.
template <int n = 16>
__device__ __forceinline__ int load_tile_idx(const int32_t* idx_t, int k0, int kend, int lane) {
  const int k = k0 + (lane & (n - 1));
  return (lane < n && k < kend) ? idx_t[k] : -1;
}

// Row addresses of that tile (wave-uniform): invalid entries (padding, out of
// range) point at the zero row instead of the pool.  Returns the validity mask.
template <int ROW, int n = 16>
__device__ __forceinline__ uint32_t tile_rows(int vidx, const uint8_t* kv, int64_t N,
                                              const uint8_t* zero_row, const uint8_t* (&rp)[n]) {
  uint32_t vm = 0;
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const int sl = __builtin_amdgcn_readlane(vidx, j);
    const bool ok = sl >= 0 && (int64_t)sl < N;
    rp[j] = ok ? kv + (int64_t)sl * ROW : zero_row;
    vm |= ok ? (1u << j) : 0u;
  }
  return vm;
}


constexpr float kSlack = 8.0f;   // log2 headroom of the lazily rescaled running max

// Swizzle key of a tile row: the 16-byte chunk c of row r sits at chunk
// position c ^ row_key(r).  row_key is a bijection on r mod 16 (so 16
// consecutive rows read at one chunk, and one row read across 16 chunks, hit
// 16 different chunk positions) and rows 2j, 2j + 1 differ in bit 3 of it, so
// the two rows a 16-lane quarter of a commit store writes side by side fall in
// different halves of the bank space.
__host__ __device__ constexpr int row_key(int r) { return ((r & 1) << 3) | ((r >> 1) & 7); }

// ---- scalar id loads, hand-counted LDS copies ---------------------------------------
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
typedef __attribute__((ext_vector_type(16))) int32_t i32x16;

// s_buffer_load_dwordx8 / x16: scalar loads through a buffer descriptor
// (dwords past num_records read 0); they use no vector memory counter.
__device__ i32x8 sbuf_load_x8(i32x4 rsrc, int offset, int cachepolicy) __asm("llvm.amdgcn.s.buffer.load.v8i32");
__device__ i32x16 sbuf_load_x16(i32x4 rsrc, int offset, int cachepolicy) __asm("llvm.amdgcn.s.buffer.load.v16i32");

// buffer descriptor over `bytes` bytes at p (wave-uniform)
__device__ __forceinline__ i32x4 scalar_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kBufferRsrcWord3;
  return r;
}

// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until this wave's LDS (and scalar memory) operations have completed
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// global_load_lds_dwordx4: 64 lanes x 16 bytes from global memory into 1 KiB
// of LDS at `lds` (wave-uniform; lane l's bytes land at lds + 16 l), with no
// register result.  Written as asm: the compiler would otherwise wait for
// every such copy (vmcnt(0)) before any LDS read it cannot prove disjoint,
// which drains a pipeline of copies; kernels that use these wait for them
// themselves (wait_vmcnt with the number of copies issued after the ones
// needed).  M0 carries the LDS address (one wait state after writing it).
// Kernels using them index no register array dynamically (M0 is theirs).
// scalar row base + per-lane byte offset
__device__ __forceinline__ void copy_s(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
// scalar row base + lane offset lane16 ^ KEY16 (lane16 = 16 * lane): the
// offset is formed inside the copy, so no register holds it between copies
template <uint32_t KEY16>
__device__ __forceinline__ void copy_sx(const uint8_t* base, uint32_t lane16, uint32_t lds) {
  uint32_t off;
  asm volatile("v_xor_b32 %0, %1, %2\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4"
               : "=&v"(off)
               : "i"(KEY16), "v"(lane16), "s"(lds), "s"(base)
               : "memory", "m0");
}
// compile-time loop: f(std::integral_constant<int, I>) for I in [B, E)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
// per-lane 64-bit address
__device__ __forceinline__ void copy_v(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

}  // namespace smla
