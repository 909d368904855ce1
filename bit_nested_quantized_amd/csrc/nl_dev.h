// nl_dev.h -- device helpers shared by the gfx950 kernels of the nested linear:
// MFMA operand types, the workgroup Walsh-Hadamard transforms (POC recipe
// section 1 of the forum post "bit-nested"), activation loads, the
// agent-coherent hand-over primitives and the weight register sets.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nl_kernels.h"

#define NL_GLOBAL __attribute__((address_space(1)))
#define NL_LOCAL __attribute__((address_space(3)))
#define NL_CONST __attribute__((address_space(4)))

namespace nl {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8 as_half8(const uint32_t *p) {
  u32x4 v = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}


// Workgroup barrier for hand-offs through LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads (the release fence of
// __syncthreads would wait for every one of them, stalling the weight stream).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The barrier of the whole workgroup, as a policy of the transforms below.
struct WgBar {
  __device__ __forceinline__ void sync() { lds_barrier(); }
};

// A barrier among the 4 waves of one 256-thread group through an LDS counter
// (zero at the group's start), for transforms run by some waves while the
// others are held up issuing memory requests: an s_barrier would wait for
// those.  Each sync adds one per wave and waits for 4 more arrivals.
struct GroupBar {
  uint32_t addr;  // LDS byte address of the counter
  uint32_t n;     // arrivals expected by the next sync
  __device__ __forceinline__ void sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes have landed
    n += 4;
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_fetch_add((NL_LOCAL uint32_t *)(size_t)addr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (*(volatile NL_LOCAL uint32_t *)(size_t)addr < n) {
    }
    asm volatile("" ::: "memory");
  }
};

// Reductions over aligned groups of 32 and 8 lanes without an LDS round trip
// (a shuffle through ds_bpermute waits ~100 cycles per step): DPP moves for
// the steps within a row of 16 lanes (quad swaps for distances 1 and 2, the
// half-row mirror for 4, the row mirror for 8) and a bit-mode swizzle (xor
// 16) for the last step of 32.  After each step every lane of the group
// holds the same value, so pairing a lane with the mirrored lane of the
// other half gives what an xor butterfly gives, bit for bit.  Every lane of
// the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_lanes32(float m) {
  m = fmaxf(m, dpp_mov<0xB1>(m));   // quad_perm [1, 0, 3, 2]
  m = fmaxf(m, dpp_mov<0x4E>(m));   // quad_perm [2, 3, 0, 1]
  m = fmaxf(m, dpp_mov<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_mov<0x140>(m));  // row_mirror
  return fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, m), 0x401F)));
}
__device__ __forceinline__ float sum_lanes8(float s) {
  s += dpp_mov<0xB1>(s);
  s += dpp_mov<0x4E>(s);
  return s + dpp_mov<0x141>(s);
}

// ===========================================================================
// Workgroup Walsh-Hadamard transforms (POC section 1: Sylvester H, applied
// block-diagonally).  A workgroup of 256 threads transforms 4096 values:
// 4096/SB independent "tasks" of SB = 2^n values (n in 9..12), TPS = SB/16
// threads per task, 16 values per thread.  Butterflies run unnormalised over
// the low `lb` bits of the element index i (block 2^lb).  The 16 values of a
// thread pass through three layouts (the stages commute, so their order is
// free):
//   B  i = 16*lt + j           low 4 bits in registers; contiguous values
//                              (16-byte loads of x, 16-byte stores of x')
//   C  i = (lt&15) + 16*j + 256*(lt>>4)   bits 4..7 in registers
//   A  i = TPS*j + lt          top 4 bits in registers
// with padded LDS transposes B->C->A->B in between.
// ===========================================================================
__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 4); }

__device__ __forceinline__ void bfly16(float (&v)[16], int bit) {
  const int h = 1 << bit;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (!(j & h)) {
      const float x0 = v[j], x1 = v[j | h];
      v[j] = x0 + x1;
      v[j | h] = x0 - x1;
    }
}

// v: layout B on entry and on exit (thread lt of the task holds points
// 16*lt + j).  The transform is a butterfly on every index bit below LB;
// four bits are done in registers at a time, with LDS transposes
//   B (bits 0-3 in registers) -> C (bits 4-7) -> A (bits N-4..N-1, those
//   from 8 up) -> B.
// N = log2 of the task size SB, LB = log2 of the Hadamard block (LB <= N);
// both compile-time, so every LDS address is a base plus an immediate.
// xch: this task's LDS (SB + SB/16 floats).  idle: a thread (uniformly per
// wave) that only keeps the barrier count.
// Every LDS slot of a layout belongs to one thread, so a thread that writes
// back the slots it has just read (C -> C, A -> A) races with no other
// thread: only the barriers after each write, and the one that opens the
// task area, are needed.
constexpr int kFwhtBarriers = 4;
template <int N, int LB, class B>
__device__ __forceinline__ void fwht_bt(float (&v)[16], float *xch, int lt, bool idle, B &bar) {
  constexpr int TPS = 1 << (N - 4);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < LB) bfly16(v, q);
  const int cbase = (lt & 15) + 256 * (lt >> 4);
  float *pb = xch + lds_pad(16 * lt);             // B: + j
  float *pc = xch + lds_pad(cbase);               // C: + 17 j
  float *pa = xch + lt + (lt >> 4);               // A: + (TPS + TPS / 16) j
  bar.sync();
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) pb[j] = v[j];
  bar.sync();
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = pc[17 * j];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 + q < LB) bfly16(v, q);
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) pc[17 * j] = v[j];
  bar.sync();
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = pa[(TPS + TPS / 16) * j];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    constexpr int base = N - 4;
    if (base + q >= 8 && base + q < LB) bfly16(v, q);
  }
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) pa[(TPS + TPS / 16) * j] = v[j];
  bar.sync();
  if (!idle)
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = pb[j];
}

// The transform for a task of SB = max(2^lb, 512) points (one uniform
// dispatch on the block size; lb is 7..12 since d_in is a multiple of 128).
template <class B>
__device__ __forceinline__ void fwht_b(float (&v)[16], float *xch, int lt, int lb, bool idle, B &bar) {
  switch (lb) {
    case 7: fwht_bt<9, 7>(v, xch, lt, idle, bar); break;
    case 8: fwht_bt<9, 8>(v, xch, lt, idle, bar); break;
    case 9: fwht_bt<9, 9>(v, xch, lt, idle, bar); break;
    case 10: fwht_bt<10, 10>(v, xch, lt, idle, bar); break;
    case 11: fwht_bt<11, 11>(v, xch, lt, idle, bar); break;
    default: fwht_bt<12, 12>(v, xch, lt, idle, bar); break;
  }
}
__device__ __forceinline__ void fwht_b(float (&v)[16], float *xch, int lt, int lb, bool idle) {
  WgBar bar;
  fwht_b(v, xch, lt, lb, idle, bar);
}

// v: layout A on entry, layout B on exit (the output rotation, whose input
// loads are coalesced in layout A).
__device__ __forceinline__ void fwht_tasks(float (&v)[16], float *xch, int lt, int TPS, int n, int lb) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (n - 4 + q < lb) bfly16(v, q);
  lds_barrier();
#pragma unroll
  for (int j = 0; j < 16; ++j) xch[lds_pad(TPS * j + lt)] = v[j];
  lds_barrier();
  const int cbase = (lt & 15) + 256 * (lt >> 4);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = xch[lds_pad(cbase + 16 * j)];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 + q < n - 4 && 4 + q < lb) bfly16(v, q);
  // the slots this thread has just read: no barrier before the write-back
#pragma unroll
  for (int j = 0; j < 16; ++j) xch[lds_pad(cbase + 16 * j)] = v[j];
  lds_barrier();
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = xch[lds_pad(16 * lt + j)];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < lb) bfly16(v, q);
}

// 16 consecutive activations (columns k0 .. k0 + 15 of row xrow) and their
// signs: two 16-byte loads of x, one of the signs.  Rows of x and the sign
// vector are 16-byte aligned and d_in is a multiple of 128, so a group of 16
// is wholly inside or wholly past d_in.  Outside (xrow < 0 or k0 >= d_in)
// the loads read the first 16 columns and the values become zeros.
struct XRaw {
  u32x4 a, b, s;
  bool in;
};
__device__ __forceinline__ XRaw load_x16(const uint16_t *x, const int8_t *sign, int xrow, int k0, int d_in) {
  XRaw r;
  r.in = xrow >= 0 && k0 < d_in;
  const size_t off = r.in ? (size_t)xrow * d_in + k0 : 0;
  // global address space: a generic (flat) load would also count in lgkmcnt,
  // and waiting for it would wait for every load in flight
  const NL_GLOBAL u32x4 *xp = (const NL_GLOBAL u32x4 *)(x + off);
  const NL_GLOBAL u32x4 *sp = (const NL_GLOBAL u32x4 *)(sign + (r.in ? k0 : 0));
  r.a = xp[0];
  r.b = xp[1];
  r.s = sp[0];
  return r;
}
// x * sign in fp32 (exact: bf16 widens exactly, signs are +-1, i.e. bytes
// 0x01 / 0xFF, so the sign byte's top bit flips the sign bit), zero outside;
// bit operations only, no branches.
__device__ __forceinline__ void cvt_x16(float (&v)[16], const XRaw &r) {
  const uint32_t xw[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
  const uint32_t sw[4] = {r.s.x, r.s.y, r.s.z, r.s.w};
  const uint32_t keep = r.in ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t hb = (j & 1) ? (xw[j >> 1] & 0xFFFF0000u) : (xw[j >> 1] << 16);
    const uint32_t sbit = (sw[j >> 2] << (24 - 8 * (j & 3))) & 0x80000000u;
    v[j] = __uint_as_float((hb ^ sbit) & keep);
  }
}

// Column offset, inside its 128-column group, of run r (0..15) of the
// contraction's activation layout: run = step * 4 + quarter holds the 8
// columns 32 * quarter + 8 * step .. + 8 (the MFMA A operand of lanes with
// l >> 4 == quarter at step `step`).
__device__ __forceinline__ int run_col(int r) { return 32 * (r & 3) + 8 * (r >> 2); }

// ===========================================================================
// Hand-over between the workgroups of one launch.  Data written by one
// workgroup and read by another (on any XCD) goes through agent-scope (sc1)
// stores and loads, and a counter is bumped only after the writer's stores
// are acknowledged (s_waitcnt vmcnt(0) in every thread, then a barrier), so
// no L2 write-back or invalidate is needed.  Counters are 64-byte apart; the
// launch leaves every counter at zero.
// ===========================================================================
constexpr int kSc1 = 16;  // cache policy of a buffer op: agent-coherent (sc1), as st_dev
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_add(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t *ctr_at(uint32_t *c, int i) { return c + kCtrStride * i; }

// Wait until at most n of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BITS>
struct WRegs {
  u32x4 b[kBasePieces];
  u32x4 r[BITS > 0 ? BITS : 1];
  uint64_t sb, sr;  // the row's 4 group scales (fp16) of each plane
};

// An ordered no-op on every register of a set: work on the set cannot be
// scheduled above it, so the wait for the set's loads lands here.
template <int BITS>
__device__ __forceinline__ void pin(WRegs<BITS> &w) {
#pragma unroll
  for (int i = 0; i < kBasePieces; ++i) asm volatile("" : "+v"(w.b[i]));
  asm volatile("" : "+v"(w.sb));
  if constexpr (BITS > 0) {
#pragma unroll
    for (int i = 0; i < BITS; ++i) asm volatile("" : "+v"(w.r[i]));
    asm volatile("" : "+v"(w.sr));
  }
}

// A wave-uniform pointer in an SGPR pair (the copies' scalar base operand).
__device__ __forceinline__ const void *sgpr_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The split-K sums of a row block, taken by its last workgroup to arrive:
//   out[(tb + t) * ld + r0 + r] = sum_s part[s * stride + (tb + t) * ld + r0 + r]
// for t < nt, r < rows, each output summed in split order from zero (the same
// order and rounding on every path).  The partials were written by other
// workgroups with agent-scope stores and are read with agent-scope loads.
// When ld, stride, r0 and rows are multiples of 4 (partials 16-byte aligned)
// a thread takes U runs of 4 rows and issues the 16-byte loads of up to 8
// splits of all of them before its first add, so a row block of 64 tokens
// costs one or two memory round trips per 8 splits (U = 2 or 4; U = 0 keeps
// only the single-output form); otherwise 4 single outputs per thread and
// round.
// RBC > 0: the row block's height as a constant (rows <= RBC), so that the
// output index splits by a constant divisor.
// out_tb: the output's row of token 0 (tb, or 0 for an output of the row
// block's own).
template <int NT, int U, int RBC = 0>
__device__ __forceinline__ void sum_splits(const float *part, size_t stride, int S, float *out, bool coh, size_t ld,
                                           int tb, int nt, int r0, int rows, int out_tb) {
  const size_t shift = (size_t)(tb - out_tb) * ld;  // output index = partial index - shift
  const int rstep = RBC > 0 ? RBC : rows;  // outputs of one token in the index space
  const size_t span = (size_t)S * stride * 4;
  const bool vec = U > 0 && ((ld | stride | (size_t)r0 | (size_t)rows) & 3) == 0 && ((uintptr_t)part & 15) == 0 &&
                   span < 0x7FFFFFFFu;
  if constexpr (U > 0) if (vec) {
    constexpr int kRaw = 0x00020000;  // raw 32-bit buffer descriptor word 3
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc((void *)sgpr_ptr(part), 0, (int)span, kRaw);
    const int rq = rstep >> 2, total = nt * rq;
    for (int base = 0; base < total; base += U * NT) {
      // o: float index (within one split) of the thread's run u, or ~0 when
      // it has none (its loads then read the first run; nothing is stored)
      uint32_t o[U];
      floatx4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * NT + (int)threadIdx.x, t = idx / rq, r4 = idx - t * rq;
        o[u] = idx < total && 4 * r4 < rows ? (uint32_t)((size_t)(tb + t) * ld + r0 + 4 * r4) : ~0u;
        v[u] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      for (int s0 = 0; s0 < S; s0 += 8) {
        floatx4 w[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[u][q] = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                             pr, (int)(((uint32_t)min(s0 + q, S - 1) * (uint32_t)stride + (o[u] == ~0u ? 0u : o[u])) * 4u),
                             0, kSc1));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < 8; ++q)
            v[u] += (s0 + q < S) ? w[u][q] : floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (o[u] != ~0u) {
          float *p = out + (o[u] - shift);
          if (coh) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st_dev(p + i, v[u][i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = v[u][i];
          }
        }
      }
    }
    return;
  }
  const int total = nt * rstep;
  for (int base = 0; base < total; base += 4 * NT) {
    size_t o[4];
    bool ok[4];
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int idx = base + e4 * NT + (int)threadIdx.x, t = idx / rstep, r = idx % rstep;
      ok[e4] = idx < total && r < rows;
      o[e4] = ok[e4] ? (size_t)(tb + t) * ld + r0 + r : 0;
    }
    for (int s0 = 0; s0 < S; s0 += 8) {
      float u[4][8];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
        for (int q = 0; q < 8; ++q) u[e4][q] = ld_dev(part + (size_t)min(s0 + q, S - 1) * stride + o[e4]);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
        for (int q = 0; q < 8; ++q) v[e4] += (s0 + q < S) ? u[e4][q] : 0.f;
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      if (!ok[e4]) continue;
      if (coh) st_dev(out + (o[e4] - shift), v[e4]); else out[o[e4] - shift] = v[e4];
    }
  }
}

}  // namespace nl
