// nl_w4w8.hip -- the BitNest W4/W8 dual-plane linear (include/nested_w4w8.h).
//
// One launch per call.  A workgroup (8 waves) owns 128 rows and one K-split
// of whole 128-column groups (about one workgroup per CU), or, for small
// T * d_in, 16, 32 or 64 rows and the whole K-range (see w48_kernel):
//   * it converts its K-range of x into LDS as fp16 (the T real tokens only,
//     in pieces when the range does not fit), each (token, group)
//     scaled by a power of two that puts its largest magnitude in
//     [2^14, 2^15) (bf16 -> fp16 is then exact), with the inverse scale and
//     the group's sum of x' beside it (a separate conversion launch cost
//     more than the repeated conversion: x is small and stays in L2);
//   * each wave streams its 16-row tile's planes through a ring of register
//     sets: per group and lane 16 bytes of the base plane (32 nibbles: the
//     lane's 32 columns), 16 of the refinement plane (verify) and the row's
//     fp16 scale.  Create repacks the canonical planes tile-major: block
//     (tile, group) holds lane l's 16 bytes at l * 16, so a wave reads one
//     contiguous 1 KiB per plane and group, and its tile is one contiguous
//     range (read straight from the row-major planes, a wave touched 16
//     rows 2-7 KiB apart per load and HBM ran at a tenth of its rate);
//   * the nibbles become the MFMA B operand as fp16 1024 + u, u the offset
//     code (q4 + 8 for the draft, 16 (q4 + 8) + (q_r + 8) = 136 + 16 q4 + q_r
//     for verify, so one v_mfma_f32_16x16x32_f16 per 32 columns and 16 tokens
//     serves both); the group's fp32 result minus bias * sum(x') times
//     scale * inverse x scale goes into the row's accumulators;
//   * with several splits, partials go to the workspace and the row block's
//     last workgroup (ticket) adds them in split order.
// Lane l holds row (l & 15) and the group's columns 32 (l >> 4) .. +32; MFMA
// step s feeds columns 8s .. 8s + 7 of that run, on both operands.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_set>

#include "../../include/nested_w4w8.h"

namespace nl {
nl_status api_error(nl_status st, const char *msg);  // nl_api.hip
}

struct nl_w4w8 {
  uint32_t magic;
  int d_out, d_in, rows_pad, G;
  bool has_ref;
  uint8_t *base;
  uint8_t *ref;
  uint16_t *scales;
};

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic = 0x4E573438u;  // "NW48"
constexpr int kGroup = 128;
constexpr int kRows = 128;      // rows per workgroup: 8 waves x 16
constexpr int kThreads = 512;
// Groups in flight per wave: 6, or 4 for verify with two token tiles (there
// the x conversion's registers and the accumulators leave no room for more
// within 128 VGPRs).
template <bool VERIFY, int MT>
constexpr int ring_depth() { return VERIFY && MT == 2 ? 4 : 6; }
// Dynamic LDS budget for x' and its metadata, and the workgroups resident
// per CU: two of 60 KiB up to two token tiles, one of 120 KiB beyond.
constexpr int lds_budget(int mt) { return mt <= 2 ? 60 * 1024 : 120 * 1024; }
constexpr int kCus = 256;

struct W48Args {
  const uint8_t *base;
  const uint8_t *ref;
  const uint16_t *scales;
  const uint16_t *x;      // [T][d_in] bf16
  float *y;
  float *part;            // [S][T][rows_pad]
  uint32_t *tick;         // [rows_pad / kRows]
  int d_out, d_in, rows_pad, G, T, S, gps, pg, pitch;
};

__device__ __forceinline__ float h2f(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

// Split-K hand-over without fences (an agent-scope fence writes back the
// whole L2): partials go out as agent-scope (sc1) stores, every thread waits
// until its stores are acknowledged, and only then is the ticket taken; the
// last workgroup reads them with agent-scope loads.
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
constexpr int kSc1 = 16;  // cache policy of a buffer load: agent-coherent (sc1), as ld_agent

// Max and sum over an aligned row of 16 lanes by DPP moves (quad swaps for
// distances 1 and 2, the half-row mirror for 4, the row mirror for 8; a
// shuffle through LDS waits ~100 cycles per step).  After each step the
// lanes of a group hold equal values, so the result is an xor butterfly's,
// bit for bit.  All 16 lanes of the row must be active.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, dpp<0xB1>(m));
  m = fmaxf(m, dpp<0x4E>(m));
  m = fmaxf(m, dpp<0x141>(m));
  return fmaxf(m, dpp<0x140>(m));
}
__device__ __forceinline__ float row16_sum(float s) {
  s += dpp<0xB1>(s);
  s += dpp<0x4E>(s);
  s += dpp<0x141>(s);
  return s + dpp<0x140>(s);
}

// Four fp16 pairs 1024 + u from one dword of each plane (8 columns).
// lo/hi: per byte j, the offset code of column 2j / 2j + 1.
__device__ __forceinline__ void pairs(uint32_t lo, uint32_t hi, uint32_t *out) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    out[j] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * j) | 0x64006400u;
}

template <bool VERIFY>
__device__ __forceinline__ void unpack(const uint4 &b, const uint4 &r, uint32_t (&B)[4][4]) {
  const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
  const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t xb = bw[s] ^ 0x88888888u;  // two's complement -> offset nibbles
    if constexpr (VERIFY) {
      const uint32_t xr = rw[s] ^ 0x88888888u;
      const uint32_t even = ((xb << 4) & 0xF0F0F0F0u) | (xr & 0x0F0F0F0Fu);
      const uint32_t odd = (xb & 0xF0F0F0F0u) | ((xr >> 4) & 0x0F0F0F0Fu);
      pairs(even, odd, B[s]);
    } else {
      pairs(xb & 0x0F0F0F0Fu, (xb >> 4) & 0x0F0F0F0Fu, B[s]);
    }
  }
}

// RT: row tiles per workgroup.  RT = 8: each wave owns one 16-row tile of a
// 128-row block over the split's groups.  RT < 8 (one token tile, the whole
// K-range in the workgroup): the 8 / RT waves of a tile take every
// (8 / RT)-th group and add their accumulators through LDS, so no split-K
// hand-over is needed.
template <bool VERIFY, int MT, int RT>
// Two workgroups per CU (4 waves per SIMD, <= 128 VGPRs) up to two token
// tiles; with three or four the accumulators need more registers and one
// workgroup per CU runs.
__global__ __launch_bounds__(kThreads, MT <= 2 ? 4 : 2) void w48_kernel(W48Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int T16 = MT * 16;
  constexpr float kBias = VERIFY ? 1160.0f : 1032.0f;
  constexpr int kRing = ring_depth<VERIFY, MT>();
  constexpr int KW = 8 / RT, RB = 16 * RT;   // waves per tile, rows per block
  _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
  // x' holds the T real tokens only; meta (inverse scale, bias * sum) all
  // T16 tokens of the tiles, zero past T
  float2 *meta = reinterpret_cast<float2 *>(smem + (size_t)a.T * a.pitch * 2);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int rb = blockIdx.x / a.S, sp = blockIdx.x - rb * a.S;
  const int g0 = sp * a.gps;
  const int ng = min(a.G, g0 + a.gps) - g0;
  const int tl = wave % RT, ks = wave / RT;   // the wave's tile and K share
  const int row = rb * RB + tl * 16 + (lane & 15);
  const int kb = lane >> 4;
  const size_t tile = (size_t)rb * RT + tl;
  // the wave's groups: split group ks + KW j for j < nwg; gidx(j) the group
  // a load names (clamped into the split)
  const int nwg = KW == 1 ? ng : ng > ks ? (ng - ks + KW - 1) / KW : 0;
  const int nwc = max(nwg, 1) - 1;
  auto gidx = [&](int j) {
    if constexpr (KW == 1) return g0 + min(j, ng - 1);
    else return g0 + min(ks + KW * min(j, nwc), ng - 1);
  };
  const uint8_t *bp = a.base + tile * a.G * 1024 + lane * 16;            // + g * 1024
  const uint8_t *rp = VERIFY ? a.ref + tile * a.G * 1024 + lane * 16 : nullptr;
  const uint16_t *sc = a.scales + tile * a.G * 16 + (lane & 15);          // + g * 16

  // The ring's loads are unconditional (group index clamped into the split)
  // so the compiler can count them and wait for one set at a time; slots
  // past the split's last group repeat it and are weighted 0.
  uint4 wb[kRing], wr[kRing];
  uint16_t ws[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    const int g = gidx(i);
    wb[i] = *reinterpret_cast<const uint4 *>(bp + (size_t)g * 1024);
    if constexpr (VERIFY) wr[i] = *reinterpret_cast<const uint4 *>(rp + (size_t)g * 1024);
    ws[i] = sc[(size_t)g * 16];
  }

  // x -> x' in LDS, one piece of the split's groups at a time (groups p0 ..
  // p0 + pg - 1; pg = the whole split when it fits).  Item = (token, group,
  // 16-byte run); the 16 lanes of a (token, group) are consecutive and
  // 16-aligned, so its max and sum are exchanges within a row of 16 lanes.
  // Four loads in flight per thread, or eight from three token tiles on;
  // items past the end reload the last one (in bounds) and are not staged.
  constexpr int kStage = MT >= 3 ? 8 : 4;
  auto stage = [&](int p0) {
    const int npc = min(a.pg, ng - p0), runs = npc * 16, items = a.T * runs;
    const uint16_t *xg = a.x + (size_t)(g0 + p0) * kGroup;
    for (int it0 = t; it0 < items; it0 += kStage * kThreads) {
      uint4 v[kStage];
#pragma unroll
      for (int j = 0; j < kStage; ++j) {
        const int it = min(it0 + j * kThreads, items - 1);
        const int tt = it / runs, pc = it - tt * runs;
        v[j] = *reinterpret_cast<const uint4 *>(xg + (size_t)tt * a.d_in + pc * 8);
      }
#pragma unroll
      for (int j = 0; j < kStage; ++j) {
        const int it = it0 + j * kThreads;
        if (it < items) {
          const int tt = it / runs, pc = it - tt * runs, gi = pc >> 4, p = pc & 15;
          const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
          float f[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(w[q] << 16);
            f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
          }
          float m = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(f[q]));
          m = row16_max(m);   // the item's 16 lanes are one aligned row, all active
          int e = 0;
          if (m > 0.0f) {
            int E;
            frexpf(m, &E);
            e = 15 - E;   // m * 2^e in [2^14, 2^15)
          }
          half8 h;
          float gs = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            h[q] = (_Float16)ldexpf(f[q], e);
            gs += (float)h[q];
          }
          gs = row16_sum(gs);
          *reinterpret_cast<half8 *>(xs + (size_t)tt * a.pitch + pc * 8) = h;
          if (p == 0) meta[gi * T16 + tt] = make_float2(ldexpf(1.0f, -e), kBias * gs);
        }
      }
    }
    for (int i = t; i < npc * (T16 - a.T); i += kThreads) {
      const int gi = i / (T16 - a.T);
      meta[gi * T16 + a.T + (i - gi * (T16 - a.T))] = make_float2(0.0f, 0.0f);
    }
  };
  stage(0);
  __syncthreads();

  floatx4 yacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) yacc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  const float sdiv = VERIFY ? 1.0f / 16.0f : 1.0f;
  // A operand rows: tokens past T read token T - 1 (their meta is zero)
  int aoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) aoff[mt] = min(mt * 16 + (lane & 15), a.T - 1) * a.pitch;
  const int nw0 = (ng + KW - 1) / KW;   // the most groups a wave takes (ks = 0)
  const int ngp = (nw0 + kRing - 1) / kRing * kRing;
  for (int gg = 0; gg < ngp; gg += kRing) {
    // With several pieces, pg is a multiple of the ring depth: a piece starts
    // at the top of a ring round.  Every wave is past the previous piece
    // before it is overwritten.
    const int pb = gg - gg % a.pg;
    if (gg > 0 && pb == gg) {
      __syncthreads();
      stage(pb);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      // slots past the split's last group only keep the ring's loads going
      const int j = gg + i;
      const bool live = j < nwg;          // uniform over the wave
      const int gc = ks + KW * j - pb;    // the group within the staged piece
      uint32_t B[4][4];
      float s = 0.0f;
      if (live) {
        unpack<VERIFY>(wb[i], VERIFY ? wr[i] : wb[i], B);
        s = h2f(ws[i]) * sdiv;
      }
      {
        const int g = gidx(j + kRing);
        wb[i] = *reinterpret_cast<const uint4 *>(bp + (size_t)g * 1024);
        if constexpr (VERIFY) wr[i] = *reinterpret_cast<const uint4 *>(rp + (size_t)g * 1024);
        ws[i] = sc[(size_t)g * 16];
      }
      if (!live) continue;
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        half8 bh;
        __builtin_memcpy(&bh, B[st], 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const half8 ah = *reinterpret_cast<const half8 *>(xs + aoff[mt] + gc * kGroup + kb * 32 + st * 8);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[mt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float4 *mp = reinterpret_cast<const float4 *>(meta + gc * T16 + mt * 16 + kb * 4);
        const float4 m01 = mp[0], m23 = mp[1];   // {inv, bias*sum} of tokens 4kb .. 4kb+3
        yacc[mt][0] += s * m01.x * (acc[mt][0] - m01.y);
        yacc[mt][1] += s * m01.z * (acc[mt][1] - m01.w);
        yacc[mt][2] += s * m23.x * (acc[mt][2] - m23.y);
        yacc[mt][3] += s * m23.z * (acc[mt][3] - m23.w);
      }
    }
  }

  // the K shares of a tile, added in share order by its first wave
  if constexpr (KW > 1) {
    floatx4 *red = reinterpret_cast<floatx4 *>(smem);   // x' is no longer read
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = yacc[mt];
    __syncthreads();
    if (ks == 0)
      for (int k = 1; k < KW; ++k)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) yacc[mt] += red[((k * RT + tl) * MT + mt) * 64 + lane];
  }
  const bool writer = ks == 0;

  // outputs: token m = 16 mt + 4 kb + i of this lane's row
  if (a.S == 1) {
    if (writer && row < a.d_out)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + kb * 4 + i;
          if (m < a.T) a.y[(size_t)m * a.d_out + row] = yacc[mt][i];
        }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + kb * 4 + i;
      if (writer && m < a.T) st_agent(a.part + ((size_t)sp * a.T + m) * a.rows_pad + row, yacc[mt][i]);
    }
  stores_done();
  __syncthreads();
  __shared__ int last;
  if (t == 0)
    last = __hip_atomic_fetch_add(&a.tick[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(a.S - 1);
  __syncthreads();
  if (!last) return;
  // Each output is summed over the splits in split order from zero.  When
  // the partials' 32-bit buffer offsets suffice, a thread takes up to two
  // runs of 4 rows and issues the 16-byte agent-scope loads of up to 8 splits
  // of both before its first add: a row block of 64 tokens costs two memory
  // round trips per 8 splits instead of sixteen.  Threads without a run
  // issue nothing.
  const size_t pstride = (size_t)a.T * a.rows_pad;
  if ((size_t)a.S * pstride * 4 < 0x7FFFFFFFu) {
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(a.part, 0, (int)((size_t)a.S * pstride * 4), 0x00020000);
    constexpr int kRuns = RB / 4;
    const int total = a.T * kRuns;
    for (int base = 0; base < total; base += 2 * kThreads) {
      if (base + t >= total) break;   // no barrier follows
      uint32_t o[2];   // float index of the run in split 0, or ~0u for none
      floatx4 v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = base + u * kThreads + t, m = idx / kRuns, r4 = idx - m * kRuns;
        o[u] = idx < total ? (uint32_t)((size_t)m * a.rows_pad + rb * RB + 4 * r4) : ~0u;
        v[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      for (int s0 = 0; s0 < a.S; s0 += 8) {
        floatx4 w[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (o[u] != ~0u)
#pragma unroll
            for (int q = 0; q < 8; ++q)
              w[u][q] = __builtin_bit_cast(
                  floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                               pr, (int)(((uint32_t)min(s0 + q, a.S - 1) * (uint32_t)pstride + o[u]) * 4u), 0, kSc1));
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (o[u] != ~0u)
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (s0 + q < a.S) v[u] += w[u][q];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (o[u] == ~0u) continue;
        const int idx = base + u * kThreads + t, m = idx / kRuns, r = rb * RB + 4 * (idx - m * kRuns);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r + i < a.d_out) a.y[(size_t)m * a.d_out + r + i] = v[u][i];
      }
    }
    if (t == 0) __hip_atomic_store(&a.tick[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // partials in split order, eight loads in flight per output
  for (int idx = t; idx < a.T * RB; idx += kThreads) {
    const int m = idx / RB, r = rb * RB + (idx - m * RB);
    const float *pp = a.part + (size_t)m * a.rows_pad + r;
    const size_t stride = (size_t)a.T * a.rows_pad;
    float acc = 0.0f;
    for (int s0 = 0; s0 < a.S; s0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_agent(pp + (size_t)min(s0 + u, a.S - 1) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < a.S) acc += v[u];
    }
    if (r < a.d_out) a.y[(size_t)m * a.d_out + r] = acc;
  }
  if (t == 0) __hip_atomic_store(&a.tick[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Canonical row-major planes -> tile-major blocks: thread = one lane's 16
// bytes of one (tile, group) block of one plane; rows past d_out are zeros.
__global__ __launch_bounds__(256) void w48_repack_kernel(const uint8_t *src, uint8_t *dst, int d_out, int d_in,
                                                         int G, int64_t n_pieces) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_pieces) return;
  const int lane = (int)(i & 63);
  const int64_t blk = i >> 6;                  // tile * G + g
  const int64_t tile = blk / G;
  const int g = (int)(blk - tile * G);
  const int64_t row = tile * 16 + (lane & 15);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < d_out) v = *reinterpret_cast<const uint4 *>(src + row * (d_in / 2) + (int64_t)g * 64 + (lane >> 4) * 16);
  *reinterpret_cast<uint4 *>(dst + i * 16) = v;
}

__global__ __launch_bounds__(256) void w48_repack_scales_kernel(const uint16_t *src, uint16_t *dst, int d_out,
                                                                int G, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (tile * G + g) * 16 + r
  if (i >= n) return;
  const int r = (int)(i & 15);
  const int64_t blk = i >> 4, tile = blk / G;
  const int g = (int)(blk - tile * G);
  const int64_t row = tile * 16 + r;
  dst[i] = row < d_out ? src[row * G + g] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
char g_msg[512];

nl_status fail(nl_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
nl_status fail(nl_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return nl::api_error(st, g_msg);
}

nl_status ok() { return nl::api_error(NL_OK, ""); }

#define HIP_OR_FAIL(expr)                                                              \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(NL_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

std::mutex g_mu;
std::unordered_set<const void *> g_live;

bool valid(nl_w4w8_handle h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return h && g_live.count(h) && h->magic == kMagic;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int mt, rt, S, gps, pg, pitch;
  size_t lds, tick_bytes, part_bytes;
  size_t total() const { return tick_bytes + part_bytes; }
};

// A workgroup may hold the whole K-range of x' and split it among the waves
// of each tile (no split-K hand-over) up to one token tile and T * d_in <=
// 16384 (each workgroup then stages all of x: down, 4096x14336, lost 0.3 us
// at T = 1 and 1-4 us at T = 2-4 where q/o, k/v and gate/up gained 1-2 us);
// the LDS that form may use (one workgroup per CU).
constexpr int kKwMaxTG = 128;   // T times the groups of 128 columns
constexpr int kKwLds = 150 * 1024;

// Split count: one workgroup per CU in one round (measured best at every T
// on the 7B/8B-class shapes, also where two would fit: 256 workgroups beat
// 512), but at least four groups per split, so that the split sums of small
// shapes stay few.  A K-range whose x' does not fit the LDS is staged in
// pieces of whole ring rounds.  For small T * d_in (kKwMaxTG), when the
// whole x' fits, a workgroup takes the whole K-range of 16 RT rows instead,
// RT the fewest row tiles (1, 2 or 4) that keep the grid within one round.
Plan make_plan(const nl_w4w8 *h, int T, bool verify) {
  Plan p{};
  p.mt = (T + 15) / 16;
  const int T16 = 16 * p.mt;
  const int ring = verify && p.mt == 2 ? ring_depth<true, 2>() : ring_depth<false, 1>();
  p.rt = 8;
  if (p.mt == 1 && T * h->G <= kKwMaxTG) {
    int rt = 1;
    while (rt < 8 && h->rows_pad / (16 * rt) > kCus) rt *= 2;
    const size_t whole = (size_t)T * (h->G * kGroup + 8) * 2 + (size_t)h->G * T16 * 8;
    if (rt < 8 && whole <= (size_t)kKwLds) {
      p.rt = rt;
      p.S = 1;
      p.gps = p.pg = h->G;
      p.pitch = h->G * kGroup + 8;
      // the tiles' K shares are added through the same LDS
      p.lds = std::max(whole, (size_t)kThreads / 64 * p.mt * 64 * 16);
      p.tick_bytes = align256((size_t)(h->rows_pad / (16 * rt)) * 4);
      p.part_bytes = 0;
      return p;
    }
  }
  // per group: T rows of 128 fp16 and T16 (inverse scale, bias * sum) pairs;
  // per row 16 bytes of padding
  const int gps_max = std::max(1, (lds_budget(p.mt) - 16 * T) / (256 * T + 8 * T16));
  const int n_rb = h->rows_pad / kRows;
  int S = std::min(kCus / n_rb, h->G / 4);
  S = std::min(std::max(S, 1), h->G);
  p.gps = (h->G + S - 1) / S;
  p.S = (h->G + p.gps - 1) / p.gps;
  p.pg = p.gps <= gps_max ? p.gps : gps_max / ring * ring;
  p.pitch = p.pg * kGroup + 8;
  p.lds = (size_t)T * p.pitch * 2 + (size_t)p.pg * T16 * 8;
  p.tick_bytes = align256((size_t)n_rb * 4);
  p.part_bytes = p.S > 1 ? (size_t)p.S * T * h->rows_pad * 4 : 0;
  return p;
}

// Kernels with more than 64 KiB of dynamic LDS must say so once per process.
hipError_t allow_lds() {
  static hipError_t e = [] {
    hipError_t r = hipSuccess;
    auto set = [&](const void *f, int bytes) {
      if (r == hipSuccess) r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    };
    set(reinterpret_cast<const void *>(&w48_kernel<true, 3, 8>), lds_budget(3));
    set(reinterpret_cast<const void *>(&w48_kernel<true, 4, 8>), lds_budget(3));
    set(reinterpret_cast<const void *>(&w48_kernel<false, 3, 8>), lds_budget(3));
    set(reinterpret_cast<const void *>(&w48_kernel<false, 4, 8>), lds_budget(3));
    set(reinterpret_cast<const void *>(&w48_kernel<true, 1, 1>), kKwLds);
    set(reinterpret_cast<const void *>(&w48_kernel<true, 1, 2>), kKwLds);
    set(reinterpret_cast<const void *>(&w48_kernel<true, 1, 4>), kKwLds);
    set(reinterpret_cast<const void *>(&w48_kernel<false, 1, 1>), kKwLds);
    set(reinterpret_cast<const void *>(&w48_kernel<false, 1, 2>), kKwLds);
    set(reinterpret_cast<const void *>(&w48_kernel<false, 1, 4>), kKwLds);
    return r;
  }();
  return e;
}

template <bool V, int MT, int RT>
hipError_t launch_mt(const W48Args &a, const Plan &p, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows_pad / (16 * RT) * p.S)), block(kThreads);
  hipLaunchKernelGGL((w48_kernel<V, MT, RT>), grid, block, p.lds, s, a);
  return hipGetLastError();
}

template <bool V>
hipError_t launch(const W48Args &a, const Plan &p, hipStream_t s) {
  if (p.mt == 1 && p.rt == 1) return launch_mt<V, 1, 1>(a, p, s);
  if (p.mt == 1 && p.rt == 2) return launch_mt<V, 1, 2>(a, p, s);
  if (p.mt == 1 && p.rt == 4) return launch_mt<V, 1, 4>(a, p, s);
  if (p.rt != 8) return hipErrorInvalidValue;
  switch (p.mt) {
    case 1: return launch_mt<V, 1, 8>(a, p, s);
    case 2: return launch_mt<V, 2, 8>(a, p, s);
    case 3: return launch_mt<V, 3, 8>(a, p, s);
    case 4: return launch_mt<V, 4, 8>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

nl_status forward(nl_w4w8_handle h, bool verify, const void *x, int32_t T, float *y, void *ws, size_t ws_bytes,
                  void *stream, const char *who) {
  if (!valid(h)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (!x || !y || !ws) return fail(NL_EINVAL, "%s: x, y and ws must not be NULL", who);
  if (T < 1) return fail(NL_EINVAL, "%s: T must be >= 1 (got %d)", who, T);
  if (T > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T = %d exceeds %d", who, T, NL_MAX_T);
  if ((uintptr_t)x & 15) return fail(NL_EINVAL, "%s: x must be 16-byte aligned", who);
  if ((uintptr_t)ws & 255) return fail(NL_EINVAL, "%s: ws must be 256-byte aligned", who);
  if (verify && !h->has_ref) return fail(NL_EINVAL, "%s: the linear has no refinement plane", who);
  const Plan p = make_plan(h, T, verify);
  if (p.pg < 1 || p.lds > (size_t)(p.rt < 8 ? kKwLds : lds_budget(p.mt)))
    return fail(NL_EUNSUPPORTED, "%s: no LDS plan for T = %d", who, T);
  if (ws_bytes < p.total())
    return fail(NL_EINVAL, "%s: workspace of %zu bytes is smaller than %zu", who, ws_bytes, p.total());
  W48Args a{};
  a.base = h->base;
  a.ref = h->ref;
  a.scales = h->scales;
  a.x = static_cast<const uint16_t *>(x);
  a.y = y;
  char *w = static_cast<char *>(ws);
  a.tick = reinterpret_cast<uint32_t *>(w);
  a.part = reinterpret_cast<float *>(w + p.tick_bytes);
  a.d_out = h->d_out;
  a.d_in = h->d_in;
  a.rows_pad = h->rows_pad;
  a.G = h->G;
  a.T = T;
  a.S = p.S;
  a.gps = p.gps;
  a.pg = p.pg;
  a.pitch = p.pitch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_OR_FAIL(verify ? launch<true>(a, p, s) : launch<false>(a, p, s));
  return ok();
}

}  // namespace

extern "C" nl_status nested_w4w8_create(const nl_w4w8_desc *d, nl_w4w8_handle *out) {
  static const char *who = "nested_w4w8_create";
  if (!d || !out) return fail(NL_EINVAL, "%s: desc and out must not be NULL", who);
  if (d->d_out < 1 || d->d_in < kGroup || d->d_in % kGroup)
    return fail(NL_EINVAL, "%s: need d_out >= 1 and d_in a positive multiple of 128 (got %d x %d)", who, d->d_out,
                d->d_in);
  if (!d->base_plane || !d->scales) return fail(NL_EINVAL, "%s: base_plane and scales must not be NULL", who);
  auto *h = new (std::nothrow) nl_w4w8{};
  if (!h) return fail(NL_ENOMEM, "%s: host allocation failed", who);
  h->magic = kMagic;
  h->d_out = d->d_out;
  h->d_in = d->d_in;
  h->rows_pad = (d->d_out + kRows - 1) / kRows * kRows;
  h->G = d->d_in / kGroup;
  h->has_ref = d->ref_plane != nullptr;
  const size_t plane = (size_t)h->rows_pad * (d->d_in / 2), sc = (size_t)h->rows_pad * h->G * 2;
  const int64_t pieces = (int64_t)(h->rows_pad / 16) * h->G * 64, nsc = (int64_t)(h->rows_pad / 16) * h->G * 16;
  hipError_t e = hipMalloc(&h->base, plane);
  if (e == hipSuccess && h->has_ref) e = hipMalloc(&h->ref, plane);
  if (e == hipSuccess) e = hipMalloc(&h->scales, sc);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(w48_repack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, nullptr,
                       d->base_plane, h->base, h->d_out, h->d_in, h->G, pieces);
    e = hipGetLastError();
  }
  if (e == hipSuccess && h->has_ref) {
    hipLaunchKernelGGL(w48_repack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, nullptr,
                       d->ref_plane, h->ref, h->d_out, h->d_in, h->G, pieces);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(w48_repack_scales_kernel, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, nullptr,
                       d->scales, h->scales, h->d_out, h->G, nsc);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = allow_lds();
  if (e != hipSuccess) {
    (void)hipFree(h->base);
    (void)hipFree(h->ref);
    (void)hipFree(h->scales);
    delete h;
    return fail(e == hipErrorOutOfMemory ? NL_ENOMEM : NL_EHIP, "%s: %s", who, hipGetErrorString(e));
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(h);
  }
  *out = h;
  return ok();
}

extern "C" nl_status nested_w4w8_destroy(nl_w4w8_handle h) {
  if (!valid(h)) return fail(NL_EINVAL, "nested_w4w8_destroy: invalid handle");
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.erase(h);
  }
  (void)hipFree(h->base);
  (void)hipFree(h->ref);
  (void)hipFree(h->scales);
  h->magic = 0;
  delete h;
  return ok();
}

extern "C" nl_status nested_w4w8_workspace_bytes(nl_w4w8_handle h, int32_t T_max, size_t *bytes) {
  static const char *who = "nested_w4w8_workspace_bytes";
  if (!valid(h)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (!bytes) return fail(NL_EINVAL, "%s: bytes is NULL", who);
  if (T_max < 1) return fail(NL_EINVAL, "%s: T_max must be >= 1", who);
  if (T_max > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T_max = %d exceeds %d", who, T_max, NL_MAX_T);
  size_t need = 0;
  for (int T = 1; T <= T_max; ++T) {
    const Plan p = make_plan(h, T, true);   // the partials do not depend on the mode
    need = std::max(need, p.total());
  }
  *bytes = need;
  return ok();
}

extern "C" nl_status nested_w4w8_verify(nl_w4w8_handle h, const void *x, int32_t T, float *y, void *ws,
                                        size_t ws_bytes, void *stream) {
  return forward(h, true, x, T, y, ws, ws_bytes, stream, "nested_w4w8_verify");
}

extern "C" nl_status nested_w4w8_draft(nl_w4w8_handle h, const void *x, int32_t T, float *y, void *ws,
                                       size_t ws_bytes, void *stream) {
  return forward(h, false, x, T, y, ws, ws_bytes, stream, "nested_w4w8_draft");
}
