// nl_kernels.hip -- gfx950 kernels of the bit-nested quantized linear.
//
//   repack_kernel     canonical planes -> internal tile-chunk layout (create)
//   decode_kernel     internal layout -> integers, through the hot unpack code
//   rotate_in_kernel  x' = H_i S_i x in LDS, stored as fp16 scaled per
//                     (token, 512-column chunk) by a power of two, plus the
//                     fp32 group sums that undo the residual code offset
//   gemm_kernel       fused unpack + v_mfma_f32_16x16x32_f16 contraction with
//                     an fp32 per-group scale epilogue
//   finish_kernel     split-K sum + y = S_o H_o y~ in LDS
//
// The method is the verifier forward of the forum post "bit-nested", POC
// recipe section 4 (rotation: section 1; base: section 2; residual:
// section 3).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "nl_kernels.h"
#include "nl_dev.h"

namespace nl {

// ===========================================================================
// Create-time repack.  One wave per tile-chunk; lane l handles row
// tile*16 + (l & 15) and columns [32*(l >> 4), +32) of the chunk's 4 groups.
// ===========================================================================
template <int BITS>
__global__ __launch_bounds__(64) void repack_kernel(const RepackArgs a) {
  const int tc = blockIdx.x;
  const int tile = tc / a.n_chunks, chunk = tc % a.n_chunks;
  const int lane = threadIdx.x;
  const int r = tile * kTileRows + (lane & 15), kq = lane >> 4;
  constexpr int RB = BITS > 0 ? BITS : 1;
  uint32_t bd[8];
  uint32_t rd[4 * RB];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int gi = chunk * kChunkGroups + g;
    const bool ok = r < a.d_out && gi < a.G;
    uint32_t w0 = 0, w1 = 0;
    uint32_t v[32];
    for (int j = 0; j < 32; ++j) {
      const int k = 32 * kq + j;  // column within the group
      uint32_t c = 0, u = BITS ? (1u << (RB - 1)) : 0u;
      if (ok) {
        const uint8_t *bg = a.base_codes + ((size_t)r * a.G + gi) * 32;
        c = ((bg[k >> 3] >> (k & 7)) & 1u) | (((bg[16 + (k >> 3)] >> (k & 7)) & 1u) << 1);
        if (BITS) {
          const uint8_t *rg = a.resid_codes + ((size_t)r * a.G + gi) * (16 * RB);
          uint32_t f = 0;
          for (int t = 0; t < RB; ++t) {
            const int bit = k * RB + t;
            f |= ((uint32_t)(rg[bit >> 3] >> (bit & 7)) & 1u) << t;
          }
          u = f ^ (1u << (RB - 1));  // two's complement -> q + 2^(b-1)
        }
      }
      if (j < 16) w0 |= c << (2 * j);
      else w1 |= c << (2 * (j - 16));
      v[j] = u;
    }
    bd[2 * g] = w0;
    bd[2 * g + 1] = w1;
    if constexpr (BITS > 0) pack_resid<BITS>(v, rd + g * BITS);
    if (kq == 0) {
      const size_t si = ((size_t)tc * kTileRows + (lane & 15)) * 4 + g;
      a.bscale[si] = ok ? a.base_scales[(size_t)r * a.G + gi] : (uint16_t)0;
      if (BITS) a.rscale[si] = ok ? a.resid_scales[(size_t)r * a.G + gi] : (uint16_t)0;
    }
  }
  uint4 *bb = a.base + (size_t)tc * (64 * kBasePieces);
#pragma unroll
  for (int i = 0; i < kBasePieces; ++i)
    bb[i * 64 + lane] = make_uint4(bd[4 * i], bd[4 * i + 1], bd[4 * i + 2], bd[4 * i + 3]);
  if constexpr (BITS > 0) {
    uint4 *rb = a.resid + (size_t)tc * (64 * BITS);
#pragma unroll
    for (int i = 0; i < BITS; ++i)
      rb[i * 64 + lane] = make_uint4(rd[4 * i], rd[4 * i + 1], rd[4 * i + 2], rd[4 * i + 3]);
  }
}

// ===========================================================================
// Weight registers of one tile-chunk and their loads (shared by the decode
// and contraction kernels so the decode hook tests the hot path's reads).
// ===========================================================================
template <int BITS>
struct ChunkRegs {
  u32x4 b[kBasePieces];
  u32x4 r[BITS > 0 ? BITS : 1];
  uint2 sb, sr;
};

template <int BITS>
__device__ __forceinline__ void load_chunk(ChunkRegs<BITS> &w, const LinearDev &L, int n_chunks,
                                           int tile, int chunk, int lane) {
  const size_t tc = (size_t)tile * n_chunks + chunk;
  const u32x4 *bp = reinterpret_cast<const u32x4 *>(L.base) + tc * (64 * kBasePieces) + lane;
#pragma unroll
  for (int i = 0; i < kBasePieces; ++i) w.b[i] = __builtin_nontemporal_load(bp + i * 64);
  w.sb = L.bscale[tc * kTileRows + (lane & 15)];
  if constexpr (BITS > 0) {
    const u32x4 *rp = reinterpret_cast<const u32x4 *>(L.resid) + tc * (64 * BITS) + lane;
#pragma unroll
    for (int i = 0; i < BITS; ++i) w.r[i] = __builtin_nontemporal_load(rp + i * 64);
    w.sr = L.rscale[tc * kTileRows + (lane & 15)];
  }
}

// ===========================================================================
// Decode hook: identity table for the base, raw offsets for the residual.
// ===========================================================================
template <int BITS>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
  __shared__ uint2 lut[256];
  const int lane = threadIdx.x;
  {
    // fp16 of the codes themselves: 0, 1, 2, 3
    const uint32_t h[4] = {0x0000u, 0x3C00u, 0x4000u, 0x4200u};
    uint32_t l16[16];
    for (int i = 0; i < 16; ++i) l16[i] = h[i & 3] | (h[i >> 2] << 16);
    for (int i = lane; i < 256; i += 64) lut[i] = base_table_entry(l16, i);
  }
  __syncthreads();
  const int tile = a.tile0 + blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  ChunkRegs<BITS> w;
  load_chunk<BITS>(w, a.lin, a.n_chunks, tile, chunk, lane);
  const int row = tile * kTileRows + (lane & 15);
  const int kq = lane >> 4;
  if (row < a.row0 || row >= a.row0 + a.nrows) return;
  const uint32_t *bw = reinterpret_cast<const uint32_t *>(w.b);
  const uint32_t *rw = reinterpret_cast<const uint32_t *>(w.r);
  for (int g = 0; g < kChunkGroups; ++g) {
    uint32_t bq[16], rq[16];
    unpack_base(bw + 2 * g, lut, bq);
    if constexpr (BITS > 0) unpack_resid<BITS>(rw + g * BITS, rq);
    for (int P = 0; P < 16; ++P) {
      for (int hh = 0; hh < 2; ++hh) {
        const int k = chunk * kChunk + g * kGroup + 32 * kq + 2 * P + hh;
        if (k >= a.d_in) continue;
        const size_t o = (size_t)(row - a.row0) * a.d_in + k;
        a.base_idx[o] = (uint8_t)(int)h2f((bq[P] >> (16 * hh)) & 0xFFFFu);
        if constexpr (BITS > 0) {
          if (a.resid)
            a.resid[o] = (int8_t)((int)((rq[P] >> (16 * hh)) & 0x3FFu) - (1 << (BITS - 1)));
        }
      }
    }
  }
}


// Largest e with offsets[e] <= row (the expert of a pair).
__device__ __forceinline__ int expert_of(const int32_t *offsets, int n, int row) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// An expert takes part in a grouped call when it owns at least one pair and
// its first pair lies inside the call's R rows.  The contraction, the count
// of waiting workgroups and the finish all use this one predicate.
__device__ __forceinline__ bool expert_active(const int32_t *offsets, int e, int R);

// Index of the slot-th linear (in index order) that has rows by the test
// of expert_active, or -1 when fewer have.  Each lane tests 8 consecutive
// experts per round of 512 (one batch of loads), a wave-wide prefix count
// finds the lane holding the slot, its bit mask the expert.  The result is
// wave-uniform; every wave of a workgroup computes it alike.
__device__ int nth_active_expert(const int32_t *offsets, int n, int R, int slot) {
  const NL_GLOBAL int32_t *o = (const NL_GLOBAL int32_t *)offsets;
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int r0 = 0; r0 < n; r0 += 512) {
    const int e0 = r0 + 8 * lane;
    int v[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) v[i] = o[min(e0 + i, n)];  // offsets holds n + 1 entries
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      bits |= (uint32_t)(e0 + i < n && v[i + 1] > v[i] && v[i] >= 0 && v[i] < R) << i;
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d, 64);
      if (lane >= d) incl += u;
    }
    const int total = __shfl(incl, 63, 64);
    if (slot < seen + total) {
      const int want = slot - seen;
      const unsigned long long m = __ballot(want >= incl - c && want < incl);
      const int L = __ffsll(m) - 1;
      uint32_t bl = __shfl(bits, L, 64);
      for (int q = want - __shfl(incl - c, L, 64); q > 0; --q) bl &= bl - 1;  // drop lower set bits
      return __builtin_amdgcn_readfirstlane(r0 + 8 * L + __ffs(bl) - 1);
    }
    seen += total;
  }
  return -1;
}

__device__ __forceinline__ bool expert_active(const int32_t *offsets, int e, int R) {
  const NL_CONST int32_t *o = (const NL_CONST int32_t *)offsets;  // scalar loads when e is uniform
  const int r0 = o[e], r1 = o[e + 1];
  return r1 > r0 && r0 >= 0 && r0 < R;
}


// Wait for a token on semaphore `sem` and take it (the output rotation's
// hand-over; same dispatch-order argument and spin limit as wait_ready).
// Returns false when the wait gave up (counted in the error word).
__device__ bool take_token(uint32_t *sem, const Handover &hv, uint32_t *err) {
  for (uint32_t it = 0; ld_dev(sem) < 1u + hv.wait_extra; ++it) {
    if (it >= hv.spin_limit) {
      ctr_add(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_fetch_sub(sem, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Wait until the ready line `line` has counted `n` rotation workgroups.
// Only a workgroup whose producers have lower indices waits, and workgroups
// are dispatched in index order, so the producers are running or done; the
// spin limit only bounds the wait if that ever fails, and counts the event in
// the error word.  Returns false when the wait gave up.
__device__ bool wait_ready(const uint32_t *line, uint32_t n, const Handover &hv, uint32_t *err) {
  for (uint32_t it = 0; ld_dev(line) < n + hv.wait_extra; ++it) {
    if (it >= hv.spin_limit) {
      ctr_add(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// ===========================================================================
// Input rotation (POC section 1: x' = H_i S_i x, computed a single time for each linear and call).
// Task = (row of x', superblock of SB = max(b, 512) columns), so every
// 512-column chunk lies in one task; a workgroup runs 4096/SB tasks.  Each
// chunk is scaled by 2^s (its largest magnitude lands in [2^14, 2^15]) and
// rounded to fp16, the contraction's MFMA operand; tsc = 2^-s / sqrt(b)
// undoes both factors.  Outputs (R = rows of x'): xh row-major [R][Kp];
// meta[(c*5+g)*R + r] = sum of the fp16 values of group g (g < 4) and
// meta[(c*5+4)*R + r] = tsc.  COH: agent-scope stores (read by other
// workgroups of the same launch), 16 bytes per store.
// ===========================================================================
// Rotation workgroup wg: each 256-thread group transforms 4096 values as
// 4096/SB tasks (row, superblock of SB columns) of TPS = SB/16 threads, 16
// values each; a workgroup of 512 threads or more runs two groups (a.groups),
// the first in the LDS area `xch`, the second in `spare` (SB + SB/16 floats
// per task each).  Threads past the groups (the fifth wave of a 320-thread
// workgroup, the ninth of 576) run the same code without touching LDS and
// store nothing: they only keep the barrier count (extra).
struct RotTask {
  int row, k0, lt, tl, grp, xrow;
  bool valid, extra;
  const int8_t *sign;
};
__device__ __forceinline__ RotTask rot_task(const RotInArgs &a, int wg, int tid) {
  RotTask t;
  const int SB = a.SB, TPS = SB >> 4;
  const int ng = a.groups > 1 ? a.groups : 1;
  t.extra = tid >= 256 * ng;
  if (t.extra) tid = 0;
  t.grp = tid >> 8;
  tid &= 255;
  t.lt = tid % TPS;
  t.tl = tid / TPS;
  const int n_sb = a.Kp / SB;
  const int task = (wg * ng + t.grp) * (256 / TPS) + t.tl;
  t.valid = !t.extra && task < a.rows * n_sb;
  t.row = t.valid ? task / n_sb : 0;
  t.k0 = (t.valid ? task % n_sb : 0) * SB + 16 * t.lt;
  t.xrow = t.valid ? t.row : -1;
  t.sign = a.sign;
  if (a.lins) {  // grouped: pair -> (token, expert); lanes without a task read expert 0's signs
    if (t.valid) {
      t.xrow = a.pair_token[t.row];
      if (t.xrow < 0 || t.xrow >= a.x_rows) t.xrow = -1;
    }
    t.sign = ((const NL_GLOBAL LinearDev *)a.lins)[t.valid ? expert_of(a.offsets, a.n_experts, t.row) : 0].sign_in;
  }
  return t;
}

// One thread's 16 rotated values as fp16 pairs under the (row, chunk)
// power-of-two scale 2^s, and the sum of its 128-column group.
struct RotOut {
  uint32_t w[8];
  float gs;
  int s;
};

// x' of one thread: x * sign, the block transform (xch: the thread's task
// area), then the scale of its 512-column chunk (32 threads) from the
// chunk's largest magnitude and the fp16 group sums (8 threads).
__device__ __forceinline__ void rot_transform(const RotInArgs &a, const RotTask &t, const XRaw &xr, float *xch,
                                              RotOut &o) {
  float v[16];
  cvt_x16(v, xr);
  fwht_b(v, xch, t.lt, a.lb, t.extra);
  // layout B: 16 consecutive columns; a chunk is 32 threads, a group 8
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  m = max_lanes32(m);
  int s = 0;
  if (m > 0.0f) {
    int e;
    frexpf(m, &e);
    s = 15 - e;
    s = s > 120 ? 120 : (s < -120 ? -120 : s);
  }
  float gs = 0.f;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const _Float16 q0 = (_Float16)ldexpf(v[2 * h], s), q1 = (_Float16)ldexpf(v[2 * h + 1], s);
    gs += (float)q0 + (float)q1;
    o.w[h] = (uint32_t)__builtin_bit_cast(uint16_t, q0) | ((uint32_t)__builtin_bit_cast(uint16_t, q1) << 16);
  }
  gs = sum_lanes8(gs);
  o.gs = gs;
  o.s = s;
}

// x' row-major [rows][Kp] fp16 (16 columns of the thread) and the metadata
// [chunk][5][rows]: four group sums and the chunk's inverse scale times
// 1/sqrt(block).  COH: device-coherent stores for a reader elsewhere in the
// same launch.
template <bool COH>
__device__ __forceinline__ void rot_store(const RotInArgs &a, const RotTask &t, const uint32_t (&w)[8], float gs,
                                          int s) {
  if (!t.valid) return;
  const int R = a.rows, k0 = t.k0, lt = t.lt;
  const size_t xo = (size_t)t.row * a.Kp + k0;  // element offset of the thread's 16 columns
  float *mg = a.meta + ((size_t)(k0 >> 9) * 5 + ((k0 >> 7) & 3)) * R + t.row;
  float *ms = a.meta + ((size_t)(k0 >> 9) * 5 + 4) * R + t.row;
  const u32x4 lo = {w[0], w[1], w[2], w[3]}, hi = {w[4], w[5], w[6], w[7]};
  if constexpr (COH) {
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.xh, 0, 0x7FFFFFF0, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(lo, xr, (int)(xo * 2), 0, kSc1);
    __builtin_amdgcn_raw_buffer_store_b128(hi, xr, (int)(xo * 2 + 16), 0, kSc1);
    if ((lt & 7) == 0) st_dev(mg, gs);
    if ((lt & 31) == 0) st_dev(ms, ldexpf(a.rsqrt_b, -s));
  } else {
    *reinterpret_cast<u32x4 *>(a.xh + xo) = lo;
    *reinterpret_cast<u32x4 *>(a.xh + xo + 8) = hi;
    if ((lt & 7) == 0) *mg = gs;
    if ((lt & 31) == 0) *ms = ldexpf(a.rsqrt_b, -s);
  }
}

template <bool COH>
__device__ __forceinline__ void rotate_body(const RotInArgs &a, int wg, float *xch, float *spare) {
  const RotTask t = rot_task(a, wg, threadIdx.x);
  const XRaw xr = load_x16(a.x, t.sign, t.xrow, t.k0, a.d_in);
  RotOut o;
  // group 0 transforms in xch, group 1 in spare (extra threads touch neither)
  rot_transform(a, t, xr, (t.extra || t.grp ? spare : xch) + t.tl * (a.SB + (a.SB >> 4)), o);
  rot_store<COH>(a, t, o.w, o.gs, o.s);
}

__global__ __launch_bounds__(256) void rotate_in_kernel(const RotInArgs a) {
  __shared__ float xch[4096 + 256];
  rotate_body<false>(a, blockIdx.x, xch, nullptr);
}

// ===========================================================================
// Fused contraction.  Workgroup = TW tile waves + 1: each tile wave owns one
// 16-row tile of a 16*TW-row block over a K-range of chunks (split-K index
// `split`), wave TW stages the activations (TW = 4, or 8 for three or more
// token tiles).
//   - each tile wave streams its own tile-chunks (2 + b pieces of 1 KiB plus
//     the scales) from HBM into a ring of register sets; it issues no other
//     loads, so the compiler's waits on them are exact;
//   - the loader wave copies x' (fp16) and its group sums / scales with
//     global_load_lds into a ring of NX LDS stages of XG groups, NX - 1
//     stages ahead; one s_barrier per stage hands a stage to the tile waves
//     and the stage before it back to the loader.
// In the single launch only the loader waits for the rotation, so the tile
// waves' first chunks stream in meanwhile.  One workgroup per CU (LDS).
// Per group: base and residual planes -> fp16 B operands (the residual field
// u = q + 2^(b-1) as the exact subnormal u * 2^-24); 4 MFMA steps per plane
// and token tile; fp32 epilogue
//   acc_chunk = fma(s_b / kappa, A_base, acc_chunk)
//   acc_chunk = fma(2^24 s_r, A_resid, fma(-2^(b-1) s_r, sum(x'), acc_chunk))
// and at the end of each chunk acc = fma(tsc, acc_chunk, acc).
// ===========================================================================

constexpr int kLdsBytes = 160 * 1024;

template <int BITS, int MT>
struct LdsPlan {
  static constexpr int TR = 16 * MT;               // token rows staged
  static constexpr int XG = MT <= 2 ? 4 : 2;       // groups per x' stage
  static constexpr int NST = kChunkGroups / XG;    // stages per chunk
  static constexpr int XI = XG * TR / 4;           // x' copies per stage (1 KiB each)
  static constexpr int MI = ((XG + 1) * TR + 63) / 64;  // metadata copies per stage (256 B each)
  static constexpr int XB = XI * 1024 + MI * 256;  // bytes per x' stage (activations, then metadata)
  static constexpr int NW = kBasePieces + 1 + (BITS > 0 ? BITS + 1 : 0);  // weight loads per chunk
  static constexpr int o_lut = 0;
  static constexpr int o_x = 256 * 8;
  // x' stages in flight: up to 4 while two workgroups still fit one CU
  static constexpr int NX_FIT = (kLdsBytes / 2 - o_x) / XB;
  static constexpr int NX_CNT = 2 + 63 / (XI + MI);  // the loader's wait count fits vmcnt
  static constexpr int NX_A = NX_FIT < NX_CNT ? NX_FIT : NX_CNT;
  static constexpr int NX = NX_A > 4 ? 4 : (NX_A < 2 ? 2 : NX_A);
  static constexpr int bytes = o_x + NX * XB;
  static constexpr int XWAIT = (NX - 2) * (XI + MI);  // loader copies after the stage it waits for
  static_assert(bytes <= kLdsBytes && XWAIT <= 63, "x' ring does not fit");
};

// Local rotation (at most kLocalRows rows of x'): the workgroup rotates the x
// blocks its K-range touches itself and keeps x' for the whole range in LDS,
// laid out [chunk][run][kLocalRows rows][8 fp16], with the group sums and
// scales as [chunk][5][kLocalRows] floats.
struct LocalPlan {
  static constexpr int o_lut = 0;
  static constexpr int o_x = 256 * 8;
  static constexpr int XC = 64 * kLocalRows * 16;            // bytes per chunk
  static constexpr int o_m = o_x + kLocalChunks * XC;
  static constexpr int o_f = o_m + kLocalChunks * 5 * kLocalRows * 4;
  static constexpr int bytes = o_f + (4096 + 256) * 4;      // + one FWHT area
};


// Register sets in the weight ring of a tile wave: deeper where the
// accumulators leave room (one or two token tiles), deepest for the draft,
// whose sets are a quarter the size.  The in-workgroup rotation (MT = 0)
// holds its transform registers while the first sets are in flight (one set
// for 7-bit planes, whose unpacking needs the most registers).  Every
// variant fits its registers without scratch.
template <int BITS, int MT, int TW>
__host__ __device__ constexpr int ring_sets() {
  if constexpr (MT == 0) return BITS == 0 ? 3 : (BITS == 7 ? 1 : 2);
  if constexpr (TW == 8) return BITS == 0 ? 2 : 1;  // eight tile waves: 168 registers each
  if constexpr (TW == 7) return BITS == 0 ? 3 : 2;
  return BITS == 0 ? 4 : 3;
}


// Direct global -> LDS copies (16 or 4 bytes per lane): lane i's bytes land
// at lds + i * size.  The compiler's builtin sets M0 itself, so no register is
// written behind its back.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const void *base) {
  __builtin_amdgcn_global_load_lds((const NL_GLOBAL void *)((const char *)base + voff), (NL_LOCAL void *)(size_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, const void *base) {
  __builtin_amdgcn_global_load_lds((const NL_GLOBAL void *)((const char *)base + voff), (NL_LOCAL void *)(size_t)lds, 4, 0, 0);
}
// A rotation task's x' is acknowledged (wait_stores) by the thread calling
// this with k < 8: it adds one to ready line k.  The last task to count on
// a line no contraction workgroup waits on clears it.  waiters: line k has
// waiting workgroups (some linear has rows and owns a workgroup on it).
__device__ __forceinline__ void publish_ready(uint32_t *ctr, int n_rot, int k, bool waiters) {
  uint32_t *line = ctr_at(ctr, kCtrReady + k);
  if (waiters)
    ctr_add(line, 1u);  // result unused: no return trip before the workgroup ends
  else if (ctr_add(line, 1u) == (uint32_t)(n_rot - 1))
    st_dev(line, 0u);
}

// MT = 0: local rotation mode (single launch only; rot describes x).
template <int BITS, int MT, bool FUSED, int TW = tile_waves(MT)>
__device__ __forceinline__ void contract_body(const GemmArgs &a, int e, int rb, int split, char *smem,
                                              const Handover &hv, const RotInArgs &rot) {
  constexpr bool LOCAL = MT == 0;
  constexpr int MTC = LOCAL ? 1 : MT;  // 16-row MFMA token tiles
  using Pl = LdsPlan<BITS, MTC>;
  constexpr int TR = LOCAL ? kLocalRows : Pl::TR, XG = LOCAL ? 4 : Pl::XG, NST = LOCAL ? 1 : Pl::NST;
  constexpr int NX = Pl::NX;
  static_assert(!LOCAL || FUSED, "local rotation runs in the single launch only");
  static_assert(TW == 4 || ((TW == 7 || TW == 8) && MT > 0), "four tile waves, or seven or eight outside the in-workgroup rotation");
  constexpr int NT = 64 * (TW + 1), RB = 16 * TW;  // threads, rows per block
  __shared__ uint32_t s_flag;
  __shared__ uint32_t s_lost;  // the loader's wait for x' gave up

  // (wave index read as a scalar so per-wave choices stay uniform branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const bool loader = wave == TW;
  // The descriptor by value, read with scalar loads (the expert array is
  // read-only for the launch and e is uniform): a generic pointer that may
  // point at the kernel arguments would turn every field into a flat load
  // and a full wait at the start of the workgroup.
  int row_base = 0, nrows = a.T;
  if (a.lins) {
    row_base = a.offsets[e];
    nrows = a.offsets[e + 1] - row_base;
    // idle expert (or offsets outside [0, rows)): uniform exit before any barrier
    if (!expert_active(a.offsets, e, a.T)) return;
  }
  const NL_CONST LinearDev &L = *(const NL_CONST LinearDev *)(a.lins ? a.lins + e : &a.lin);
  nrows = min(min(nrows, TR), a.T - row_base);
  const int tile_id = rb * TW + (loader ? 0 : wave);
  const bool active = !loader && tile_id < a.n_tiles;
  const int tile = min(tile_id, a.n_tiles - 1);
  const int c_begin = split * a.cps;
  const int c_end = min(a.n_chunks, c_begin + a.cps);
  const int nchk = c_end - c_begin;
  {  // byte-indexed base table (LocalPlan::o_lut == LdsPlan::o_lut == 0) from
     // the descriptor's 16 pair words, staged through LDS by one thread (they
     // are scalar loads; a per-lane choice among them would become an
     // indexed memory load and a full wait)
    __shared__ uint32_t s_l16[16];
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) s_l16[k] = L.lut[k];
    }
    __syncthreads();
    if (threadIdx.x < 256)
      reinterpret_cast<uint2 *>(smem)[threadIdx.x] = make_uint2(s_l16[threadIdx.x & 15], s_l16[threadIdx.x >> 4]);
  }
  const int tl = lane & 15, kq = lane >> 4;
  const int R = a.T;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(NL_LOCAL void *)smem;

  floatx4 acc[MTC];
#pragma unroll
  for (int m = 0; m < MTC; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (!LOCAL && loader) {
    // ---- x' stager: stage q = (chunk c_begin + q / NST, groups [g0, g0 + XG))
    // rows past nrows re-read row nrows - 1 (they only feed output rows that
    // are never stored), so every stage issues the same copies.
    const void *xsrc = sgpr_ptr(a.xh), *msrc = sgpr_ptr(a.meta);
    const int Q = nchk * NST;
    auto stage = [&](int q) {
      q = min(q, Q - 1);  // past the end: re-copy the last stage into a free buffer
      const int c = c_begin + q / NST, g0 = (q % NST) * XG;
      const uint32_t xl = lds0 + Pl::o_x + (q % NX) * Pl::XB, ml = xl + Pl::XI * 1024;
#pragma unroll
      for (int j = 0; j < Pl::XI; ++j) {  // x' is row-major [R][Kp]: gather 16-byte runs into the stage
        const int slot = 64 * j + lane;
        const int run = slot / TR, t = min(slot % TR, nrows - 1);
        const int col = (c * 4 + g0 + (run >> 4)) * 128 + run_col(run & 15);
        dma16(xl + 1024 * j, (uint32_t)(((size_t)(row_base + t) * a.Kp + col) * 2), xsrc);
      }
#pragma unroll
      for (int j = 0; j < Pl::MI; ++j) {
        const int slot = min(64 * j + lane, (XG + 1) * TR - 1);
        const int k = slot / TR, t = min(slot % TR, nrows - 1);
        const int gi = k < XG ? g0 + k : 4;
        dma4(ml + 256 * j, (uint32_t)(((c * 5 + gi) * R + row_base + t) * 4), msrc);
      }
    };
    if constexpr (FUSED && !LOCAL) {
      // a wait that gave up leaves stale x': the tile waves then write NaN
      if (lane == 0) {
        const bool ok = wait_ready(ctr_at(hv.ctr, kCtrReady + hv.line), (uint32_t)hv.n_rot, hv, ctr_at(hv.ctr, kCtrErr));
        s_lost = ok ? 0u : 1u;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible at the first stage barrier
    }
    // Stage q lives in buffer q % NX.  Barrier #q publishes stage q and
    // tells the loader the tile waves are done with stage q - 1, whose
    // buffer then receives stage q + NX - 1.
    for (int q = 0; q < NX - 1; ++q) stage(q);
#pragma unroll 1
    for (int q = 0; q < Q; ++q) {
      wait_vm<Pl::XWAIT>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      stage(q + NX - 1);
    }
    wait_vm<0>();
  } else {
    // ---- tile wave: this wave's tile codes, two chunks in flight in registers.
    // Raw buffer loads through descriptors that end at the split's last
    // chunk: a request past it (the pipeline's padding) returns zeros without
    // a memory access, and every trip still issues the same loads.
    const size_t tc0 = (size_t)tile * a.n_chunks;
    constexpr int kRaw = 0x00020000;  // raw 32-bit buffer descriptor word 3
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)sgpr_ptr(L.base + tc0 * 128), 0, c_end * kBaseBlockBytes, kRaw);
    const __amdgpu_buffer_rsrc_t rsb =
        __builtin_amdgcn_make_buffer_rsrc((void *)sgpr_ptr(L.bscale + tc0 * 16), 0, c_end * kScaleBlockBytes, kRaw);
    __amdgpu_buffer_rsrc_t rr = rb, rsr = rsb;
    if constexpr (BITS > 0) {
      rr = __builtin_amdgcn_make_buffer_rsrc((void *)sgpr_ptr(L.resid + tc0 * (64 * BITS)), 0,
                                             c_end * resid_block_bytes(BITS), kRaw);
      rsr = __builtin_amdgcn_make_buffer_rsrc((void *)sgpr_ptr(L.rscale + tc0 * 16), 0, c_end * kScaleBlockBytes,
                                              kRaw);
    }
    constexpr int kNt = 2;  // non-temporal: the codes are streamed once
    // one fixed issue order everywhere (the fences keep the scheduler from
    // interleaving), so the waits the compiler counts agree on every path
    auto fence = []() { asm volatile("" ::: "memory"); };
    auto loadw = [&](WRegs<BITS> &w, int c) {
#pragma unroll
      for (int i = 0; i < kBasePieces; ++i) {
        w.b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (c * 128 + i * 64 + lane) * 16, 0, kNt));
        fence();
      }
      w.sb = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rsb, (c * 16 + tl) * 8, 0, 0));
      fence();
      if constexpr (BITS > 0) {
#pragma unroll
        for (int i = 0; i < BITS; ++i) {
          w.r[i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (c * 64 * BITS + i * 64 + lane) * 16, 0, kNt));
          fence();
        }
        w.sr = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rsr, (c * 16 + tl) * 8, 0, 0));
        fence();
      }
    };
    // the same loads in four parts: part g is issued after group g of the
    // compute in progress (refilling the set computed just before it), so
    // the memory pipeline takes them between groups rather than in bursts
    auto loadpart = [&](WRegs<BITS> &w, int c, int g) {
      if (g == 0) {
#pragma unroll
        for (int i = 0; i < kBasePieces; ++i)
          w.b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (c * 128 + i * 64 + lane) * 16, 0, kNt));
        w.sb = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rsb, (c * 16 + tl) * 8, 0, 0));
      }
      if constexpr (BITS > 0) {
        constexpr int per = (BITS + 2) / 3;
        if (g > 0) {
#pragma unroll
          for (int i = (g - 1) * per; i < (g == 3 ? BITS : g * per); ++i)
            w.r[i] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (c * 64 * BITS + i * 64 + lane) * 16, 0, kNt));
        }
        if (g == 3) w.sr = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rsr, (c * 16 + tl) * 8, 0, 0));
      }
    };
    const uint2 *s_lut = reinterpret_cast<const uint2 *>(smem);
    const float kinv = L.kinv;
    // compute chunk ci (its NST stages, a barrier before every stage but the
    // first overall); refill(g) runs after group g
    auto compute = [&](WRegs<BITS> &w, int ci, auto refill) {
      pin(w);
      const uint32_t *bw = reinterpret_cast<const uint32_t *>(w.b);
      const uint32_t *rw = reinterpret_cast<const uint32_t *>(w.r);
      floatx4 accC[MTC];
#pragma unroll
      for (int m = 0; m < MTC; ++m) accC[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const _Float16 *xb;
        const float *mb;
        if constexpr (LOCAL) {  // resident x': rows past kLocalRows repeat (never stored)
          xb = reinterpret_cast<const _Float16 *>(smem + LocalPlan::o_x + ci * LocalPlan::XC) +
               (kq * TR + (tl & (TR - 1))) * 8;
          mb = reinterpret_cast<const float *>(smem + LocalPlan::o_m) + ci * 5 * TR;
        } else {
          const int q = ci * NST + st, buf = q % NX;
          if (q > 0) {  // stage q published, stage q - 1's buffer released
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
          }
          xb = reinterpret_cast<const _Float16 *>(smem + Pl::o_x + buf * Pl::XB) + (kq * TR + tl) * 8;
          mb = reinterpret_cast<const float *>(smem + Pl::o_x + buf * Pl::XB + Pl::XI * 1024) + 4 * kq;
        }
        // One token tile (HA): a group's activations, sums and base table
        // entries are read before its unpacking, so their LDS latency passes
        // under it; for the draft, whose unpacking is short, group gl + 1's
        // are requested before group gl's MFMAs instead (group 0's at the
        // start of the stage).  More tiles read theirs at the MFMAs: the
        // registers would not fit.
        constexpr int HA = MTC == 1 && TW == 4 ? 1 : 0;
        constexpr bool PIPE = HA && BITS == 0;
        half8 Ah[2][4];
        floatx4 xh[2];
        uint32_t bqh[2][16];
        auto load_group = [&](int gl, int slot) {
#pragma unroll
          for (int s = 0; s < 4; ++s) Ah[slot][s] = *reinterpret_cast<const half8 *>(xb + (gl * 4 + s) * 4 * TR * 8);
          if constexpr (BITS > 0) xh[slot] = *reinterpret_cast<const floatx4 *>(mb + gl * TR);
          unpack_base(reinterpret_cast<const uint32_t *>(w.b) + 2 * (st * XG + gl), s_lut, bqh[slot]);
        };
        if constexpr (PIPE) load_group(0, 0);
#pragma unroll
        for (int gl = 0; gl < XG; ++gl) {
          const int g = st * XG + gl;
          const int cur = gl & 1;
          if constexpr (PIPE) {
            if (gl + 1 < XG) load_group(gl + 1, cur ^ 1);
          } else if constexpr (HA) {
            load_group(gl, cur);
          }
          auto act = [&](int m, int s) -> half8 {
            if constexpr (HA) return Ah[cur][s];
            return *reinterpret_cast<const half8 *>(xb + ((gl * 4 + s) * 4 * TR + 16 * m) * 8);
          };
          auto sums = [&](int m) -> floatx4 {
            if constexpr (BITS == 0) return floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (HA) return xh[cur];
            return *reinterpret_cast<const floatx4 *>(mb + gl * TR + 16 * m);
          };
          // Three or four token tiles: tile m + 1's activations and sums are
          // requested before tile m's MFMAs (tile 0's before the unpacking),
          // so each LDS read's latency passes under other work instead of
          // stalling the MFMA that needs it (two tiles keep reading at the
          // MFMAs: with the prefetch their 7- and 8-bit forms spill).
          constexpr bool PF = MTC >= 3;
          half8 Ac[4], An[4];
          floatx4 xc = {0.f, 0.f, 0.f, 0.f}, xn = {0.f, 0.f, 0.f, 0.f};
          auto load_tile = [&](half8 (&Ad)[4], floatx4 &xd, int m) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Ad[s] = act(m, s);
            xd = sums(m);
          };
          if constexpr (PF) load_tile(Ac, xc, 0);
          uint32_t bq[16];
          if constexpr (HA) {
#pragma unroll
            for (int k = 0; k < 16; ++k) bq[k] = bqh[cur][k];
          } else {
            unpack_base(bw + 2 * g, s_lut, bq);
          }
          // residual fields u = q + 2^(b-1) as the exact fp16 subnormals
          // u * 2^-24; the offset leaves in fp32 with the group sums of x':
          // s_r * (2^24 * sum(u 2^-24 x') - 2^(b-1) * sum(x'))
          uint32_t rq[16];
          if constexpr (BITS > 0) unpack_resid<BITS, true>(rw + g * BITS, rq);
          const float sb = h2f((uint32_t)(w.sb >> (16 * g)) & 0xFFFFu) * kinv;
          float srA = 0.f, srB = 0.f;
          if constexpr (BITS > 0) {
            const float sr = h2f((uint32_t)(w.sr >> (16 * g)) & 0xFFFFu);
            srA = sr * 16777216.0f;
            srB = -sr * (float)(1 << (BITS > 0 ? BITS - 1 : 0));
          }
#pragma unroll
          for (int m = 0; m < MTC; ++m) {
            if constexpr (PF) {
              if (m + 1 < MTC) load_tile(An, xn, m + 1);
            }
            floatx4 aB = {0.f, 0.f, 0.f, 0.f}, aR = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const half8 a = PF ? Ac[s] : act(m, s);
              aB = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_half8(bq + 4 * s), aB, 0, 0, 0);
              if constexpr (BITS > 0)
                aR = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_half8(rq + 4 * s), aR, 0, 0, 0);
            }
            const floatx4 xsv = PF ? xc : sums(m);
            // Draft and verify round identically: with s_r = 0 both residual
            // fmas return accC unchanged, so verify(0 residual) == draft bitwise.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              accC[m][i] = fmaf(sb, aB[i], accC[m][i]);
              if constexpr (BITS > 0) accC[m][i] = fmaf(srA, aR[i], fmaf(srB, xsv[i], accC[m][i]));
            }
            if constexpr (PF) {
#pragma unroll
              for (int s = 0; s < 4; ++s) Ac[s] = An[s];
              xc = xn;
            }
          }
          refill(g);
        }
        if (st == NST - 1) {
#pragma unroll
          for (int m = 0; m < MTC; ++m) {
            const floatx4 ts = *reinterpret_cast<const floatx4 *>(mb + XG * TR + 16 * m);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][i] = fmaf(ts[i], accC[m][i], acc[m][i]);
          }
        }
      }
    };
    // A ring of NS register sets: while one set is computed the other NS - 1
    // are in flight.  NS chunks per trip and no exit in the middle, so the
    // compiler's waits on the weight registers stay counted; requests past
    // the split's last chunk fall outside the descriptors (zeros, no memory
    // access), and the last nchk % NS chunks are computed after the loop.
    constexpr int NS = ring_sets<BITS, MT, TW>();
    WRegs<BITS> w[NS];
    if constexpr (LOCAL) {
      // ---- x' of this K-range, rotated here (the rotation role's arithmetic):
      // tasks (row t, superblock of SB columns), 4096/SB per pass over the
      // first four waves; the fifth wave only keeps the barrier count.  The
      // first pass's x lands before the weights are requested (behind the
      // weight burst of every workgroup it would arrive later); the weight
      // loads are then in flight during the transform.
      const RotInArgs &ra = rot;
      const int SB = ra.SB, TPS = SB >> 4;
      const bool idle = threadIdx.x >= 256;
      const int rtid = idle ? 0 : threadIdx.x, lt = rtid % TPS, tg = rtid / TPS;
      const int kbeg = c_begin * kChunk, kend = c_end * kChunk;
      const int sb0 = kbeg / SB, nsb = (kend - 1) / SB - sb0 + 1;
      const int per_pass = 4096 / SB, ntask = nrows * nsb, npass = (ntask + per_pass - 1) / per_pass;
      const int8_t *sign = L.sign_in;
      float *xs = reinterpret_cast<float *>(smem + LocalPlan::o_f) + tg * (SB + (SB >> 4));
      char *xres = smem + LocalPlan::o_x;
      float *mres = reinterpret_cast<float *>(smem + LocalPlan::o_m);
      XRaw xraw{};
      int t = 0, kb = 0, xrow = -1;
      bool valid = false;
      auto rload = [&](int p) __attribute__((always_inline)) {
        const int task = p * per_pass + tg;
        valid = !idle && task < ntask;
        t = valid ? task % nrows : 0;
        kb = (sb0 + (valid ? task / nrows : 0)) * SB;
        xrow = valid ? row_base + t : -1;
        if (a.lins && valid) {
          xrow = ra.pair_token[row_base + t];
          if (xrow < 0 || xrow >= ra.x_rows) xrow = -1;
        }
        if (idle) return;
        xraw = load_x16(ra.x, sign, xrow, kb + 16 * lt, ra.d_in);  // converted in rproc
      };
      auto rproc = [&]() __attribute__((always_inline)) {
        float v[16];
        cvt_x16(v, xraw);
        fwht_b(v, xs, lt, ra.lb, idle);
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[j]));
        mx = max_lanes32(mx);
        int sc = 0;
        if (mx > 0.0f) {
          int ex;
          frexpf(mx, &ex);
          sc = 15 - ex;
          sc = sc > 120 ? 120 : (sc < -120 ? -120 : sc);
        }
        uint32_t wv[8];
        float gs = 0.f;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const _Float16 q0 = (_Float16)ldexpf(v[2 * h], sc), q1 = (_Float16)ldexpf(v[2 * h + 1], sc);
          gs += (float)q0 + (float)q1;
          wv[h] = (uint32_t)__builtin_bit_cast(uint16_t, q0) | ((uint32_t)__builtin_bit_cast(uint16_t, q1) << 16);
        }
        gs = sum_lanes8(gs);
        const int k0 = kb + 16 * lt;
        if (!valid || k0 < kbeg || k0 >= kend) return;
        const int cl = (k0 >> 9) - c_begin;
        const int run0 = ((k0 >> 3) & 3) * 4 + ((k0 >> 5) & 3) + ((k0 >> 7) & 3) * 16;
        const int run1 = (((k0 + 8) >> 3) & 3) * 4 + ((k0 >> 5) & 3) + ((k0 >> 7) & 3) * 16;
        *reinterpret_cast<uint4 *>(xres + ((cl * 64 + run0) * TR + t) * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        *reinterpret_cast<uint4 *>(xres + ((cl * 64 + run1) * TR + t) * 16) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
        if ((lt & 7) == 0) mres[(cl * 5 + ((k0 >> 7) & 3)) * TR + t] = gs;
        if ((lt & 31) == 0) mres[(cl * 5 + 4) * TR + t] = ldexpf(ra.rsqrt_b, -sc);
      };
      rload(0);
      fence();
      wait_vm<0>();
      // the fifth wave issues the same loads past its descriptors' range
      // (zeros, no memory access), so every wave counts the same loads
#pragma unroll
      for (int k = 0; k < NS; ++k) loadw(w[k], (loader ? c_end : c_begin) + k);
      rproc();
#pragma unroll 1
      for (int p = 1; p < npass; ++p) {
        rload(p);
        rproc();
      }
      __syncthreads();  // x' resident, lookup table written
    } else {
      fence();
#pragma unroll
      for (int k = 0; k < NS; ++k) loadw(w[k], c_begin + k);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // lookup table written
      __builtin_amdgcn_s_barrier();                         // stage 0 of x' ready
      asm volatile("" ::: "memory");
    }
    if (!loader && (MT >= 3 || NS == 1)) {
      // (three or more token tiles: a chunk's compute is long, so each set is
      // refilled in one piece right after it is computed; a one-set ring
      // has no other set to refill during the compute)
      int ci = 0;
#pragma unroll 1
      for (; ci + NS - 1 < nchk; ci += NS) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          compute(w[k], ci + k, [](int) {});
          fence();
          loadw(w[k], c_begin + ci + k + NS);
        }
      }
#pragma unroll
      for (int k = 0; k < NS - 1; ++k)
        if (ci + k < nchk) compute(w[k], ci + k, [](int) {});
    } else if (!loader) {
      // chunk j is computed from set j % NS while set (j - 1) % NS, computed
      // just before, is refilled with chunk j - 1 + NS; chunk 0 refills
      // nothing.  NS chunks per trip, the last < NS after the loop.
      compute(w[0], 0, [](int) {});
      int j = 1;
#pragma unroll 1
      for (; j + NS <= nchk; j += NS) {
#pragma unroll
        for (int k = 1; k <= NS; ++k) {
          const int s = k % NS, pr = k - 1;
          compute(w[s], j + k - 1, [&](int g) { loadpart(w[pr], c_begin + j + k - 2 + NS, g); });
        }
      }
#pragma unroll
      for (int k = 1; k < NS; ++k)
        if (j + k - 1 < nchk) compute(w[k], j + k - 1, [&](int g) { loadpart(w[k - 1], c_begin + j + k - 2 + NS, g); });
    }
  }

  if constexpr (FUSED && !LOCAL) {
    if (s_lost) {  // written by the loader before the first stage barrier
#pragma unroll
      for (int m = 0; m < MTC; ++m) acc[m] = floatx4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
  }
  const int row = tile * kTileRows + tl;  // output row of this lane (B column)
  const bool store = active && row < a.d_out;
  // multi-linear form: the expert's rows land in its own output from row 0
  // (it runs at 24 tokens and more; the eight-tile-wave variants of one and
  // two token tiles, which short grouped experts take, leave it out and keep
  // their registers)
  constexpr bool OWN = FUSED && !(TW == 8 && MT < 3);
  const bool own_out = OWN && a.ys[0] != nullptr;
  float *const y_own = own_out ? a.ys[min(e, 3)] : nullptr;
  auto put = [&](float *out, size_t ld, bool coh, int rbase) {
    if (!store) return;
#pragma unroll
    for (int m = 0; m < MTC; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m * 16 + 4 * kq + i;
        if (t < nrows) {
          float *p = out + (size_t)(rbase + t) * ld + row;
          if (coh) st_dev(p, acc[m][i]); else *p = acc[m][i];
        }
      }
  };
  if constexpr (!FUSED) {
    put(a.out + split * a.split_stride, a.ldo, false, row_base);
    return;
  } else {
    const int lin = a.lins ? e : 0;
    if (hv.mode == kOutDirect) {
      if (own_out) put(y_own, a.ldo, false, 0); else put(a.out, a.ldo, false, row_base);
      return;
    }
    // Split partials, then the last workgroup of the row block to arrive sums
    // them in split order (deterministic) into y (one-sided) or ysum.
    float *dst = hv.mode == kOutTwoSided ? hv.ysum : hv.y;
    if (hv.S > 1) {
      put(a.out + split * a.split_stride, a.ldo, true, row_base);
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t *cnt = ctr_at(hv.ctr, hv.rb_base + lin * a.n_rb + rb);
        const bool last = ctr_add(cnt, 1u) == (uint32_t)(hv.S - 1);
        if (last) st_dev(cnt, 0u);
        s_flag = last;
      }
      __syncthreads();
      if (!s_flag) return;
      // 16-byte runs in flight per thread: two (measured faster than four
      // wherever the main loop holds many registers); the draft at four token
      // tiles takes four, with which its code needs no private segment;
      // eight tile waves keep the single-output form, with which their
      // allocation stays as it is
      constexpr int RU = TW == 8 ? 0 : (BITS == 0 && MT == 4 ? 4 : 2);
      sum_splits<NT, RU, RB>(a.out, a.split_stride, hv.S, own_out ? y_own : dst, hv.mode == kOutTwoSided, a.ldo,
                             row_base, nrows, rb * RB, min(RB, a.d_out - rb * RB), own_out ? 0 : row_base);
    } else {
      put(dst, a.ldo, hv.mode == kOutTwoSided, row_base);
    }
    if (hv.mode != kOutTwoSided) return;
    // Two-sided: count the row block into each output superblock it overlaps
    // (two at most: a superblock holds at least 512 rows, a row block at most
    // 128, and with seven tile waves the two need not align); a superblock's
    // last row block releases one token per finish task of it.
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int r0 = rb * RB, r1 = min(r0 + RB, a.d_out);  // rows [r0, r1)
      for (int sbi = r0 / hv.sb_rows; sbi <= (r1 - 1) / hv.sb_rows; ++sbi) {
        const int s0 = sbi * hv.sb_rows, s1 = min(s0 + hv.sb_rows, a.d_out);
        const int rb_in_sb = (s1 - 1) / RB - s0 / RB + 1;  // row blocks overlapping [s0, s1)
        uint32_t *cnt = ctr_at(hv.ctr, hv.ob_base + lin * hv.n_sb + sbi);
        if (ctr_add(cnt, 1u) == (uint32_t)(rb_in_sb - 1)) {
          st_dev(cnt, 0u);
          const int tasks = a.lins ? min(a.offsets[e + 1], a.T) - a.offsets[e] : a.T;
          ctr_add(ctr_at(hv.ctr, hv.obr_base + lin * hv.n_sb + sbi), (uint32_t)tasks);
        }
      }
    }
  }
}

template <int BITS, int MT>
__global__ __launch_bounds__(wg_threads(MT)) void gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LdsPlan<BITS, MT>::bytes];
  int rb = blockIdx.x, e = 0;
  if (a.lins) {  // grouped: blockIdx.x = expert * n_rb + row block
    e = rb / a.n_rb;
    rb -= e * a.n_rb;
  }
  Handover hv{};
  const RotInArgs none{};
  contract_body<BITS, MT, false>(a, e, rb, blockIdx.y, smem, hv, none);
}

// ===========================================================================
// Finish: y = S_o H_o y~ per task = (row of y, superblock of SB = max(b, 512)
// output rows), the FWHT of fwht_tasks; without S_o it only sums the splits
// (SB = 4096, same task mapping).  Staged: y~ = sum of the split partials.
// Single launch: y~ comes summed (ysum) once the task's superblock is
// complete, signalled by one token per task.
// ===========================================================================
template <bool FUSED>
__device__ __forceinline__ void finish_body(const FinishArgs &a, int wg, float *xch, float *spare,
                                            const Handover &hv) {
  const int SB = a.OB, TPS = SB >> 4, n = 31 - __builtin_clz(SB);
  const bool extra = threadIdx.x >= 256;
  const int tid = extra ? 0 : threadIdx.x, lt = tid % TPS, tl = tid / TPS;
  const int n_sb = (a.d_out + SB - 1) / SB;
  const int task = wg * (256 / TPS) + tl;
  const bool valid = !extra && task < a.T * n_sb;
  const int t = valid ? task / n_sb : 0, sb = valid ? task % n_sb : 0;
  const int rb = sb * SB;
  float *x = extra ? spare : xch + tl * (SB + (SB >> 4));
  // the output rotation is a property of the call (uniform: fwht_tasks has
  // barriers); lanes without a task read expert 0's signs and store nothing
  const bool rotate_out = a.lins ? a.lins[0].sign_out != nullptr : a.sign_out != nullptr;
  const int8_t *so = a.sign_out;
  int e = 0;
  if (a.lins) {
    if (valid) e = expert_of(a.offsets, a.n_experts, t);
    so = a.lins[e].sign_out;
  }
  float *y = a.y + (size_t)t * a.d_out;
  // single launch with the output rotation: the thread's 16 output signs
  // (inputs of the call), requested before the wait on the superblock so
  // that no load is left after the transform
  const int r0 = rb + 16 * lt;
  int sg[16];
  if constexpr (FUSED) {
    if (rotate_out) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sg[j] = so[min(r0 + j, a.d_out - 1)];
    }
  }
  float v[16];
  if constexpr (FUSED) {
    __shared__ uint32_t s_lost[8];  // per task of the workgroup (256 / TPS <= 8): its wait gave up
    if (lt == 0 && !extra) {
      bool ok = true;
      const bool waits = valid && (!a.lins || (expert_active(a.offsets, e, a.T) && t < a.offsets[e + 1]));
      if (waits) ok = take_token(ctr_at(hv.ctr, hv.obr_base + e * n_sb + sb), hv, ctr_at(hv.ctr, kCtrErr));
      s_lost[tl] = ok ? 0u : 1u;
    }
    __syncthreads();
    const bool lost = !extra && s_lost[tl] != 0u;
    const float *ys = hv.ysum + (size_t)t * a.d_out;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = lost ? __builtin_nanf("") : ld_dev(ys + min(rb + TPS * j + lt, a.d_out - 1));
  } else {
    const float *p = a.part + (size_t)t * a.d_out;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
    // four splits per round, all 64 loads issued before any add; the adds
    // keep the split order, so the sum is deterministic
    for (int sp0 = 0; sp0 < a.S; sp0 += 4) {
      float u[4][16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sp = min(sp0 + q, a.S - 1);
#pragma unroll
        for (int j = 0; j < 16; ++j) u[q][j] = p[sp * a.split_stride + min(rb + TPS * j + lt, a.d_out - 1)];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] += (sp0 + q < a.S) ? u[q][j] : 0.f;
    }
  }
  if (rotate_out) {
    fwht_tasks(v, x, lt, TPS, n, a.lb);
    // layout B: 16 consecutive outputs per thread
    if (!valid) return;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + j;
      if (r < a.d_out) y[r] = v[j] * a.rsqrt_b * (float)(FUSED ? sg[j] : so[r]);
    }
  } else {
    if (!valid) return;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = rb + TPS * j + lt;
      if (r < a.d_out) y[r] = v[j];
    }
  }
}

__global__ __launch_bounds__(256) void finish_kernel(const FinishArgs a) {
  __shared__ float xch[4096 + 256];
  Handover hv{};
  finish_body<false>(a, blockIdx.x, xch, nullptr, hv);
}

// ===========================================================================
// Single-launch forward: workgroups [0, n_rot) rotate x, the next n_gemm
// contract (each once all of x' is stored), the rest (two-sided only)
// finish.  Every wait is on workgroups of lower index.
// ===========================================================================
template <int BITS, int MT, int TW>
__global__ __launch_bounds__(64 * (TW + 1)) void forward_kernel(const FwdArgs f) {
  constexpr int kFwht = (4096 + 256) * 4;  // one workgroup FWHT area (bytes)
  constexpr int kPlan = MT == 0 ? LocalPlan::bytes : LdsPlan<BITS, (MT == 0 ? 1 : MT)>::bytes;
  constexpr int kLds = kPlan > 2 * kFwht ? kPlan : 2 * kFwht;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  float *xch = reinterpret_cast<float *>(smem), *spare = reinterpret_cast<float *>(smem + kFwht);
  int b = blockIdx.x;
  uint32_t *ctr = f.hv.ctr;
  if (b < f.n_rot) {
    rotate_body<true>(f.rot, b, xch, spare);
    // linears whose contraction workgroups will wait: those with rows, up
    // to the number of linear slots in the grid
    const int per = f.g.n_rb * f.hv.S;
    uint32_t n_active = 1;
    if (f.rot.lins) {
      n_active = 0;
      if (threadIdx.x < 64)
        for (int e = threadIdx.x; e < f.rot.n_experts; e += 64) n_active += expert_active(f.rot.offsets, e, f.rot.rows);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) n_active += __shfl_xor(n_active, o, 64);
      n_active = min(n_active, (uint32_t)(f.n_gemm / per));
    }
    // line k is waited on iff some linear has rows and owns a workgroup on it
    const int k = threadIdx.x;
    const bool waiters = n_active > 0 && k < per;
    if (b == 0 && k < 8 && waiters) st_dev(ctr_at(ctr, kCtrActive + k), n_active);
    wait_stores();  // x' and its metadata (and the active count) acknowledged in every thread
    __syncthreads();
    if (k < 8) publish_ready(ctr, f.n_rot, k, waiters);
    return;
  }
  b -= f.n_rot;
  if (b < f.n_gemm) {
    const int per = f.g.n_rb * f.hv.S;
    int e = b / per;
    const int j = b - e * per;
    const int split = j / f.g.n_rb, rb = j - split * f.g.n_rb;
    if (f.g.lins && f.g.slots) {  // slot e of the grid takes the e-th expert with rows
      e = nth_active_expert(f.g.offsets, f.g.n_experts, f.g.T, e);
      if (e < 0) return;
    }
    Handover hv = f.hv;
    hv.line = j & 7;
    contract_body<BITS, MT, true, TW>(f.g, e, rb, split, smem, hv, f.rot);
    // A workgroup that waited on its ready line (thread 0 passed a barrier
    // after the loader's wait) counts itself on the line's exit counter; the
    // line's last one clears the line.  Idle experts neither wait nor count.
    const bool waited = f.n_rot > 0 && (!f.g.lins || f.g.slots || expert_active(f.g.offsets, e, f.g.T));
    if (waited && threadIdx.x == 0) {
      const int k = j & 7;
      const uint32_t per_k = (uint32_t)((per - 1 - k) / 8 + 1);  // workgroups of a linear on line k
      const uint32_t target = ld_dev(ctr_at(ctr, kCtrActive + k)) * per_k;
      if (ctr_add(ctr_at(ctr, kCtrExit + k), 1u) == target - 1) {
        st_dev(ctr_at(ctr, kCtrReady + k), 0u);
        st_dev(ctr_at(ctr, kCtrExit + k), 0u);
        st_dev(ctr_at(ctr, kCtrActive + k), 0u);
      }
    }
    return;
  }
  finish_body<true>(f.fin, b - f.n_gemm, xch, spare, f.hv);
}

// ===========================================================================
// Host launchers
// ===========================================================================
hipError_t launch_repack(const RepackArgs &a, int bits, hipStream_t s) {
  const dim3 grid(a.n_tiles * a.n_chunks);
  switch (bits) {
    case 0: repack_kernel<0><<<grid, 64, 0, s>>>(a); break;
    case 6: repack_kernel<6><<<grid, 64, 0, s>>>(a); break;
    case 7: repack_kernel<7><<<grid, 64, 0, s>>>(a); break;
    case 8: repack_kernel<8><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int bits, int ntiles, hipStream_t s) {
  const dim3 grid(ntiles * a.n_chunks);
  switch (bits) {
    case 0: decode_kernel<0><<<grid, 64, 0, s>>>(a); break;
    case 6: decode_kernel<6><<<grid, 64, 0, s>>>(a); break;
    case 7: decode_kernel<7><<<grid, 64, 0, s>>>(a); break;
    case 8: decode_kernel<8><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int rotate_workgroups(int rows, int Kp, int SB, int groups) {
  const int tasks = rows * (Kp / SB), per_wg = (groups > 1 ? groups : 1) * (4096 / SB);
  return (tasks + per_wg - 1) / per_wg;
}

int finish_workgroups(int rows, int d_out, int OB) {
  const int tasks = rows * ((d_out + OB - 1) / OB), per_wg = 4096 / OB;
  return (tasks + per_wg - 1) / per_wg;
}

hipError_t launch_rotate_in(const RotInArgs &a, int rows, hipStream_t s) {
  if (a.SB < 512 || a.SB > 4096) return hipErrorInvalidValue;
  rotate_in_kernel<<<dim3(rotate_workgroups(rows, a.Kp, a.SB)), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_gemm_bits(const GemmArgs &a, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: gemm_kernel<BITS, 1><<<grid, wg_threads(1), 0, s>>>(a); break;
    case 2: gemm_kernel<BITS, 2><<<grid, wg_threads(2), 0, s>>>(a); break;
    case 3: gemm_kernel<BITS, 3><<<grid, wg_threads(3), 0, s>>>(a); break;
    case 4: gemm_kernel<BITS, 4><<<grid, wg_threads(4), 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, int bits, int mt, int splits, hipStream_t s) {
  const dim3 grid(a.n_rb * (a.lins ? a.n_experts : 1), splits);
  switch (bits) {
    case 0: return launch_gemm_bits<0>(a, mt, grid, s);
    case 6: return launch_gemm_bits<6>(a, mt, grid, s);
    case 7: return launch_gemm_bits<7>(a, mt, grid, s);
    case 8: return launch_gemm_bits<8>(a, mt, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_finish(const FinishArgs &a, hipStream_t s) {
  if (a.OB < 512 || a.OB > 4096) return hipErrorInvalidValue;
  finish_kernel<<<dim3(finish_workgroups(a.T, a.d_out, a.OB)), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, int MT, int TW>
static void launch_forward_mt(const FwdArgs &f, dim3 grid, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0)
    hipExtLaunchKernelGGL(forward_kernel<BITS, MT, TW>, grid, dim3(64 * (TW + 1)), 0, s, ev0, ev1, 0, f);
  else
    forward_kernel<BITS, MT, TW><<<grid, 64 * (TW + 1), 0, s>>>(f);
}

// (mt, tw): the pairs the planner picks (tile_waves, and eight tile waves for
// one or two token tiles of short grouped linears).
template <int BITS>
static hipError_t launch_forward_bits(const FwdArgs &f, int mt, int tw, dim3 grid, hipStream_t s, hipEvent_t ev0,
                                      hipEvent_t ev1) {
  switch (mt * 16 + tw) {
    case 0 * 16 + 4: launch_forward_mt<BITS, 0, 4>(f, grid, s, ev0, ev1); break;
    case 1 * 16 + 4: launch_forward_mt<BITS, 1, 4>(f, grid, s, ev0, ev1); break;
    case 1 * 16 + 8: launch_forward_mt<BITS, 1, 8>(f, grid, s, ev0, ev1); break;
    case 2 * 16 + 4: launch_forward_mt<BITS, 2, 4>(f, grid, s, ev0, ev1); break;
    case 2 * 16 + 8: launch_forward_mt<BITS, 2, 8>(f, grid, s, ev0, ev1); break;
    case 3 * 16 + 8: launch_forward_mt<BITS, 3, 8>(f, grid, s, ev0, ev1); break;
    case 4 * 16 + 7: launch_forward_mt<BITS, 4, 7>(f, grid, s, ev0, ev1); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs &f, int bits, int mt, int tw, int n_fin, hipStream_t s, hipEvent_t ev0,
                          hipEvent_t ev1) {
  if (f.rot.SB < 512 || f.rot.SB > 4096) return hipErrorInvalidValue;
  if (f.hv.mode == kOutTwoSided && (f.fin.OB < 512 || f.fin.OB > 4096)) return hipErrorInvalidValue;
  const dim3 grid(f.n_rot + f.n_gemm + n_fin);
  switch (bits) {
    case 0: return launch_forward_bits<0>(f, mt, tw, grid, s, ev0, ev1);
    case 6: return launch_forward_bits<6>(f, mt, tw, grid, s, ev0, ev1);
    case 7: return launch_forward_bits<7>(f, mt, tw, grid, s, ev0, ev1);
    case 8: return launch_forward_bits<8>(f, mt, tw, grid, s, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nl
