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
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "nl_kernels.h"

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

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
  __shared__ uint32_t lut[16];
  const int lane = threadIdx.x;
  if (lane < 16) {
    // fp16 of the codes themselves: 0, 1, 2, 3
    const uint32_t h[4] = {0x0000u, 0x3C00u, 0x4000u, 0x4200u};
    lut[lane] = h[lane & 3] | (h[lane >> 2] << 16);
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

// ===========================================================================
// Input rotation (POC section 1: x' = H_i S_i x, "once per Linear").
// One workgroup per (row of x', superblock of SB columns); SB = max(b, 512)
// so every 512-column chunk lies in one workgroup.  The butterflies run
// unnormalised in fp32 in LDS; each chunk is then scaled by 2^s (s chosen so
// its largest magnitude lands in [2^14, 2^15)) and rounded to fp16, the
// kernels' MFMA operand.  tsc = 2^-s / sqrt(b) undoes both factors.
// ===========================================================================
__global__ __launch_bounds__(256) void rotate_in_kernel(const RotInArgs a) {
  __shared__ float v[4096];
  __shared__ float red[8][4];
  __shared__ int s_exp[8];
  const int row = blockIdx.x, sbk = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int k0 = sbk * a.SB;

  int xrow = row;
  const int8_t *sign = a.sign;
  if (a.lins) {  // grouped: pair -> (token, expert)
    xrow = a.pair_token[row];
    if (xrow < 0 || xrow >= a.x_rows) xrow = -1;
    int lo = 0, hi = a.n_experts;  // largest e with offsets[e] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= row) lo = mid; else hi = mid;
    }
    sign = a.lins[lo].sign_in;
  }
  const uint16_t *xr = a.x + (size_t)(xrow < 0 ? 0 : xrow) * a.d_in;
  for (int i = tid; i < a.SB; i += 256) {
    const int k = k0 + i;
    v[i] = (k < a.d_in && xrow >= 0) ? bf16_to_float(xr[k]) * (float)sign[k] : 0.0f;
  }
  __syncthreads();
  for (int h = 1; h < a.b; h <<= 1) {
    for (int p = tid; p < (a.SB >> 1); p += 256) {
      const int i = ((p / h) * 2 * h) + (p % h);
      const float x0 = v[i], x1 = v[i + h];
      v[i] = x0 + x1;
      v[i + h] = x0 - x1;
    }
    __syncthreads();
  }
  const int nck = a.SB / kChunk;
  for (int cc = 0; cc < nck; ++cc) {
    float m = fmaxf(fabsf(v[cc * kChunk + tid]), fabsf(v[cc * kChunk + 256 + tid]));
    m = wave_max(m);
    if (lane == 0) red[cc][wave] = m;
  }
  __syncthreads();
  if (tid < nck) {
    const float m = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
    int e = 0;
    int s = 0;
    if (m > 0.0f) {
      frexpf(m, &e);
      s = 15 - e;
      s = s > 120 ? 120 : (s < -120 ? -120 : s);
    }
    s_exp[tid] = s;
    a.tsc[(size_t)row * a.n_chunks + k0 / kChunk + tid] = ldexpf(a.rsqrt_b, -s);
  }
  __syncthreads();
  uint16_t *xo = a.xh + (size_t)row * a.Kp + k0;
  for (int cc = 0; cc < nck; ++cc) {
    const int s = s_exp[cc];
    float gs[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int i = cc * kChunk + hh * 256 + tid;
      const _Float16 q = (_Float16)ldexpf(v[i], s);
      xo[i] = __builtin_bit_cast(uint16_t, q);
      gs[hh] = wave_sum((float)q);
    }
    // wave w covers columns [64w, 64w + 64) of each half: groups 2*hh + (w >> 1)
    __syncthreads();
    if (lane == 0) { red[0][wave] = gs[0]; red[1][wave] = gs[1]; }
    __syncthreads();
    if (tid < 4) {
      const int hh = tid >> 1, w2 = (tid & 1) * 2;
      a.xs[(size_t)row * a.Gp + k0 / kGroup + cc * 4 + tid] = red[hh][w2] + red[hh][w2 + 1];
    }
  }
}

// ===========================================================================
// Fused contraction.  Workgroup = 4 waves = 4 row tiles (64 rows) over a
// K-range of `cps` chunks (split-K index blockIdx.y).  The workgroup stages
// WCH chunks of x' at a time in LDS; each wave streams its own tile's codes
// from HBM with a one-chunk register prefetch.
// Per group: base and residual planes -> fp16 B operands; 4 MFMA steps per
// plane and token tile; fp32 epilogue
//   acc_chunk = fma(s_b / kappa, A_base, acc_chunk)
//   acc_chunk = fma(s_r, A_resid - bias * sum(x'), acc_chunk)
// and at the end of each chunk acc += tsc * acc_chunk.
// ===========================================================================
template <int BITS, int MT>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  constexpr int WCH = (MT == 1) ? 2 : 1;
  constexpr int XROW = WCH * kChunk + 8;  // fp16 per LDS row (+16 B pad)
  constexpr int NR = MT * 16;
  __shared__ uint32_t s_lut[16];
  __shared__ float s_xsb[NR][WCH * 4];
  __shared__ float s_tsc[NR][WCH];
  __shared__ __attribute__((aligned(16))) _Float16 s_x[NR * XROW];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int rb = blockIdx.x;
  const LinearDev *Lp = &a.lin;
  int row_base = 0, nrows = a.T;
  if (a.lins) {  // grouped: blockIdx.x = expert * n_rb + row block
    const int e = rb / a.n_rb;
    rb -= e * a.n_rb;
    row_base = a.offsets[e];
    nrows = a.offsets[e + 1] - row_base;
    // idle expert (or offsets outside [0, rows)): uniform exit before any barrier
    if (nrows <= 0 || row_base < 0 || row_base >= a.T) return;
    nrows = min(min(nrows, NR), a.T - row_base);
    Lp = a.lins + e;
  }
  const LinearDev &L = *Lp;
  const int tile = rb * 4 + wave;
  const bool active = tile < a.n_tiles;
  const int c_begin = blockIdx.y * a.cps;
  const int c_end = min(a.n_chunks, c_begin + a.cps);
  if (threadIdx.x < 16) s_lut[threadIdx.x] = L.lut[threadIdx.x];
  const float kinv = L.kinv;
  const int tokl = lane & 15, kq = lane >> 4;
  const float bias = BITS > 0 ? resid_bias(BITS > 0 ? BITS : 8) : 0.0f;

  floatx4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto fill = [&](int c0) {
    const int nw = min(WCH, c_end - c0);
    __syncthreads();
    const int per_row = nw * (kChunk / 8);
    for (int idx = threadIdx.x; idx < nrows * per_row; idx += 256) {
      const int t = idx / per_row, u = idx - t * per_row;
      const uint4 val = *reinterpret_cast<const uint4 *>(
          a.xh + (size_t)(row_base + t) * a.Kp + (size_t)c0 * kChunk + u * 8);
      *reinterpret_cast<uint4 *>(s_x + t * XROW + u * 8) = val;
    }
    for (int idx = threadIdx.x; idx < nrows * nw * 4; idx += 256) {
      const int t = idx / (nw * 4), gg = idx - t * (nw * 4);
      s_xsb[t][gg] = bias * a.xs[(size_t)(row_base + t) * a.Gp + c0 * 4 + gg];
    }
    for (int idx = threadIdx.x; idx < nrows * nw; idx += 256) {
      const int t = idx / nw, cc = idx - t * nw;
      s_tsc[t][cc] = a.tsc[(size_t)(row_base + t) * a.n_chunks + c0 + cc];
    }
    __syncthreads();
  };

  auto process = [&](const ChunkRegs<BITS> &w, int ci) {
    const uint32_t *bw = reinterpret_cast<const uint32_t *>(w.b);
    const uint32_t *rw = reinterpret_cast<const uint32_t *>(w.r);
    floatx4 accC[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) accC[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
      uint32_t bq[16];
      unpack_base(bw + 2 * g, s_lut, bq);
      uint32_t rq[16];
      if constexpr (BITS > 0) unpack_resid<BITS>(rw + g * BITS, rq);
      const uint32_t sbh = (g < 2 ? w.sb.x : w.sb.y) >> (16 * (g & 1));
      const float sb = h2f(sbh & 0xFFFFu) * kinv;
      float sr = 0.f;
      if constexpr (BITS > 0) sr = h2f(((g < 2 ? w.sr.x : w.sr.y) >> (16 * (g & 1))) & 0xFFFFu);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        floatx4 aB = {0.f, 0.f, 0.f, 0.f}, aR = {0.f, 0.f, 0.f, 0.f};
        const int t = m * 16 + tokl;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          half8 A = {0, 0, 0, 0, 0, 0, 0, 0};
          if (t < nrows)
            A = *reinterpret_cast<const half8 *>(s_x + t * XROW + ci * kChunk + g * kGroup +
                                                 32 * kq + 8 * s);
          aB = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(bq + 4 * s), aB, 0, 0, 0);
          if constexpr (BITS > 0)
            aR = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(rq + 4 * s), aR, 0, 0, 0);
        }
        // Draft and verify round identically: with s_r = 0 the residual
        // fma returns accC unchanged, so verify(0 residual) == draft bitwise.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = m * 16 + 4 * kq + i;
          accC[m][i] = fmaf(sb, aB[i], accC[m][i]);
          if constexpr (BITS > 0) accC[m][i] = fmaf(sr, aR[i] - s_xsb[tt][ci * 4 + g], accC[m][i]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = m * 16 + 4 * kq + i;
        acc[m][i] = fmaf(s_tsc[tt][ci], accC[m][i], acc[m][i]);
      }
  };

  ChunkRegs<BITS> w0, w1;
  if (active && c_begin < c_end) load_chunk<BITS>(w0, L, a.n_chunks, tile, c_begin, lane);
  for (int c = c_begin; c < c_end; c += 2) {
    if (active && c + 1 < c_end) load_chunk<BITS>(w1, L, a.n_chunks, tile, c + 1, lane);
    if ((c - c_begin) % WCH == 0) fill(c);
    if (active) process(w0, (c - c_begin) % WCH);
    if (c + 1 < c_end) {
      if (active && c + 2 < c_end) load_chunk<BITS>(w0, L, a.n_chunks, tile, c + 2, lane);
      if ((c + 1 - c_begin) % WCH == 0) fill(c + 1);
      if (active) process(w1, (c + 1 - c_begin) % WCH);
    }
  }

  if (!active) return;
  const int row = tile * kTileRows + tokl;  // output row of this lane (B column)
  if (row >= a.d_out) return;
  float *out = a.out + blockIdx.y * a.split_stride;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = m * 16 + 4 * kq + i;
      if (t < nrows) out[(size_t)(row_base + t) * a.ldo + row] = acc[m][i];
    }
}

// ===========================================================================
// Finish: y = S_o H_o (sum over splits of the partial y~) per (row of y,
// output block of b rows); without S_o it only sums the splits.
// ===========================================================================
__global__ __launch_bounds__(256) void finish_kernel(const FinishArgs a) {
  __shared__ float v[4096];
  const int t = blockIdx.x, r0 = blockIdx.y * a.OB;
  const int tid = threadIdx.x;
  const int n = min(a.OB, a.d_out - r0);
  const int8_t *so = a.sign_out;
  if (a.lins) {
    int lo = 0, hi = a.n_experts;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= t) lo = mid; else hi = mid;
    }
    so = a.lins[lo].sign_out;
  }
  const float *p = a.part + (size_t)t * a.d_out + r0;
  float *y = a.y + (size_t)t * a.d_out + r0;
  if (!so) {
    for (int i = tid; i < n; i += 256) {
      float s = 0.f;
      for (int sp = 0; sp < a.S; ++sp) s += p[sp * a.split_stride + i];
      y[i] = s;
    }
    return;
  }
  for (int i = tid; i < n; i += 256) {
    float s = 0.f;
    for (int sp = 0; sp < a.S; ++sp) s += p[sp * a.split_stride + i];
    v[i] = s;
  }
  __syncthreads();
  for (int h = 1; h < a.b; h <<= 1) {
    for (int q = tid; q < (n >> 1); q += 256) {
      const int i = ((q / h) * 2 * h) + (q % h);
      const float x0 = v[i], x1 = v[i + h];
      v[i] = x0 + x1;
      v[i + h] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = tid; i < n; i += 256) y[i] = v[i] * a.rsqrt_b * (float)so[r0 + i];
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

hipError_t launch_rotate_in(const RotInArgs &a, int rows, hipStream_t s) {
  const dim3 grid(rows, a.Kp / a.SB);
  rotate_in_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_gemm_bits(const GemmArgs &a, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: gemm_kernel<BITS, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: gemm_kernel<BITS, 2><<<grid, 256, 0, s>>>(a); break;
    case 3: gemm_kernel<BITS, 3><<<grid, 256, 0, s>>>(a); break;
    case 4: gemm_kernel<BITS, 4><<<grid, 256, 0, s>>>(a); break;
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
  const dim3 grid(a.T, (a.d_out + a.OB - 1) / a.OB);
  finish_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nl
