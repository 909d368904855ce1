// nl_kv.hip -- the nested KV cache and the tree-masked attention over it
// (include/nested_kv.h).
//
// kv_write_kernel: one wave per 128-value row; lane l holds dimensions 2l and
// 2l + 1 (one byte of each plane).  The row maximum is a wave reduction.
//
// kv_attn_mfma_kernel: one workgroup per (span of positions, KV head, block
// of 64 query rows; with 16 or fewer rows the waves split keys instead), at
// most 64 spans per head, in an XCD-aware order.  For each 64-position
// sub-chunk it decodes the K and V rows into LDS as the exact integer codes
// (16 q4 + q_r for KV8, q4 for KV4; the row scales are applied to the score
// and to the softmax weight), and both products run on the matrix cores.
// Partial (max, sum, output) per span go to the workspace; kv_combine_kernel
// merges them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/nested_kv.h"

namespace nl {
nl_status api_error(nl_status st, const char *msg);  // nl_api.hip
}

namespace {

constexpr int kD = NL_KV_HEAD_DIM;
constexpr int kChunk = 64;   // key positions per workgroup


__global__ __launch_bounds__(256) void kv_write_kernel(const uint32_t *x, int n, const int32_t *row, uint8_t *base,
                                                       uint8_t *ref, float *scale) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv >= n) return;   // whole waves leave together
  const uint32_t w = x[(size_t)wv * 64 + lane];
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  float m = fmaxf(fabsf(x0), fabsf(x1));
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = __fdiv_rn(m, 7.0f);
  int q0 = 0, q1 = 0, r0 = 0, r1 = 0;
  if (s > 0.0f) {
    const float s16 = __fdiv_rn(s, 16.0f);
    q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(x0, s)), -8.0f), 7.0f);
    q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(x1, s)), -8.0f), 7.0f);
    // the residual x - q4 s, formed exactly and rounded once (one fused multiply-add)
    const float e0 = fmaf(-(float)q0, s, x0);
    const float e1 = fmaf(-(float)q1, s, x1);
    r0 = (int)fminf(fmaxf(rintf(__fdiv_rn(e0, s16)), -8.0f), 7.0f);
    r1 = (int)fminf(fmaxf(rintf(__fdiv_rn(e1, s16)), -8.0f), 7.0f);
  }
  const size_t dst = (size_t)row[wv] * 64 + lane;
  base[dst] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
  ref[dst] = (uint8_t)((r0 & 15) | ((r1 & 15) << 4));
  if (lane == 0) scale[row[wv]] = s;
}

struct AttnArgs {
  const uint16_t *q;
  const uint8_t *kb, *kr, *vb, *vr;
  const float *ks, *vs;
  const uint64_t *anc;
  float *part_o;   // [chunks][H_kv][RQ][128]
  float *part_ml;  // [chunks][H_kv][RQ][2]: running maximum (base-2 units), sum
  int T, H_q, H_kv, L, g, RQ;
  int span;        // key positions per workgroup (a multiple of 64)
  int chunks;      // spans per KV head
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Offset-binary codes of the 8 dimensions in one word of each plane: byte k
// of E holds dimension 2k, byte k of O dimension 2k + 1, as u = 16 (q4 + 8) +
// (q_r + 8) for KV8 or u = q4 + 8 for KV4 (a two's-complement nibble plus 8
// is the nibble with its top bit flipped).
template <bool VERIFY>
__device__ __forceinline__ void ucodes(uint32_t b, uint32_t r, uint32_t &E, uint32_t &O) {
  const uint32_t bx = b ^ 0x88888888u;
  if constexpr (VERIFY) {
    const uint32_t rx = r ^ 0x88888888u;
    E = ((bx & 0x0F0F0F0Fu) << 4) | (rx & 0x0F0F0F0Fu);
    O = (bx & 0xF0F0F0F0u) | ((rx >> 4) & 0x0F0F0F0Fu);
  } else {
    E = bx & 0x0F0F0F0Fu;
    O = (bx >> 4) & 0x0F0F0F0Fu;
  }
}

// fp16 pair {byte K of lo, byte K of hi} as the signed codes: 1024 + u is an
// fp16 integer (bits 0x6400 | u), and subtracting 1024 + the offset is exact.
template <bool VERIFY, int K>
__device__ __forceinline__ uint32_t hpair(uint32_t hi, uint32_t lo) {
  const uint32_t bits = __builtin_amdgcn_perm(hi, lo, K | (0x0c << 8) | ((4 + K) << 16) | (0x0c << 24)) | 0x64006400u;
  const _Float16 off = VERIFY ? (_Float16)1160.0f : (_Float16)1032.0f;
  const half2v h = __builtin_bit_cast(half2v, bits) - half2v{off, off};
  return __builtin_bit_cast(uint32_t, h);
}

// 16-lane row maximum through DPP: swap within pairs, within quads, then
// mirror across the half row and across the row.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  return fmaxf(v, dppf<0x140>(v));
}

// One thread's share of a 64-key sub-chunk: threads 0..127 read half a K
// row (32 bytes of each plane), threads 128..255 one word of each plane of
// 8 V rows.  Loads are issued one sub-chunk ahead of their use.
template <bool VERIFY>
struct Fill {
  uint32_t b[8], r[8];
  float sc[8];
};

// MFMA attention: one workgroup of four waves per (span, KV head, block of
// 64 query rows); wave w owns the 16 rows 64 z + 16 w .. +15 (rows past RQ
// are zero queries whose results are dropped).  Per 64-key sub-chunk
// threads 0..127 decode K key-major and threads 128..255 V dimension-major
// into LDS as fp16 integer codes (exact; the planes are loaded one sub-chunk
// ahead), then each wave with live rows computes, transposed so that a lane
// owns one query row:
//   S^T = K Q^T      16 v_mfma_f32_16x16x32_f16 (4 key tiles x 4 dim steps),
//                    Q widened to fp16 with a power of two per row (exact
//                    unless an element is below 2^-30 of its row maximum);
//   online softmax   in base 2 (log2 e folded into the query scale), one
//                    rescale per sub-chunk; the visibility mask is applied
//                    only where the sub-chunk reaches the tree or the end;
//   O^T += V^T P'^T  32 MFMAs: P' = p * v_scale / (largest v_scale of the
//                    sub-chunk) is an fp16 pair hi + lo (about 22
//                    significant bits) built in registers; O is kept in
//                    units of the latest nonzero such scale.
// C layout of a 16x16 tile: lane (lr = lane & 15, lg = lane >> 4) holds rows
// 4 lg .. 4 lg + 3 of column lr; an A/B operand lane holds row/column lr and
// the 8 reduction elements 8 lg .. 8 lg + 7 of a 32-wide step (any order
// works as long as A and B agree: the P' V step uses keys 4 lg .. +3 and
// 16 + 4 lg .. +3 of each 32-key window, where the S^T tiles left them).
//
// SPLIT (at most 16 query rows per KV head): the four waves share the 16 rows
// and split each sub-chunk's keys, 16 per wave (4 score MFMAs, and the P' V
// step as 16 v_mfma_f32_16x16x16_f16); at the span's end the four softmax
// states merge in the freed K/V tiles.
template <bool VERIFY, bool SPLIT>
__global__ __launch_bounds__(256) void kv_attn_mfma_kernel(AttnArgs a) {
  constexpr int kKP = kD + 8;      // K: [key][dim] pitch (halves)
  constexpr int kVP = kChunk + 8;  // V: [dim][8-key block] pitch (halves); block b of
                                   // dimension row r sits at b ^ ((r >> 4) & 7), which keeps
                                   // the fill's 16-byte stores off shared banks
  __shared__ __attribute__((aligned(16))) _Float16 kt[kChunk * kKP];
  __shared__ __attribute__((aligned(16))) _Float16 vt[kD * kVP];
  __shared__ __attribute__((aligned(16))) float ksc[kChunk], vsc[kChunk];
  // The two KV heads of a pair share every 128-byte line of the cache (64
  // bytes each), so their workgroups get linear ids 8 apart: the dispatcher
  // deals ids round-robin over the 8 XCDs, which puts both on one XCD and
  // its L2 then fetches each line once.  Ids past the last pair exit.
  const int npair = (a.H_kv + 1) >> 1, bid = blockIdx.x, q = (bid >> 4) * 8 + (bid & 7);
  const int c = q / npair, h = 2 * (q % npair) + ((bid >> 3) & 1), tid = threadIdx.x;
  if (c >= a.chunks || h >= a.H_kv) return;   // whole workgroup, before any barrier
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = tid >> 6;
  const int r0 = SPLIT ? 0 : 64 * blockIdx.y + 16 * wave;   // this wave's first query row
  const bool live = r0 < a.RQ;                          // wave-uniform
  const int P = a.L + a.T;
  const int pb = c * a.span, pe = min(pb + a.span, P);

  // Q operand: row r0 + lr, dimensions 32 st + 8 lg .. +8
  const int qrow = r0 + lr;
  const bool real = qrow < a.RQ;
  half8 qa[4];
  float qinv;
  uint64_t am;
  {
    const int t = real ? qrow / a.g : 0, j = h * a.g + (real ? qrow % a.g : 0);
    const uint16_t *qp = a.q + ((size_t)t * a.H_q + j) * kD;
    float qf[32];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 v = *reinterpret_cast<const uint4 *>(qp + 32 * st + 8 * lg);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[8 * st + 2 * k] = real ? __uint_as_float(w[k] << 16) : 0.0f;
        qf[8 * st + 2 * k + 1] = real ? __uint_as_float(w[k] & 0xFFFF0000u) : 0.0f;
      }
    }
    float qm = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) qm = fmaxf(qm, fabsf(qf[k]));
    qm = fmaxf(qm, __shfl_xor(qm, 16));
    qm = fmaxf(qm, __shfl_xor(qm, 32));
    int qe = 0;
    if (qm > 0.0f) {
      int E;
      frexpf(qm, &E);
      qe = 15 - E;   // row maximum * 2^qe in [2^14, 2^15)
    }
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int k = 0; k < 8; ++k) qa[st][k] = (_Float16)ldexpf(qf[8 * st + k], qe);
    qinv = ldexpf(0.12751743082459868f, -qe);   // 2^-qe log2(e) / sqrt(128): scores in base 2
    am = a.anc[t];
  }

  float m = -INFINITY, l = 0.0f, R = 1.0f;   // O = o * R
  floatx4 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  const float unit = VERIFY ? 0.0625f : 1.0f;

  const bool kside = tid < 128;   // wave-uniform
  const int fkey = tid >> 1, fhh = tid & 1;               // K side
  const int fdg = tid & 15, fkg = (tid >> 4) & 7;         // V side
  // V block fkg holds the 8 keys a P'V operand lane reads together: keys
  // 4 (fkg & 3) .. +3 and 16 + 4 (fkg & 3) .. +3 of the 32-key window fkg / 4
  auto vkey = [&](int kk) { return 32 * (fkg >> 2) + 4 * (fkg & 3) + (kk & 3) + 16 * (kk >> 2); };
  const uint32_t rs = (uint32_t)a.H_kv * 64;              // bytes between positions
  Fill<VERIFY> f;
  auto load = [&](int q0) {
    const int n = min(kChunk, pe - q0);   // keys past n repeat key n - 1 (masked later)
    const size_t cr = (size_t)q0 * a.H_kv + h;   // first row of the sub-chunk
    if (kside) {
      const uint32_t kr = (uint32_t)min(fkey, n - 1);
      const uint32_t off = kr * rs + fhh * 32;
      const uint4 *bp = reinterpret_cast<const uint4 *>(a.kb + cr * 64 + off);
      const uint4 b0 = bp[0], b1 = bp[1];
      f.b[0] = b0.x; f.b[1] = b0.y; f.b[2] = b0.z; f.b[3] = b0.w;
      f.b[4] = b1.x; f.b[5] = b1.y; f.b[6] = b1.z; f.b[7] = b1.w;
      if constexpr (VERIFY) {
        const uint4 *rp = reinterpret_cast<const uint4 *>(a.kr + cr * 64 + off);
        const uint4 r0v = rp[0], r1v = rp[1];
        f.r[0] = r0v.x; f.r[1] = r0v.y; f.r[2] = r0v.z; f.r[3] = r0v.w;
        f.r[4] = r1v.x; f.r[5] = r1v.y; f.r[6] = r1v.z; f.r[7] = r1v.w;
      }
      f.sc[0] = a.ks[cr + kr * a.H_kv];
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const uint32_t kr = (uint32_t)min(vkey(kk), n - 1);
        const uint32_t off = kr * rs + fdg * 4;
        f.b[kk] = *reinterpret_cast<const uint32_t *>(a.vb + cr * 64 + off);
        if constexpr (VERIFY) f.r[kk] = *reinterpret_cast<const uint32_t *>(a.vr + cr * 64 + off);
        f.sc[kk] = a.vs[cr + kr * a.H_kv];
      }
    }
  };
  if (pb < pe) load(pb);

  for (int p0 = pb; p0 < pe; p0 += kChunk) {
    const int nk = min(kChunk, pe - p0);   // >= 1; keys past nk are masked
    __syncthreads();                       // the previous sub-chunk's LDS reads are done
    if (kside) {   // K row fkey, dimensions 64 fhh .. +64, key-major
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t E, O;
        ucodes<VERIFY>(f.b[w], f.r[w], E, O);
        uint4 v;
        v.x = hpair<VERIFY, 0>(O, E);
        v.y = hpair<VERIFY, 1>(O, E);
        v.z = hpair<VERIFY, 2>(O, E);
        v.w = hpair<VERIFY, 3>(O, E);
        *reinterpret_cast<uint4 *>(kt + fkey * kKP + fhh * 64 + 8 * w) = v;
      }
      if (fhh == 0) ksc[fkey] = f.sc[0] * unit;
    } else {       // V rows 8 fkg .. +8, dimensions 8 fdg .. +8, dimension-major
      uint32_t E[8], O[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) ucodes<VERIFY>(f.b[kk], f.r[kk], E[kk], O[kk]);
#define NL_VROW(I, X)                                                                             \
  {                                                                                               \
    uint4 v;                                                                                      \
    v.x = hpair<VERIFY, (I) / 2>(X[1], X[0]);                                                     \
    v.y = hpair<VERIFY, (I) / 2>(X[3], X[2]);                                                     \
    v.z = hpair<VERIFY, (I) / 2>(X[5], X[4]);                                                     \
    v.w = hpair<VERIFY, (I) / 2>(X[7], X[6]);                                                     \
    *reinterpret_cast<uint4 *>(vt + (8 * fdg + (I)) * kVP + 8 * (fkg ^ ((fdg >> 1) & 7))) = v;   \
  }
      NL_VROW(0, E) NL_VROW(1, O) NL_VROW(2, E) NL_VROW(3, O)
      NL_VROW(4, E) NL_VROW(5, O) NL_VROW(6, E) NL_VROW(7, O)
#undef NL_VROW
      if (fdg == 0)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) vsc[vkey(kk)] = f.sc[kk] * unit;
    }
    if (p0 + kChunk < pe) load(p0 + kChunk);   // in flight during this sub-chunk's products
    __syncthreads();
    if (!live) continue;

    auto step = [&](auto masked) {
      const float4 v4 = reinterpret_cast<const float4 *>(vsc)[lr];   // largest V scale of the sub-chunk
      const float vm = row_max(fmaxf(fmaxf(v4.x, v4.y), fmaxf(v4.z, v4.w)));
      const float vinv = vm > 0.0f ? 1.0f / vm : 0.0f;
      const float Rn = vm > 0.0f ? vm : R;

      // lane holds S[row lr][key 16 t + 4 lg + i] for this wave's tiles t
      constexpr int NT = SPLIT ? 1 : 4;
      const int t0 = SPLIT ? wave : 0;
      floatx4 sc[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int t = t0 + u;
        floatx4 &sct = sc[u];
        sct = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const half8 kb8 = *reinterpret_cast<const half8 *>(kt + (16 * t + lr) * kKP + 32 * st + 8 * lg);
          sct = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb8, qa[st], sct, 0, 0, 0);
        }
        const float4 k4 = reinterpret_cast<const float4 *>(ksc)[4 * t + lg];
        sct[0] *= qinv * k4.x;
        sct[1] *= qinv * k4.y;
        sct[2] *= qinv * k4.z;
        sct[3] *= qinv * k4.w;
      }
      if constexpr (decltype(masked)::value) {   // the sub-chunk reaches the tree or the span's end
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 16 * (t0 + u) + 4 * lg + i, pos = p0 + key;
            const uint32_t bit = (uint32_t)min(max(pos - a.L, 0), 63);
            const bool vis = (key < nk) & ((pos < a.L) | (((am >> bit) & 1ull) != 0));
            sc[u][i] = vis ? sc[u][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NT; ++u) mx = fmaxf(mx, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float msub = mn == -INFINITY ? 0.0f : mn;   // nothing visible yet: every weight is 2^-inf = 0
      const float al = __builtin_amdgcn_exp2f(m - msub);
      m = mn;
      l *= al;
      const float f_o = al * (R / Rn);
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d] *= f_o;
      R = Rn;
      if constexpr (SPLIT) {
        // P'^T operand of this wave's 16 keys (16 t0 + 4 lg + i); the V^T
        // operand is half of the 8-key block that holds them
        half4 bh, bl;
        const float4 s4 = reinterpret_cast<const float4 *>(vsc)[4 * t0 + lg];
        const float vsk[4] = {s4.x, s4.y, s4.z, s4.w};
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[0][i] - msub);
          ps += p;
          const float x = p * (vsk[i] * vinv);
          const _Float16 hi = (_Float16)x;
          bh[i] = hi;
          bl[i] = (_Float16)(x - (float)hi);   // x - hi is exact
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l += ps;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const half4 va = *reinterpret_cast<const half4 *>(vt + (16 * d + lr) * kVP +
                                                             8 * ((4 * (t0 >> 1) + lg) ^ d) + 4 * (t0 & 1));
          o[d] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, bh, o[d], 0, 0, 0);
          o[d] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, bl, o[d], 0, 0, 0);
        }
        return;
      }
      // P'^T operands of the two 32-key windows: keys 32 w + 4 lg + i (tile 2w)
      // then 32 w + 16 + 4 lg + i (tile 2w + 1)
      half8 bh[2], bl[2];
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 s4 = reinterpret_cast<const float4 *>(vsc)[4 * t + lg];
        const float vsk[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[t][i] - msub);
          ps += p;
          const float x = p * (vsk[i] * vinv);
          const _Float16 hi = (_Float16)x;
          bh[t >> 1][4 * (t & 1) + i] = hi;
          bl[t >> 1][4 * (t & 1) + i] = (_Float16)(x - (float)hi);   // x - hi is exact
        }
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l += ps;
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const half8 va = *reinterpret_cast<const half8 *>(vt + (16 * d + lr) * kVP + 8 * ((4 * w + lg) ^ d));
          o[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, bh[w], o[d], 0, 0, 0);
          o[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, bl[w], o[d], 0, 0, 0);
        }
    };
    if (p0 + kChunk > a.L)
      step(std::true_type{});
    else
      step(std::false_type{});   // context keys only: nothing to mask
  }
  if constexpr (SPLIT) {
    // the four waves' states for the same 16 rows: O (times R) into the
    // freed K/V tiles, (max, sum) into the scale arrays, then wave w merges
    // dimension tiles 2w and 2w + 1
    __syncthreads();
    float *own = reinterpret_cast<float *>(wave < 2 ? static_cast<void *>(kt) : static_cast<void *>(vt)) +
                 (wave & 1) * 16 * kD;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4 *>(own + lr * kD + 16 * d + 4 * lg) =
          make_float4(o[d][0] * R, o[d][1] * R, o[d][2] * R, o[d][3] * R);
    if (lg == 0) {
      ksc[16 * wave + lr] = m;
      vsc[16 * wave + lr] = l;
    }
    __syncthreads();
    float M = -INFINITY, L = 0.0f, ew[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ksc[16 * w + lr]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ksc[16 * w + lr];
      ew[w] = mw == -INFINITY ? 0.0f : exp2f(mw - M);   // a wave that saw no visible key weighs 0
      L += ew[w] * vsc[16 * w + lr];
    }
    if (!real) return;
    const size_t base = ((size_t)c * a.H_kv + h) * a.RQ + qrow;
#pragma unroll
    for (int dd = 2 * wave; dd < 2 * wave + 2; ++dd) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float *src = reinterpret_cast<const float *>(w < 2 ? static_cast<const void *>(kt)
                                                                 : static_cast<const void *>(vt)) +
                           (w & 1) * 16 * kD + lr * kD + 16 * dd + 4 * lg;
        const float4 v = *reinterpret_cast<const float4 *>(src);
        acc.x += ew[w] * v.x;
        acc.y += ew[w] * v.y;
        acc.z += ew[w] * v.z;
        acc.w += ew[w] * v.w;
      }
      *reinterpret_cast<float4 *>(a.part_o + base * kD + 16 * dd + 4 * lg) = acc;
    }
    if (wave == 0 && lg == 0) {
      a.part_ml[base * 2] = M;
      a.part_ml[base * 2 + 1] = L;
    }
    return;
  }
  if (!live || !real) return;
  // partials: lane holds O[row qrow][dimension 16 d + 4 lg + i]
  const size_t base = ((size_t)c * a.H_kv + h) * a.RQ + qrow;
#pragma unroll
  for (int d = 0; d < 8; ++d)
    *reinterpret_cast<float4 *>(a.part_o + base * kD + 16 * d + 4 * lg) =
        make_float4(o[d][0] * R, o[d][1] * R, o[d][2] * R, o[d][3] * R);
  if (lg == 0) {
    a.part_ml[base * 2] = m;
    a.part_ml[base * 2 + 1] = l;
  }
}

// Max and sum over the 64 lanes of a wave (all active): DPP steps within
// rows of 16 lanes (quad swaps, half-row and row mirrors; a shuffle through
// LDS waits ~100 cycles per step), then the four row results read as
// uniform values.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lane(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}

// One workgroup per (KV head, query row): wave 0 turns the chunks' maxima
// and sums into weights (at most 64 chunks, one per lane), then four waves
// add the weighted chunk outputs, all loads in flight, 2 dimensions a lane.
__global__ __launch_bounds__(256) void kv_combine_kernel(AttnArgs a, int chunks, float *out) {
  __shared__ float wsh[64];
  __shared__ float osum[4][kD];
  __shared__ float lsh;
  const int h = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const int t = r / a.g, j = h * a.g + r % a.g;
  const int cg = tid >> 6, ld = tid & 63;
  // every load is issued before any result is needed: each thread's two
  // dimensions of chunks cg, cg + 4, ... and wave 0's (max, sum) pairs
  float2 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int cc = cg + 4 * k;
    v[k] = cc < chunks
               ? reinterpret_cast<const float2 *>(a.part_o + (((size_t)cc * a.H_kv + h) * a.RQ + r) * kD)[ld]
               : make_float2(0.0f, 0.0f);
  }
  if (tid < 64) {
    const size_t base = ((size_t)tid * a.H_kv + h) * a.RQ + r;
    const float mc = tid < chunks ? a.part_ml[base * 2] : -INFINITY;
    const float lc = tid < chunks ? a.part_ml[base * 2 + 1] : 0.0f;
    const float M = wave_max(mc);
    const float w = mc == -INFINITY ? 0.0f : exp2f(mc - M);   // a chunk with no visible key weighs 0
    const float ls = wave_sum(lc * w);
    wsh[tid] = w;
    if (tid == 0) lsh = ls;
  }
  __syncthreads();
  float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int cc = cg + 4 * k;
    const float w = cc < chunks ? wsh[cc] : 0.0f;
    o0 += w * v[k].x;
    o1 += w * v[k].y;
  }
  osum[cg][2 * ld] = o0;
  osum[cg][2 * ld + 1] = o1;
  __syncthreads();
  if (tid < kD)
    out[((size_t)t * a.H_q + j) * kD + tid] = (osum[0][tid] + osum[1][tid] + osum[2][tid] + osum[3][tid]) / lsh;
}

char g_msg[256];

nl_status fail(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
nl_status fail(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return nl::api_error(NL_EINVAL, g_msg);
}

nl_status launched(const char *who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_msg, sizeof g_msg, "%s: launch failed: %s", who, hipGetErrorString(e));
    return nl::api_error(NL_EHIP, g_msg);
  }
  return nl::api_error(NL_OK, "");
}

// Key positions per workgroup: 64-key sub-chunks, as many per workgroup as
// keep the chunks of a head at 64 or fewer (the combine's one-lane-per-chunk
// weights).
int attn_span(int P) { return (P + 64 * kChunk - 1) / (64 * kChunk) * kChunk; }
int attn_chunks(int P) { return (P + attn_span(P) - 1) / attn_span(P); }

size_t attn_ws(int T, int H_q, int H_kv, int L) {
  const int RQ = T * (H_q / H_kv), chunks = attn_chunks(L + T);
  const size_t o = (size_t)chunks * H_kv * RQ * kD * 4;
  return ((o + 255) & ~(size_t)255) + (size_t)chunks * H_kv * RQ * 8;
}

nl_status check_shape(const char *who, int T, int H_q, int H_kv, int L) {
  if (T < 1 || T > NL_MAX_T) return fail("%s: T must be in 1..%d (got %d)", who, NL_MAX_T, T);
  if (H_kv < 1 || H_q < 1 || H_q % H_kv) return fail("%s: H_q must be a positive multiple of H_kv", who);
  if (T * (H_q / H_kv) > NL_KV_MAX_ROWS)
    return fail("%s: T * H_q / H_kv must be at most %d", who, NL_KV_MAX_ROWS);
  if (L < 0) return fail("%s: L must be >= 0", who);
  return NL_OK;
}

}  // namespace

extern "C" nl_status nested_kv_write(const void *x, int32_t n, const int32_t *row, uint8_t *base, uint8_t *ref,
                                     float *scale, void *stream) {
  if (n < 1) return fail("nested_kv_write: n must be >= 1 (got %d)", n);
  if (!x || !row || !base || !ref || !scale) return fail("nested_kv_write: NULL pointer");
  if ((uintptr_t)x & 3) return fail("nested_kv_write: x must be 4-byte aligned");
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint32_t *>(x), n, row, base, ref, scale);
  return launched("nested_kv_write");
}

extern "C" nl_status nested_kv_attention_workspace_bytes(int32_t T, int32_t H_q, int32_t H_kv, int32_t L,
                                                         size_t *bytes) {
  if (nl_status st = check_shape("nested_kv_attention_workspace_bytes", T, H_q, H_kv, L)) return st;
  if (!bytes) return fail("nested_kv_attention_workspace_bytes: bytes is NULL");
  *bytes = attn_ws(T, H_q, H_kv, L);
  return nl::api_error(NL_OK, "");
}

extern "C" nl_status nested_kv_attention(const void *q, int32_t T, int32_t H_q, int32_t H_kv, int32_t L,
                                         const uint8_t *k_base, const uint8_t *k_ref, const float *k_scale,
                                         const uint8_t *v_base, const uint8_t *v_ref, const float *v_scale,
                                         const uint64_t *anc, int32_t verify, float *out, void *ws, size_t ws_bytes,
                                         void *stream) {
  static const char *who = "nested_kv_attention";
  if (nl_status st = check_shape(who, T, H_q, H_kv, L)) return st;
  if (!q || !k_base || !k_scale || !v_base || !v_scale || !anc || !out || !ws) return fail("%s: NULL pointer", who);
  if (verify && (!k_ref || !v_ref)) return fail("%s: verify reads the refinement planes (k_ref, v_ref)", who);
  if (((uintptr_t)q | (uintptr_t)k_base | (uintptr_t)v_base | (uintptr_t)(verify ? k_ref : k_base) |
       (uintptr_t)(verify ? v_ref : v_base)) & 15)
    return fail("%s: q and the planes must be 16-byte aligned", who);
  if (((uintptr_t)ws & 255) || ws_bytes < attn_ws(T, H_q, H_kv, L))
    return fail("%s: needs a 256-byte aligned workspace of %zu bytes", who, attn_ws(T, H_q, H_kv, L));
  AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.kb = k_base;
  a.kr = k_ref;
  a.vb = v_base;
  a.vr = v_ref;
  a.ks = k_scale;
  a.vs = v_scale;
  a.anc = anc;
  a.T = T;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.L = L;
  a.g = H_q / H_kv;
  a.RQ = T * a.g;
  a.span = attn_span(L + T);
  const int chunks = attn_chunks(L + T);
  a.chunks = chunks;
  const size_t o = (size_t)chunks * H_kv * a.RQ * kD * 4;
  a.part_o = static_cast<float *>(ws);
  a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((o + 255) & ~(size_t)255));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int pairs = chunks * ((H_kv + 1) / 2);   // (span, KV-head pair) tasks, 16 ids per 8
  // up to 16 query rows per KV head: the four waves split the keys instead
  const bool split = a.RQ <= 16;
  const dim3 grid((unsigned)((pairs + 7) / 8 * 16), split ? 1u : (unsigned)((a.RQ + 63) / 64));
  if (verify && split)
    hipLaunchKernelGGL((kv_attn_mfma_kernel<true, true>), grid, dim3(256), 0, s, a);
  else if (verify)
    hipLaunchKernelGGL((kv_attn_mfma_kernel<true, false>), grid, dim3(256), 0, s, a);
  else if (split)
    hipLaunchKernelGGL((kv_attn_mfma_kernel<false, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kv_attn_mfma_kernel<false, false>), grid, dim3(256), 0, s, a);
  if (nl_status st = launched(who)) return st;
  hipLaunchKernelGGL(kv_combine_kernel, dim3((unsigned)a.RQ, (unsigned)H_kv), dim3(256), 0, s, a, chunks, out);
  return launched(who);
}
