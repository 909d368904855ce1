// nl_kv.hip -- the nested KV cache and the tree-masked attention over it
// (include/nested_kv.h).
//
// kv_write_kernel: one wave per 128-value row; lane l holds dimensions 2l and
// 2l + 1 (one byte of each plane).  The row maximum is a wave reduction.
//
// kv_attn_mfma_kernel: one workgroup per (span of positions, KV head, block
// of 64 query rows), at most 64 spans per head.  For each 64-position
// sub-chunk it decodes the K and V rows into LDS as the exact integer codes
// (16 q4 + q_r for KV8, q4 for KV4; the row scales are applied to the score
// and to the softmax weight), and both products run on the matrix cores.
// Partial (max, sum, output) per span go to the workspace; kv_combine_kernel
// merges them.
#include <hip/hip_runtime.h>

#include <algorithm>
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

__device__ __forceinline__ int nib(uint32_t w, int i) {   // two's-complement nibble i of w
  return ((int)(w << (28 - 4 * i))) >> 28;
}

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
  float *part_ml;  // [chunks][H_kv][RQ][2]
  int T, H_q, H_kv, L, g, RQ;
  int span;        // key positions per workgroup (a multiple of 64)
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ _Float16 code(uint32_t b, uint32_t r, int i, bool verify) {
  return (_Float16)(verify ? 16 * nib(b, i) + nib(r, i) : nib(b, i));   // |code| <= 136: exact
}

// MFMA attention: one workgroup of four waves per (span, KV head, block of
// 64 query rows); wave w owns the 16 rows 64 z + 16 w .. +15 (rows past RQ
// are zero queries whose results are dropped).  Per 64-key sub-chunk the
// four waves decode K key-major and V dimension-major into LDS as fp16
// integer codes (exact), then each wave with live rows computes
//   S = Q K^T        16 v_mfma_f32_16x16x32_f16 (4 key tiles x 4 dim steps),
//                    Q widened to fp16 with a power of two per row (exact
//                    unless an element is below 2^-30 of its row maximum);
//   online softmax   one rescale per sub-chunk, row reductions across the
//                    16 key lanes of the C layout;
//   O += P' V        32 MFMAs: P' = p * v_scale / (largest v_scale of the
//                    sub-chunk) goes through a per-wave LDS tile as an fp16
//                    pair hi + lo (about 22 significant bits), and the
//                    sub-chunk's product is scaled back in fp32.
// C layout of a 16x16 tile: lane (lr = lane & 15, lg = lane >> 4) holds rows
// 4 lg .. 4 lg + 3 of column lr; an A/B operand lane holds row/column lr and
// the 8 reduction elements 8 lg .. 8 lg + 7 of a 32-wide step.
template <bool VERIFY>
__global__ __launch_bounds__(256) void kv_attn_mfma_kernel(AttnArgs a) {
  constexpr int kKP = kD + 8;      // K: [key][dim] pitch (halves)
  constexpr int kVP = kChunk + 8;  // V: [dim][key] pitch (halves)
  constexpr int kPP = kChunk + 8;  // P': [row][key] pitch (halves)
  __shared__ __attribute__((aligned(16))) _Float16 kt[kChunk * kKP];
  __shared__ __attribute__((aligned(16))) _Float16 vt[kD * kVP];
  __shared__ __attribute__((aligned(16))) _Float16 pt[4][2][16 * kPP];   // per wave: P' hi, lo
  __shared__ float ksc[kChunk], vsc[kChunk];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int r0 = 64 * blockIdx.z + 16 * wave;   // this wave's first query row
  const bool live = r0 < a.RQ;                   // wave-uniform
  const int P = a.L + a.T;
  const int pb = c * a.span, pe = min(pb + a.span, P);

  // Q operand: row r0 + lr, dimensions 32 st + 8 lg .. +8
  half8 qa[4];
  float qinv[4];
  uint64_t am[4];
  {
    const int qrow = r0 + lr;
    const bool real = qrow < a.RQ;
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
    const float qi = ldexpf(0.08838834764831845f, -qe);   // 2^-qe / sqrt(128)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qinv[i] = __shfl(qi, 4 * lg + i);
      const int row = r0 + 4 * lg + i;
      am[i] = a.anc[row < a.RQ ? row / a.g : 0];
    }
  }

  float m[4], l[4];
  floatx4 o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  _Float16 *ph = pt[wave][0], *pl = pt[wave][1];
  const float unit = VERIFY ? 0.0625f : 1.0f;

  for (int p0 = pb; p0 < pe; p0 += kChunk) {
    const int nk = min(kChunk, pe - p0);   // >= 1; keys past nk repeat key nk - 1 and are masked
    __syncthreads();                       // the previous sub-chunk's LDS reads are done
    for (int it = tid; it < 256; it += blockDim.x) {
      if (it < 128) {   // K: key it / 2, dimensions 64 (it & 1) .. +64
        const int key = it >> 1, hh = it & 1;
        const size_t row = (size_t)(p0 + min(key, nk - 1)) * a.H_kv + h;
        const uint4 *bp = reinterpret_cast<const uint4 *>(a.kb + row * 64 + hh * 32);
        const uint4 b0 = bp[0], b1 = bp[1];
        uint4 q0 = make_uint4(0, 0, 0, 0), q1 = q0;
        if constexpr (VERIFY) {
          const uint4 *rp = reinterpret_cast<const uint4 *>(a.kr + row * 64 + hh * 32);
          q0 = rp[0];
          q1 = rp[1];
        }
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t rw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          half8 hv;
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[i] = code(bw[w], rw[w], i, VERIFY);
          *reinterpret_cast<half8 *>(kt + key * kKP + hh * 64 + 8 * w) = hv;
        }
        if (hh == 0) ksc[key] = a.ks[row] * unit;
      } else {          // V: keys 8 kg .. +8 x dimensions 8 dg .. +8, stored transposed
        const int dg = it & 15, kg = (it >> 4) & 7;
        uint32_t bw[8], rw[8];
        size_t rows[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          rows[kk] = (size_t)(p0 + min(8 * kg + kk, nk - 1)) * a.H_kv + h;
          bw[kk] = reinterpret_cast<const uint32_t *>(a.vb + rows[kk] * 64)[dg];
          rw[kk] = VERIFY ? reinterpret_cast<const uint32_t *>(a.vr + rows[kk] * 64)[dg] : 0u;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          half8 hv;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) hv[kk] = code(bw[kk], rw[kk], i, VERIFY);
          *reinterpret_cast<half8 *>(vt + (8 * dg + i) * kVP + 8 * kg) = hv;
        }
        if (dg == 0)
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) vsc[8 * kg + kk] = a.vs[rows[kk]] * unit;
      }
    }
    __syncthreads();
    if (!live) continue;

    float vm = vsc[lane];   // largest V scale of the sub-chunk
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) vm = fmaxf(vm, __shfl_xor(vm, o2));
    const float vinv = vm > 0.0f ? 1.0f / vm : 0.0f;

    floatx4 sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const half8 kb8 = *reinterpret_cast<const half8 *>(kt + (16 * t + lr) * kKP + 32 * st + 8 * lg);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[st], kb8, sc[t], 0, 0, 0);
      }
    }
    // lane holds S[row 4 lg + i][key 16 t + lr]
    float tmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 16 * t + lr, pos = p0 + key;
      const float ks = ksc[key];
      const int bit = min(max(pos - a.L, 0), 63);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = key < nk && (pos < a.L || ((am[i] >> bit) & 1ull));
        sc[t][i] = vis ? sc[t][i] * qinv[i] * ks : -INFINITY;
        tmax[i] = fmaxf(tmax[i], sc[t][i]);
      }
    }
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax[i] = fmaxf(tmax[i], __shfl_xor(tmax[i], o2));
    float psum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(m[i], tmax[i]);
      const float al = mn == -INFINITY ? 1.0f : expf(m[i] - mn);
      m[i] = mn;
      l[i] *= al;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d][i] *= al;
      psum[i] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float vs = vsc[16 * t + lr] * vinv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = sc[t][i] == -INFINITY ? 0.0f : expf(sc[t][i] - m[i]);
        psum[i] += p;
        const float x = p * vs;
        const _Float16 hi = (_Float16)x;
        ph[(4 * lg + i) * kPP + 16 * t + lr] = hi;
        pl[(4 * lg + i) * kPP + 16 * t + lr] = (_Float16)(x - (float)hi);   // x - hi is exact
      }
    }
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) psum[i] += __shfl_xor(psum[i], o2);
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] += psum[i];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's P' tile is in LDS

    floatx4 oc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) oc[d] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const half8 pah = *reinterpret_cast<const half8 *>(ph + lr * kPP + 32 * w + 8 * lg);
      const half8 pal = *reinterpret_cast<const half8 *>(pl + lr * kPP + 32 * w + 8 * lg);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const half8 vb8 = *reinterpret_cast<const half8 *>(vt + (16 * d + lr) * kVP + 32 * w + 8 * lg);
        oc[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pah, vb8, oc[d], 0, 0, 0);
        oc[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pal, vb8, oc[d], 0, 0, 0);
      }
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] += vm * oc[d];
  }
  if (!live) return;
  // partials: lane holds O[row 4 lg + i][dimension 16 d + lr]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + 4 * lg + i;
    if (row < a.RQ) {
      const size_t base = ((size_t)c * a.H_kv + h) * a.RQ + row;
#pragma unroll
      for (int d = 0; d < 8; ++d) a.part_o[base * kD + 16 * d + lr] = o[d][i];
      if (lr == 0) {
        a.part_ml[base * 2] = m[i];
        a.part_ml[base * 2 + 1] = l[i];
      }
    }
  }
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
  if (tid < 64) {
    const size_t base = ((size_t)tid * a.H_kv + h) * a.RQ + r;
    const float mc = tid < chunks ? a.part_ml[base * 2] : -INFINITY;
    const float lc = tid < chunks ? a.part_ml[base * 2 + 1] : 0.0f;
    float M = mc;
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float w = mc == -INFINITY ? 0.0f : expf(mc - M);   // a chunk with no visible key weighs 0
    float ls = lc * w;
    for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o);
    wsh[tid] = w;
    if (tid == 0) lsh = ls;
  }
  __syncthreads();
  const int cg = tid >> 6, ld = tid & 63;
  float o0 = 0.0f, o1 = 0.0f;
#pragma unroll 16
  for (int cc = cg; cc < chunks; cc += 4) {
    const float2 v = reinterpret_cast<const float2 *>(a.part_o + (((size_t)cc * a.H_kv + h) * a.RQ + r) * kD)[ld];
    o0 += wsh[cc] * v.x;
    o1 += wsh[cc] * v.y;
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
  const size_t o = (size_t)chunks * H_kv * a.RQ * kD * 4;
  a.part_o = static_cast<float *>(ws);
  a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((o + 255) & ~(size_t)255));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)chunks, (unsigned)H_kv, (unsigned)((a.RQ + 63) / 64));
  if (verify)
    hipLaunchKernelGGL(kv_attn_mfma_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_attn_mfma_kernel<false>, grid, dim3(256), 0, s, a);
  if (nl_status st = launched(who)) return st;
  hipLaunchKernelGGL(kv_combine_kernel, dim3((unsigned)a.RQ, (unsigned)H_kv), dim3(256), 0, s, a, chunks, out);
  return launched(who);
}
