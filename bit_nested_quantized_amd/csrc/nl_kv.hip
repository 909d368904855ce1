// nl_kv.hip -- the nested KV cache and the tree-masked attention over it
// (include/nested_kv.h).
//
// kv_write_kernel: one wave per 128-value row; lane l holds dimensions 2l and
// 2l + 1 (one byte of each plane).  The row maximum is a wave reduction.
//
// kv_attn_kernel: one workgroup per (span of positions, KV head), at most 64
// spans per head.  For each 64-position sub-chunk it decodes the K and V rows
// into LDS as the exact integer codes (16 q4 + q_r for KV8, q4 for KV4; the
// row scale is applied to the score and to the softmax weight), then four
// lanes per query row (32 dimensions each) run an online softmax over the
// visible keys, eight keys per rescale.  Partial (max, sum, output) per span
// go to the workspace; kv_combine_kernel merges them.
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
  int G;           // key groups per query row (power of two, <= 16)
};

template <bool VERIFY>
__global__ __launch_bounds__(1024) void kv_attn_kernel(AttnArgs a) {
  __shared__ float kc[kChunk][kD + 4];
  __shared__ float vc[kChunk][kD + 4];
  __shared__ float ksc[kChunk], vsc[kChunk];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int P = a.L + a.T;
  const int pb = c * a.span, pe = min(pb + a.span, P);
  // thread = (query row, dimension quarter, key group): the G key groups of
  // a (row, quarter) are adjacent lanes and the 4 quarters of a (row, group)
  // are G lanes apart, so both reductions are lane exchanges in one wave
  const int G = a.G, grp = tid & (G - 1), part = (tid / G) & 3, r = tid / (4 * G);
  const bool act = r < a.RQ;
  const int t = act ? r / a.g : 0, j = h * a.g + (act ? r % a.g : 0);
  float q[32];
  const float qs = 0.08838834764831845f;   // 1/sqrt(128)
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + ((size_t)t * a.H_q + j) * kD + part * 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 v = qp[u];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q[u * 8 + 2 * k] = __uint_as_float(w[k] << 16) * qs;
        q[u * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u) * qs;
      }
    }
  }
  const uint64_t am = a.anc[t];
  // keys in blocks of 8: eight independent dot products, one block maximum,
  // one rescale of the running output per block
  constexpr int kB = 8;
  float m = -INFINITY, l = 0.0f, o[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) o[k] = 0.0f;
  for (int p0 = pb; p0 < pe; p0 += kChunk) {
    const int nk = min(kChunk, pe - p0);
    __syncthreads();   // the previous sub-chunk's LDS reads are done
    // decode: item = (key, plane K or V, 16-byte piece)
    for (int it = tid; it < nk * 8; it += blockDim.x) {
      const int key = it >> 3, isv = (it >> 2) & 1, pc = it & 3;
      const size_t row = (size_t)(p0 + key) * a.H_kv + h;
      const uint8_t *bp = (isv ? a.vb : a.kb) + row * 64 + pc * 16;
      const uint4 b = *reinterpret_cast<const uint4 *>(bp);
      uint4 rf = make_uint4(0, 0, 0, 0);
      if constexpr (VERIFY) rf = *reinterpret_cast<const uint4 *>((isv ? a.vr : a.kr) + row * 64 + pc * 16);
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w}, rw[4] = {rf.x, rf.y, rf.z, rf.w};
      float *dst = (isv ? vc[key] : kc[key]) + pc * 32;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          dst[w4 * 8 + i] = VERIFY ? (float)(16 * nib(bw[w4], i) + nib(rw[w4], i)) : (float)nib(bw[w4], i);
      if (pc == 0) {
        const float sc = (isv ? a.vs : a.ks)[row] * (VERIFY ? 0.0625f : 1.0f);
        if (isv) vsc[key] = sc; else ksc[key] = sc;
      }
    }
    __syncthreads();

    // this group's keys: grp, grp + G, ... of the sub-chunk
    const int nkg = (nk - grp + G - 1) / G;
    for (int k0 = 0; k0 < nkg; k0 += kB) {
      float sc[kB];
#pragma unroll 2
      for (int u = 0; u < kB; ++u) {
        const int key = grp + G * min(k0 + u, max(nkg - 1, 0));
        const float *kr = kc[min(key, nk - 1)] + part * 32;
        float dot = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) dot += q[k] * kr[k];
        sc[u] = dot;
      }
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        sc[u] += __shfl_xor(sc[u], G);
        sc[u] += __shfl_xor(sc[u], 2 * G);
        const int key = min(grp + G * (k0 + u), nk - 1), pos = p0 + key;   // clamped: in bounds
        const bool vis = k0 + u < nkg && (pos < a.L || ((am >> (pos - a.L)) & 1ull));
        sc[u] = vis ? sc[u] * ksc[key] : -INFINITY;
        bm = fmaxf(bm, sc[u]);
      }
      if (bm == -INFINITY) continue;   // nothing visible in this block
      const float mn = fmaxf(m, bm);
      const float al = expf(m - mn);
      l *= al;
#pragma unroll
      for (int k = 0; k < 32; ++k) o[k] *= al;
#pragma unroll 1
      for (int u = 0; u < kB; ++u) {
        if (sc[u] == -INFINITY) continue;
        const int key = grp + G * (k0 + u);
        const float be = expf(sc[u] - mn);
        l += be;
        const float wv = be * vsc[key];
        const float *vr = vc[key] + part * 32;
#pragma unroll
        for (int k = 0; k < 32; ++k) o[k] += wv * vr[k];
      }
      m = mn;
    }
  }
  // merge the G key groups' (max, sum, output) of each (row, quarter)
  for (int st = 1; st < G; st <<= 1) {
    const float mo = __shfl_xor(m, st), lo = __shfl_xor(l, st);
    const float M = fmaxf(m, mo);
    const float wa = M == -INFINITY ? 0.0f : expf(m - M), wb = M == -INFINITY ? 0.0f : expf(mo - M);
    l = l * wa + lo * wb;
#pragma unroll
    for (int k = 0; k < 32; ++k) o[k] = o[k] * wa + __shfl_xor(o[k], st) * wb;
    m = M;
  }
  if (act && grp == 0) {
    const size_t base = ((size_t)c * a.H_kv + h) * a.RQ + r;
    float4 *op = reinterpret_cast<float4 *>(a.part_o + base * kD + part * 32);
#pragma unroll
    for (int u = 0; u < 8; ++u) op[u] = make_float4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
    if (part == 0) {
      a.part_ml[base * 2] = m;
      a.part_ml[base * 2 + 1] = l;
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
  // key groups: as many as keep 4 * RQ * G <= 1024 threads, at most 16
  // (a power of two); at least 256 threads share the decode
  a.G = 1;
  while (a.G < 16 && 4 * a.RQ * a.G * 2 <= 1024) a.G *= 2;
  const int threads = std::max(256, (4 * a.RQ * a.G + 63) / 64 * 64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (verify)
    hipLaunchKernelGGL(kv_attn_kernel<true>, dim3((unsigned)chunks, (unsigned)H_kv), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(kv_attn_kernel<false>, dim3((unsigned)chunks, (unsigned)H_kv), dim3(threads), 0, s, a);
  if (nl_status st = launched(who)) return st;
  hipLaunchKernelGGL(kv_combine_kernel, dim3((unsigned)a.RQ, (unsigned)H_kv), dim3(256), 0, s, a, chunks, out);
  return launched(who);
}
