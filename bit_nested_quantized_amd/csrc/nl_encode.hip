// nl_encode.hip -- the round-to-nearest encoder and the Lloyd-Max level fitter
// (include/nested_encode.h).
//
// Tile kernel: a workgroup of 256 threads owns 4096 consecutive elements of
// the row-major matrix.  d_in is a multiple of 128 and of the Hadamard block
// b (b | 4096), so a tile holds whole blocks and whole 128-groups and never
// mixes rows inside a block.  The fp64 Hadamard butterflies run stride by
// stride (1, 2, 4, ...): four strides in registers per layout, with LDS
// transposes between three layouts of the tile's 12 index bits
//   P1  thread = bits 4..11, register = bits 0..3  (16 consecutive weights)
//   P2  thread = bits 0..3 and 8..11, register = bits 4..7
//   P3  thread = bits 0..7, register = bits 8..11
// and back to P1, where each thread holds an eighth of a 128-group: group
// sums and maxima are three lane exchanges, the thread's 16 codes are two
// bytes of each base plane and 2*b bytes of the residual string.
//
// Column pass (two-sided form): the output-side Hadamard along d_out, one
// workgroup per 2^m rows x 32 columns, m <= 6 of the row bits per pass.
//
// Fitter: an exact radix select (six digit passes over order-preserving
// 64-bit keys) finds the eight order statistics the quantile start needs;
// each Lloyd iteration is one launch whose last workgroup (ticket counter)
// adds the per-workgroup cell sums in workgroup order and moves the levels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/nested_encode.h"

namespace nl {
nl_status api_error(nl_status st, const char *msg);  // nl_api.hip
}

namespace {

constexpr int kTile = 4096;
constexpr int kThreads = 256;
constexpr int kLds = kTile + kTile / 16;  // one pad double per 16

enum Mode { kFused = 0, kRotate = 1, kQuant = 2, kNorm = 3 };



struct TileArgs {
  const float *w;        // fused, rotate: dense fp32 input
  const double *wt;      // quant, norm: rotated fp64 input
  double *out;           // rotate: rotated fp64 output; norm: samples
  const int8_t *sign_in;
  int64_t total;         // d_out * d_in
  int d_in;
  int log2b;             // log2 of the input-side block (7..12)
  double inv;            // 1 / sqrt(b)
  float lev[4];
  int tie_up;            // bit k: a weight on midpoint k takes level k + 1
  int zero_code;         // code of every weight of a zero-scale group
  uint8_t *base;
  uint16_t *bscale;
  uint8_t *resid;
  uint16_t *rscale;
};

// LDS slot of tile index i: i + i/16 (one pad double per 16).  In each layout
// a thread's 16 slots are one base plus constant strides:
//   P1  i = 16t + j                              -> 17t + j
//   P2  i = (t & 15) + 16j + 256(t >> 4)         -> (t & 15) + 272(t >> 4) + 17j
//   P3  i = t + 256j                             -> t + (t >> 4) + 272j
template <int L>
__device__ __forceinline__ int lds_base(int t) {
  if constexpr (L == 1) return 17 * t;
  else if constexpr (L == 2) return (t & 15) + 272 * (t >> 4);
  else return t + (t >> 4);
}
template <int L>
constexpr int lds_stride() { return L == 1 ? 1 : L == 2 ? 17 : 272; }

template <int L>
__device__ __forceinline__ void lds_put(double *s, const double (&v)[16], int t) {
  double *p = s + lds_base<L>(t);
#pragma unroll
  for (int j = 0; j < 16; ++j) p[j * lds_stride<L>()] = v[j];
}

template <int L>
__device__ __forceinline__ void lds_get(const double *s, double (&v)[16], int t) {
  const double *p = s + lds_base<L>(t);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = p[j * lds_stride<L>()];
}

// Butterflies (a, c) -> (a + c, a - c) over register-index bit M.
template <int M>
__device__ __forceinline__ void reg_stage(double (&v)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (!(j & (1 << M))) {
      const double a = v[j], c = v[j | (1 << M)];
      v[j] = a + c;
      v[j | (1 << M)] = a - c;
    }
}

// Register-index bits 0..N-1, in increasing order.
template <int N>
__device__ __forceinline__ void reg_stages(double (&v)[16]) {
  if constexpr (N > 0) reg_stage<0>(v);
  if constexpr (N > 1) reg_stage<1>(v);
  if constexpr (N > 2) reg_stage<2>(v);
  if constexpr (N > 3) reg_stage<3>(v);
}

// The largest double below m: "x > below(m)" is "x >= m".
__device__ __forceinline__ double below(double m) {
  const long long b = __double_as_longlong(m);
  if (m > 0.0) return __longlong_as_double(b - 1);
  if (m < 0.0) return __longlong_as_double(b + 1);
  return -4.9406564584124654e-324;   // m is +-0: the negative of the smallest subnormal
}

// fp64 -> fp16 bits, round to nearest even straight from fp64 (no detour
// through fp32), saturating at +-65504.
__device__ __forceinline__ uint16_t f64_to_f16(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x40EFFE0000000000ull) return (uint16_t)(sign | 0x7BFFu);  // >= 65520 (or NaN)
  const int e = (int)(a >> 52) - 1023;
  const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  int sh;
  uint32_t hi;
  if (e >= -14) {            // normal: 10 fraction bits
    sh = 42;
    hi = (uint32_t)(e + 14) << 10;
  } else {                   // subnormal: units of 2^-24
    sh = 28 - e;
    hi = 0;
    if (sh > 62) return (uint16_t)sign;   // below 2^-26: rounds to zero
  }
  uint64_t q = m >> sh;
  const uint64_t rem = m & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  q += (rem > half || (rem == half && (q & 1))) ? 1 : 0;
  return (uint16_t)(sign | (hi + (uint32_t)q));
}

__device__ __forceinline__ double h2d(uint16_t h) {
  const int e = (h >> 10) & 31, f = h & 1023;
  const double v = e ? ldexp((double)(1024 + f), e - 25) : ldexp((double)f, -24);
  return (h & 0x8000) ? -v : v;
}

__device__ __forceinline__ int tile_valid(const TileArgs &a, int64_t tile) {
  const int64_t left = a.total - tile * kTile;
  return left < kTile ? (int)left : kTile;
}

// One tile per workgroup.  LOG2B (the input-side block, 7..12) fixes the
// butterfly stages of each layout; the fp64-input modes take LOG2B = 0.
// Threads past the end of a partial tile read the first 16 elements (in
// bounds, never stored) instead of selecting zeros.
template <int MODE, int BITS, int LOG2B>
__global__ __launch_bounds__(kThreads) void tile_kernel(TileArgs a) {
  __shared__ double s[kLds];
  const int t = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t base = tile * kTile;
  const bool act = (t << 4) < tile_valid(a, tile);
  const int64_t off = act ? base + (t << 4) : 0;
  double v[16];
  if constexpr (MODE == kFused || MODE == kRotate) {
    const float4 *p = reinterpret_cast<const float4 *>(a.w + off);
    const uint4 sg = *reinterpret_cast<const uint4 *>(a.sign_in + (int)(off % a.d_in));
    const int8_t *sb = reinterpret_cast<const int8_t *>(&sg);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = p[q];
      v[4 * q + 0] = (double)f.x * (double)sb[4 * q + 0];
      v[4 * q + 1] = (double)f.y * (double)sb[4 * q + 1];
      v[4 * q + 2] = (double)f.z * (double)sb[4 * q + 2];
      v[4 * q + 3] = (double)f.w * (double)sb[4 * q + 3];
    }
    static_assert(LOG2B >= 7 && LOG2B <= 12, "block size");
    reg_stages<4>(v);                                  // strides 1..8
    lds_put<1>(s, v, t);
    __syncthreads();
    lds_get<2>(s, v, t);
    reg_stages<(LOG2B - 4 < 4 ? LOG2B - 4 : 4)>(v);    // strides 16..128
    __syncthreads();
    lds_put<2>(s, v, t);
    if constexpr (LOG2B > 8) {                         // strides 256..2048
      __syncthreads();
      lds_get<3>(s, v, t);
      reg_stages<LOG2B - 8>(v);
      __syncthreads();
      lds_put<3>(s, v, t);
    }
    __syncthreads();
    lds_get<1>(s, v, t);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= a.inv;
    if constexpr (MODE == kRotate) {
      if (act) {
        double2 *o = reinterpret_cast<double2 *>(a.out + base + (t << 4));
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = make_double2(v[2 * q], v[2 * q + 1]);
      }
      return;
    }
  } else {
    const double2 *p = reinterpret_cast<const double2 *>(a.wt + off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const double2 d = p[q];
      v[2 * q] = d.x;
      v[2 * q + 1] = d.y;
    }
  }

  if constexpr (MODE != kRotate) {
    // P1: lanes 8k..8k+7 of a wave hold one 128-group.
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    const uint16_t sh = f64_to_f16(sqrt(ss * (1.0 / 128.0)));
    const double sd = h2d(sh);

    if constexpr (MODE == kNorm) {
      if (act) {
        double2 *o = reinterpret_cast<double2 *>(a.out + base + (t << 4));
#pragma unroll
        for (int q = 0; q < 8; ++q)
          o[q] = sd > 0.0 ? make_double2(v[2 * q] / sd, v[2 * q + 1] / sd) : make_double2(0.0, 0.0);
      }
    } else {
      double pt[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) pt[c] = (double)a.lev[c] * sd;        // exact
      // Boundary k (between points k and k+1) is their midpoint, exact in
      // fp64; a weight on it goes up when tie_up says so, i.e. the test is
      // "> below(mid)".  A zero scale makes every point 0 and the code
      // zero_code: boundaries below it at -inf, the others at +inf.
      double th[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const double mid = (pt[k] + pt[k + 1]) * 0.5;
        const double tk = ((a.tie_up >> k) & 1) ? below(mid) : mid;
        th[k] = sd == 0.0 ? (k < a.zero_code ? -INFINITY : INFINITY) : tk;
      }
      // The three flags are monotone (b2 => b1 => b0), so the code is their
      // sum: bit 1 = b1, bit 0 = b0 ^ b1 ^ b2.  v becomes the residual.
      uint32_t p0 = 0, p1 = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool b0 = v[j] > th[0], b1 = v[j] > th[1], b2 = v[j] > th[2];
        p0 |= (uint32_t)(b0 ^ b1 ^ b2) << j;
        p1 |= (uint32_t)b1 << j;
        v[j] -= b1 ? (b2 ? pt[3] : pt[2]) : (b0 ? pt[1] : pt[0]);
      }
      const int64_t g = (base >> 7) + (t >> 3);
      const int q8 = t & 7;
      if (act) {
        uint16_t *bp = reinterpret_cast<uint16_t *>(a.base + g * 32);
        bp[q8] = (uint16_t)p0;
        bp[8 + q8] = (uint16_t)p1;
        if (q8 == 0) a.bscale[g] = sh;
      }
      if constexpr (BITS > 0) {
        constexpr int qm = (1 << (BITS - 1)) - 1;
        double am = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) am = fmax(am, fabs(v[j]));
        am = fmax(am, __shfl_xor(am, 1));
        am = fmax(am, __shfl_xor(am, 2));
        am = fmax(am, __shfl_xor(am, 4));
        const uint16_t rh = f64_to_f16(am / (double)qm);
        const double rd = h2d(rh);
        uint64_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const double x = fmin(fmax(rint(v[j] / rd), (double)-qm), (double)qm);
          const int qi = rd > 0.0 ? (int)x : 0;
          const uint64_t f = (uint64_t)(qi & ((1 << BITS) - 1));
          if (j < 8) lo |= f << (BITS * j);
          else hi |= f << (BITS * (j - 8));
        }
        // the thread's 2*BITS bytes: fields 0..7 fill bytes [0, BITS), 8..15 the next BITS
        const unsigned __int128 str = (unsigned __int128)lo | ((unsigned __int128)hi << (8 * BITS));
        if (act) {
          uint8_t *dst = a.resid + g * (16 * BITS) + 2 * BITS * q8;
          if constexpr (BITS % 2 == 0) {
            uint32_t *d32 = reinterpret_cast<uint32_t *>(dst);
#pragma unroll
            for (int k = 0; k < BITS / 2; ++k) d32[k] = (uint32_t)(str >> (32 * k));
          } else {
            uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
#pragma unroll
            for (int k = 0; k < BITS; ++k) d16[k] = (uint16_t)(str >> (16 * k));
          }
          if (q8 == 0) a.rscale[g] = rh;
        }
      }
    }
  }
}

// Output-side Hadamard over row-index bits [lo, lo + m) of 2^m rows x 32
// columns; the first pass multiplies by the output signs, the last by
// 1/sqrt(b_out) (inv != 0).
__global__ __launch_bounds__(kThreads) void col_pass_kernel(double *wt, int d_in, int lo, int m,
                                                            const int8_t *sign_out, double inv) {
  __shared__ double s[64][33];
  const int t = threadIdx.x;
  const int ctiles = d_in >> 5;
  const int u = blockIdx.x / ctiles;
  const int col = (blockIdx.x - u * ctiles) * 32 + (t & 31);
  const int64_t r0 = ((int64_t)(u >> lo) << (lo + m)) | (u & ((1 << lo) - 1));
  const int rows = 1 << m;
  for (int i = t >> 5; i < rows; i += 8) {
    const int64_t r = r0 + ((int64_t)i << lo);
    double x = wt[r * d_in + col];
    if (sign_out) x *= (double)sign_out[r];
    s[i][t & 31] = x;
  }
  __syncthreads();
  for (int h = 1; h < rows; h <<= 1) {
    for (int p = t; p < (rows >> 1) * 32; p += kThreads) {
      const int c = p & 31, pr = p >> 5;
      const int i = ((pr & ~(h - 1)) << 1) | (pr & (h - 1));
      const double x = s[i][c], y = s[i + h][c];
      s[i][c] = x + y;
      s[i + h][c] = x - y;
    }
    __syncthreads();
  }
  for (int i = t >> 5; i < rows; i += 8) {
    const int64_t r = r0 + ((int64_t)i << lo);
    double x = s[i][t & 31];
    if (inv != 0.0) x *= inv;
    wt[r * d_in + col] = x;
  }
}

// ---------------------------------------------------------------------------
// Level fitter.
// ---------------------------------------------------------------------------
constexpr int kFitWgs = 512;   // Lloyd partial sums
constexpr int kHistWgs = 1024;
constexpr int kBins = 2048;

struct FitState {
  uint32_t ticket;
  uint32_t pad0[15];
  double lev[4];          // current levels
  double out[4];          // symmetrised result
  uint64_t prefix[8];     // radix select: key bits fixed so far
  uint64_t rank[8];       // rank left inside that prefix
  int32_t rep[8];         // first target with the same prefix (shares its histogram)
  int32_t pad1[8];
  double frac[4];         // interpolation weights of the quantiles
  double pad2[4];
};
constexpr size_t kHistOff = 512;
constexpr size_t kPartOff = kHistOff + sizeof(uint32_t) * 8 * kBins;
constexpr size_t kFitWsBytes = kPartOff + sizeof(double) * 8 * kFitWgs;
static_assert(sizeof(FitState) <= kHistOff, "fit state");

__device__ __forceinline__ uint64_t okey(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double ikey(uint64_t k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

__global__ __launch_bounds__(kThreads) void select_init_kernel(char *ws, uint64_t r0, uint64_t r1, uint64_t r2,
                                                               uint64_t r3, uint64_t r4, uint64_t r5,
                                                               uint64_t r6, uint64_t r7, double f0, double f1,
                                                               double f2, double f3) {
  FitState *st = reinterpret_cast<FitState *>(ws);
  uint32_t *hist = reinterpret_cast<uint32_t *>(ws + kHistOff);
  const int t = threadIdx.x;
  for (int i = t; i < 8 * kBins; i += kThreads) hist[i] = 0;
  if (t < 8) {
    const uint64_t r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
    st->prefix[t] = 0;
    st->rank[t] = r[t];
    st->rep[t] = 0;
  }
  if (t < 4) {
    const double f[4] = {f0, f1, f2, f3};
    st->frac[t] = f[t];
  }
  if (t == 0) st->ticket = 0;
}

// Histogram of digit (key >> shift) & (2^width - 1) over the keys whose bits
// above the digit equal each distinct target's prefix.
__global__ __launch_bounds__(kThreads) void select_hist_kernel(const double *v, int64_t n, char *ws,
                                                               int shift, int width) {
  __shared__ uint32_t h[8][kBins];
  const FitState *st = reinterpret_cast<const FitState *>(ws);
  uint32_t *hist = reinterpret_cast<uint32_t *>(ws + kHistOff);
  const int t = threadIdx.x;
  for (int i = t; i < 8 * kBins; i += kThreads) (&h[0][0])[i] = 0;
  uint64_t pre[8];
  bool own[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    pre[k] = st->prefix[k];
    own[k] = st->rep[k] == k;
  }
  __syncthreads();
  const int top = shift + width;
  const uint32_t mask = (1u << width) - 1;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + t; i < n; i += (int64_t)gridDim.x * kThreads) {
    const uint64_t key = okey(v[i]);
    const uint32_t d = (uint32_t)(key >> shift) & mask;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (own[k] && (top == 64 || (key >> top) == (pre[k] >> top))) atomicAdd(&h[k][d], 1u);
  }
  __syncthreads();
  for (int i = t; i < 8 * kBins; i += kThreads) {
    const uint32_t c = (&h[0][0])[i];
    if (c) atomicAdd(&hist[i], c);
  }
}

// One wave per target: find the digit whose cumulative count passes the
// target's rank, fix it in the prefix; then clear the histograms and group
// equal prefixes.  After the last digit, the eight order statistics give the
// starting levels.
__global__ __launch_bounds__(512) void select_step_kernel(char *ws, int shift, int last) {
  __shared__ uint64_t npre[8], nrank[8];
  FitState *st = reinterpret_cast<FitState *>(ws);
  uint32_t *hist = reinterpret_cast<uint32_t *>(ws + kHistOff);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const uint32_t *hh = hist + st->rep[w] * kBins;
  const uint64_t rank = st->rank[w];
  uint64_t sum = 0;
  for (int k = 0; k < 32; ++k) sum += hh[lane * 32 + k];
  uint64_t inc = sum;
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  const uint64_t exc = inc - sum;
  if (exc <= rank && rank < inc) {
    uint64_t c = exc;
    for (int k = 0; k < 32; ++k) {
      const uint64_t b = hh[lane * 32 + k];
      if (c + b > rank) {
        npre[w] = st->prefix[w] | ((uint64_t)(lane * 32 + k) << shift);
        nrank[w] = rank - c;
        break;
      }
      c += b;
    }
  }
  __syncthreads();
  for (int i = t; i < 8 * kBins; i += 512) hist[i] = 0;
  if (t < 8) {
    st->prefix[t] = npre[t];
    st->rank[t] = nrank[t];
    int r = t;
    for (int k = 0; k < t; ++k)
      if (npre[k] == npre[t]) {
        r = k;
        break;
      }
    st->rep[t] = r;
  }
  if (last && t < 4) {
#pragma clang fp contract(off)
    const double a = ikey(npre[2 * t]), b = ikey(npre[2 * t + 1]);
    st->lev[t] = a + (b - a) * st->frac[t];
  }
}

__device__ __forceinline__ double ld_agent(const double *p) {
  return __longlong_as_double((long long)__hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// One Lloyd iteration: cell sums per workgroup, then the last workgroup to
// finish adds them in a fixed order and moves the levels.  Each thread reads
// its samples eight at a time (independent loads in flight).
constexpr int kLloydUnroll = 8;

__device__ __forceinline__ void lloyd_add(double x, const double (&mid)[3], const bool (&up)[3], double (&sm)[4],
                                          uint32_t (&ct)[4]) {
  int c = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) c += (x > mid[k] || (x == mid[k] && up[k])) ? 1 : 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (c == k) {
      sm[k] += x;
      ct[k] += 1;
    }
}

__global__ __launch_bounds__(kThreads) void lloyd_kernel(const double *v, int64_t n, char *ws) {
  __shared__ double red[32][8];
  __shared__ int last;
  FitState *st = reinterpret_cast<FitState *>(ws);
  double *part = reinterpret_cast<double *>(ws + kPartOff);
  const int t = threadIdx.x;
  double L[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) L[k] = st->lev[k];
  double mid[3];
  bool up[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    mid[k] = (L[k] + L[k + 1]) * 0.5;
    up[k] = fabs(L[k + 1]) <= fabs(L[k]);
  }
  double sm[4] = {0.0, 0.0, 0.0, 0.0};
  uint32_t ct[4] = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + t;
  for (; i + (kLloydUnroll - 1) * stride < n; i += kLloydUnroll * stride) {
    double x[kLloydUnroll];
#pragma unroll
    for (int u = 0; u < kLloydUnroll; ++u) x[u] = v[i + u * stride];
#pragma unroll
    for (int u = 0; u < kLloydUnroll; ++u) lloyd_add(x[u], mid, up, sm, ct);
  }
  for (; i < n; i += stride) lloyd_add(v[i], mid, up, sm, ct);
  double val[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    val[k] = sm[k];
    val[4 + k] = (double)ct[k];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    for (int o = 32; o >= 1; o >>= 1) val[k] += __shfl_xor(val[k], o);
  if ((t & 63) == 0)
#pragma unroll
    for (int k = 0; k < 8; ++k) red[t >> 6][k] = val[k];
  __syncthreads();
  // hand-over without fences (an agent-scope fence writes back the whole
  // L2): agent-scope stores, acknowledged before the ticket is taken
  if (t < 8) {
    const double p = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    __hip_atomic_store(part + blockIdx.x * 8 + t, p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t == 0)
    last = __hip_atomic_fetch_add(&st->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  // quantity k = t & 7 over workgroups j, j + 32, ... (j = t >> 3), then a
  // fixed tree over j
  const int k = t & 7, j = t >> 3;
  double acc = 0.0;
  for (unsigned b = j; b < gridDim.x; b += 32) acc += ld_agent(part + b * 8 + k);
  __syncthreads();
  red[j][k] = acc;
  __syncthreads();
  for (int w = 16; w >= 1; w >>= 1) {
    if (j < w) red[j][k] += red[j + w][k];
    __syncthreads();
  }
  if (t < 4 && red[0][4 + t] > 0.0) st->lev[t] = red[0][t] / red[0][4 + t];
  if (t == 0) __hip_atomic_store(&st->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fit_finish_kernel(char *ws) {
  FitState *st = reinterpret_cast<FitState *>(ws);
  if (threadIdx.x == 0) {
    const double a0 = (st->lev[2] - st->lev[1]) * 0.5;
    const double a1 = (st->lev[3] - st->lev[0]) * 0.5;
    st->out[0] = -a1;
    st->out[1] = -a0;
    st->out[2] = a0;
    st->out[3] = a1;
  }
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

int log2_block(int n) {  // block-size rule: largest power of two dividing n, at most 4096
  int l = 0;
  while (l < 12 && n % (2 << l) == 0) ++l;
  return l;
}

nl_status check_shape(const char *who, int d_out, int d_in) {
  if (d_out < 1 || d_in < 128 || d_in % 128)
    return fail(NL_EINVAL, "%s: need d_out >= 1 and d_in a positive multiple of 128 (got %d x %d)", who,
                d_out, d_in);
  const int64_t tiles = ((int64_t)d_out * d_in + kTile - 1) / kTile;
  if (tiles > 0x7FFFFFFF) return fail(NL_EINVAL, "%s: matrix too large", who);
  return NL_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return x < y + nb && y < x + na;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

void fill_rot(TileArgs &a, int d_out, int d_in, const int8_t *sign_in) {
  a.total = (int64_t)d_out * d_in;
  a.d_in = d_in;
  a.sign_in = sign_in;
  a.log2b = log2_block(d_in);
  a.inv = 1.0 / std::sqrt((double)(1 << a.log2b));
}

nl_status check_codes(const char *who, const nl_codes *o, TileArgs &a) {
  if (!o) return fail(NL_EINVAL, "%s: codes descriptor is NULL", who);
  if (nl_status st = check_shape(who, o->d_out, o->d_in)) return st;
  const int b = o->residual_bits;
  if (b != 0 && b != 6 && b != 7 && b != 8)
    return fail(NL_EINVAL, "%s: residual_bits must be 0, 6, 7 or 8 (got %d)", who, b);
  if (!o->base_codes || !o->base_scales) return fail(NL_EINVAL, "%s: base arrays must not be NULL", who);
  if (b && (!o->resid_codes || !o->resid_scales))
    return fail(NL_EINVAL, "%s: residual arrays must not be NULL when residual_bits > 0", who);
  if (!b && (o->resid_codes || o->resid_scales))
    return fail(NL_EINVAL, "%s: residual arrays must be NULL when residual_bits == 0", who);
  for (int c = 0; c < 4; ++c)
    if (!std::isfinite(o->levels[c])) return fail(NL_EINVAL, "%s: level %d is not finite", who, c);
  for (int c = 0; c < 3; ++c)
    if (!(o->levels[c] < o->levels[c + 1]))
      return fail(NL_EINVAL, "%s: levels must be strictly ascending", who);
  if (((uintptr_t)o->base_codes | (uintptr_t)o->base_scales | (uintptr_t)o->resid_codes |
       (uintptr_t)o->resid_scales) & 3)
    return fail(NL_EINVAL, "%s: output arrays must be 4-byte aligned", who);
  a.base = o->base_codes;
  a.bscale = o->base_scales;
  a.resid = o->resid_codes;
  a.rscale = o->resid_scales;
  a.tie_up = 0;
  for (int k = 0; k < 3; ++k)
    if (std::fabs(o->levels[k + 1]) <= std::fabs(o->levels[k])) a.tie_up |= 1 << k;
  int zc = 0;
  for (int c = 1; c < 4; ++c)   // smallest |level|, the larger level on equal magnitudes
    if (std::fabs(o->levels[c]) <= std::fabs(o->levels[zc])) zc = c;
  a.zero_code = zc;
  for (int c = 0; c < 4; ++c) a.lev[c] = o->levels[c];
  return NL_OK;
}

template <int MODE, int LOG2B>
hipError_t launch_tiles_b(const TileArgs &a, int bits, hipStream_t s) {
  const dim3 grid((unsigned)((a.total + kTile - 1) / kTile)), block(kThreads);
  if constexpr (MODE == kRotate || MODE == kNorm) {
    hipLaunchKernelGGL((tile_kernel<MODE, 0, LOG2B>), grid, block, 0, s, a);
  } else {
    switch (bits) {
      case 0: hipLaunchKernelGGL((tile_kernel<MODE, 0, LOG2B>), grid, block, 0, s, a); break;
      case 6: hipLaunchKernelGGL((tile_kernel<MODE, 6, LOG2B>), grid, block, 0, s, a); break;
      case 7: hipLaunchKernelGGL((tile_kernel<MODE, 7, LOG2B>), grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL((tile_kernel<MODE, 8, LOG2B>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_tiles(const TileArgs &a, int bits, hipStream_t s) {
  if constexpr (MODE == kQuant || MODE == kNorm) {
    return launch_tiles_b<MODE, 0>(a, bits, s);
  } else {
    switch (a.log2b) {
      case 7: return launch_tiles_b<MODE, 7>(a, bits, s);
      case 8: return launch_tiles_b<MODE, 8>(a, bits, s);
      case 9: return launch_tiles_b<MODE, 9>(a, bits, s);
      case 10: return launch_tiles_b<MODE, 10>(a, bits, s);
      case 11: return launch_tiles_b<MODE, 11>(a, bits, s);
      case 12: return launch_tiles_b<MODE, 12>(a, bits, s);
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_cols(double *wt, int d_out, int d_in, const int8_t *sign_out, hipStream_t s) {
  const int K = log2_block(d_out);
  const double inv = 1.0 / std::sqrt((double)(1 << K));
  const int m1 = K < 6 ? K : 6;
  const int ctiles = d_in / 32;
  hipLaunchKernelGGL(col_pass_kernel, dim3((unsigned)((d_out >> m1) * ctiles)), dim3(kThreads), 0, s, wt,
                     d_in, 0, m1, sign_out, K > 6 ? 0.0 : inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || K <= 6) return e;
  hipLaunchKernelGGL(col_pass_kernel, dim3((unsigned)((d_out >> (K - 6)) * ctiles)), dim3(kThreads), 0, s,
                     wt, d_in, 6, K - 6, (const int8_t *)nullptr, inv);
  return hipGetLastError();
}

}  // namespace

extern "C" nl_status nested_encode_rotate(int32_t d_out, int32_t d_in, const float *w, const int8_t *sign_in,
                                          const int8_t *sign_out, double *wt, void *stream) {
  static const char *who = "nested_encode_rotate";
  if (nl_status st = check_shape(who, d_out, d_in)) return st;
  if (!w || !sign_in || !wt) return fail(NL_EINVAL, "%s: w, sign_in and wt must not be NULL", who);
  const size_t n = (size_t)d_out * d_in;
  if (((uintptr_t)w & 15) || ((uintptr_t)wt & 15) || ((uintptr_t)sign_in & 15))
    return fail(NL_EINVAL, "%s: w, wt and sign_in must be 16-byte aligned", who);
  if (overlap(w, 4 * n, wt, 8 * n)) return fail(NL_EINVAL, "%s: w and wt overlap", who);
  TileArgs a{};
  fill_rot(a, d_out, d_in, sign_in);
  a.w = w;
  a.out = wt;
  HIP_OR_FAIL((launch_tiles<kRotate>(a, 0, as_stream(stream))));
  if (sign_out) HIP_OR_FAIL(launch_cols(wt, d_out, d_in, sign_out, as_stream(stream)));
  return ok();
}

extern "C" nl_status nested_encode_quantize(const double *wt, const nl_codes *out, void *stream) {
  static const char *who = "nested_encode_quantize";
  TileArgs a{};
  if (nl_status st = check_codes(who, out, a)) return st;
  if (!wt || ((uintptr_t)wt & 15)) return fail(NL_EINVAL, "%s: wt must be a 16-byte aligned pointer", who);
  a.total = (int64_t)out->d_out * out->d_in;
  a.d_in = out->d_in;
  a.wt = wt;
  HIP_OR_FAIL((launch_tiles<kQuant>(a, out->residual_bits, as_stream(stream))));
  return ok();
}

extern "C" nl_status nested_encode_workspace_bytes(int32_t d_out, int32_t d_in, int32_t two_sided,
                                                   size_t *bytes) {
  if (nl_status st = check_shape("nested_encode_workspace_bytes", d_out, d_in)) return st;
  if (!bytes) return fail(NL_EINVAL, "nested_encode_workspace_bytes: bytes is NULL");
  *bytes = two_sided ? (size_t)8 * d_out * d_in : 0;
  return ok();
}

extern "C" nl_status nested_encode(const float *w, const int8_t *sign_in, const int8_t *sign_out,
                                   const nl_codes *out, void *ws, size_t ws_bytes, void *stream) {
  static const char *who = "nested_encode";
  TileArgs a{};
  if (nl_status st = check_codes(who, out, a)) return st;
  if (!w || !sign_in) return fail(NL_EINVAL, "%s: w and sign_in must not be NULL", who);
  if (((uintptr_t)w & 15) || ((uintptr_t)sign_in & 15))
    return fail(NL_EINVAL, "%s: w and sign_in must be 16-byte aligned", who);
  const int d_out = out->d_out, d_in = out->d_in;
  if (!sign_out) {
    fill_rot(a, d_out, d_in, sign_in);
    a.w = w;
    HIP_OR_FAIL((launch_tiles<kFused>(a, out->residual_bits, as_stream(stream))));
    return ok();
  }
  const size_t need = (size_t)8 * d_out * d_in;
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
    return fail(NL_EINVAL, "%s: two-sided form needs a 256-byte aligned workspace of %zu bytes", who, need);
  double *wt = static_cast<double *>(ws);
  if (nl_status st = nested_encode_rotate(d_out, d_in, w, sign_in, sign_out, wt, stream)) return st;
  return nested_encode_quantize(wt, out, stream);
}

extern "C" nl_status nested_encode_normalize(int32_t d_out, int32_t d_in, const double *wt, double *v,
                                             void *stream) {
  static const char *who = "nested_encode_normalize";
  if (nl_status st = check_shape(who, d_out, d_in)) return st;
  if (!wt || !v || ((uintptr_t)wt & 15) || ((uintptr_t)v & 15))
    return fail(NL_EINVAL, "%s: wt and v must be 16-byte aligned pointers", who);
  const size_t n = (size_t)d_out * d_in;
  if (overlap(wt, 8 * n, v, 8 * n)) return fail(NL_EINVAL, "%s: wt and v overlap", who);
  TileArgs a{};
  a.total = (int64_t)n;
  a.d_in = d_in;
  a.wt = wt;
  a.out = v;
  HIP_OR_FAIL((launch_tiles<kNorm>(a, 0, as_stream(stream))));
  return ok();
}

extern "C" nl_status nested_encode_fit_workspace_bytes(int64_t n, size_t *bytes) {
  if (n < 1 || n > ((int64_t)1 << 31))
    return fail(NL_EINVAL, "nested_encode_fit_workspace_bytes: n must be in 1..2^31");
  if (!bytes) return fail(NL_EINVAL, "nested_encode_fit_workspace_bytes: bytes is NULL");
  *bytes = kFitWsBytes;
  return ok();
}

extern "C" nl_status nested_encode_fit_levels(const double *v, int64_t n, int32_t iters, double *levels,
                                              void *ws, size_t ws_bytes, void *stream) {
  static const char *who = "nested_encode_fit_levels";
  if (n < 1 || n > ((int64_t)1 << 31)) return fail(NL_EINVAL, "%s: n must be in 1..2^31", who);
  if (iters < 0 || iters > 100000) return fail(NL_EINVAL, "%s: iters must be in 0..100000", who);
  if (!v || !levels) return fail(NL_EINVAL, "%s: v and levels must not be NULL", who);
  if (!ws || ws_bytes < kFitWsBytes || ((uintptr_t)ws & 255))
    return fail(NL_EINVAL, "%s: needs a 256-byte aligned workspace of %zu bytes", who, kFitWsBytes);
  if (overlap(v, 8 * (size_t)n, ws, kFitWsBytes)) return fail(NL_EINVAL, "%s: v and ws overlap", who);
  hipStream_t s = as_stream(stream);
  char *w = static_cast<char *>(ws);
  // ranks and interpolation weights of the four quantiles, at q (n - 1)
  static const double kQ[4] = {0.125, 0.375, 0.625, 0.875};
  uint64_t r[8];
  double f[4];
  for (int i = 0; i < 4; ++i) {
    const double pos = kQ[i] * (double)(n - 1);
    const double lo = std::floor(pos);
    r[2 * i] = (uint64_t)lo;
    r[2 * i + 1] = (uint64_t)lo + 1 < (uint64_t)n ? (uint64_t)lo + 1 : (uint64_t)(n - 1);
    f[i] = pos - lo;
  }
  hipLaunchKernelGGL(select_init_kernel, dim3(1), dim3(kThreads), 0, s, w, r[0], r[1], r[2], r[3], r[4], r[5],
                     r[6], r[7], f[0], f[1], f[2], f[3]);
  HIP_OR_FAIL(hipGetLastError());
  static const int kShift[6] = {53, 42, 31, 20, 9, 0};
  static const int kWidth[6] = {11, 11, 11, 11, 11, 9};
  const int64_t hw = (n + 4 * kThreads - 1) / (4 * kThreads);
  const unsigned hist_wgs = (unsigned)(hw < kHistWgs ? hw : kHistWgs);
  for (int p = 0; p < 6; ++p) {
    hipLaunchKernelGGL(select_hist_kernel, dim3(hist_wgs), dim3(kThreads), 0, s, v, n, w, kShift[p],
                       kWidth[p]);
    HIP_OR_FAIL(hipGetLastError());
    hipLaunchKernelGGL(select_step_kernel, dim3(1), dim3(512), 0, s, w, kShift[p], p == 5 ? 1 : 0);
    HIP_OR_FAIL(hipGetLastError());
  }
  const int64_t lw = (n + 4 * kThreads - 1) / (4 * kThreads);
  const unsigned lloyd_wgs = (unsigned)(lw < kFitWgs ? lw : kFitWgs);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(lloyd_kernel, dim3(lloyd_wgs), dim3(kThreads), 0, s, v, n, w);
    HIP_OR_FAIL(hipGetLastError());
  }
  hipLaunchKernelGGL(fit_finish_kernel, dim3(1), dim3(64), 0, s, w);
  HIP_OR_FAIL(hipGetLastError());
  HIP_OR_FAIL(hipMemcpyAsync(levels, w + offsetof(FitState, out), 4 * sizeof(double), hipMemcpyDeviceToHost, s));
  HIP_OR_FAIL(hipStreamSynchronize(s));
  return ok();
}
