// nl_tree.hip -- best-first draft tree and greedy acceptance
// (include/nested_tree.h).
//
// Build: one wave.  Candidate slot s < R is the root's child of rank s; slot
// R + k R + r is node k's child of rank r, so slot order is push order and
// "largest priority, then smallest slot" is the heap-with-counter order.
// The probability rows the build can reach sit in LDS.  When every such row
// is non-increasing in rank (the usual rank statistics), lane l keeps only
// the next child of node l - 1 (lane 0: the root's), since a node's children
// are popped in rank order; otherwise lane l keeps the priorities of slots
// l, l + 64, ... in registers.  Each step is a wave-wide argmax (largest
// priority, then smallest slot); the winner becomes node k, its slot dies,
// and the lanes that own its sibling's and children's slots compute them.
//
// Accept: one wave per sequence; lane c holds node c's parent and token, and
// each step is one ballot for the child of the current node whose token is
// the verifier's argmax.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "../../include/nested_tree.h"

namespace nl {
nl_status api_error(nl_status st, const char *msg);  // nl_api.hip
}

namespace {

constexpr int kMaxSlots = NL_TREE_MAX_RANKS * (1 + NL_TREE_MAX_NODES);

// One reduction step of (priority, slot) under "larger priority, then
// smaller slot" (associative and commutative, so any exchange pattern that
// reaches every lane gives every lane the same winner).
__device__ __forceinline__ void arg_merge(double &bp, int &bs, double op, int os) {
  if (op > bp || (op == bp && os < bs)) {
    bp = op;
    bs = os;
  }
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ void arg_dpp(double &bp, int &bs) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(bp);
  const unsigned lo = (unsigned)dppi<CTRL>((int)(unsigned)b), hi = (unsigned)dppi<CTRL>((int)(unsigned)(b >> 32));
  arg_merge(bp, bs, __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo)), dppi<CTRL>(bs));
}

// The wave's best (priority, slot): DPP steps within rows of 16 lanes (pairs,
// quads, half-row and row mirrors), then the four row results read as
// uniform values and merged.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(double &bp, int &bs) {
  arg_dpp<0xB1>(bp, bs);
  arg_dpp<0x4E>(bp, bs);
  arg_dpp<0x141>(bp, bs);
  arg_dpp<0x140>(bp, bs);
  const unsigned long long b = (unsigned long long)__double_as_longlong(bp);
  const int lo = (int)(unsigned)b, hi = (int)(unsigned)(b >> 32);
  double best = -2.0;
  int slot = 0x7FFFFFFF;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const unsigned rl = (unsigned)__builtin_amdgcn_readlane(lo, 16 * row);
    const unsigned rh = (unsigned)__builtin_amdgcn_readlane(hi, 16 * row);
    arg_merge(best, slot, __longlong_as_double((long long)(((unsigned long long)rh << 32) | rl)),
              __builtin_amdgcn_readlane(bs, 16 * row));
  }
  bp = best;
  bs = slot;
}

// The wave's largest value (DPP steps within rows of 16 lanes, then the four
// row results read as uniform values).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)dppi<CTRL>((int)(unsigned)b), hi = (unsigned)dppi<CTRL>((int)(unsigned)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double read_lane(double v, int src) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, src);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), src);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, dpp_d<0xB1>(v));
  v = fmax(v, dpp_d<0x4E>(v));
  v = fmax(v, dpp_d<0x141>(v));
  v = fmax(v, dpp_d<0x140>(v));
  return fmax(fmax(read_lane(v, 0), read_lane(v, 16)), fmax(read_lane(v, 32), read_lane(v, 48)));
}

__global__ __launch_bounds__(64) void tree_build_kernel(const double *p, int D, int R, int N, int32_t *parent,
                                                        int32_t *depth, int32_t *rank, double *prio,
                                                        uint64_t *anc, int32_t *count) {
  constexpr int kJ = (kMaxSlots + 63) / 64;   // slots per lane: slot lane + 64 j
  __shared__ double pl[(NL_TREE_MAX_NODES + 1) * NL_TREE_MAX_RANKS];
  __shared__ int ndep[NL_TREE_MAX_NODES], npar[NL_TREE_MAX_NODES], nrank[NL_TREE_MAX_NODES];
  __shared__ uint64_t nanc[NL_TREE_MAX_NODES];
  __shared__ double nprio[NL_TREE_MAX_NODES];
  const int lane = threadIdx.x;
  // a node's depth is at most N, so rows 0 .. min(D, N + 1) - 1 of p are all
  // the build reads
  const int rows = min(D, N + 1);
  for (int i = lane; i < rows * R; i += 64) pl[i] = p[i];
  double cp[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int s = lane + 64 * j;
    cp[j] = s < R ? p[s] : -1.0;   // depth-1 paths; -1 marks a dead or unwritten slot
  }
  __syncthreads();
  // Every row the build reads non-increasing in rank: a node's children are
  // then popped in rank order (an earlier sibling has the larger or equal
  // priority and the smaller slot), so the best live slot is always some
  // node's next child.  Lane l keeps only that candidate for node l - 1
  // (lane 0: the root), and a step is one argmax over 64 values.  The
  // products and the tie order are those of the full candidate set.
  bool ok = true;
  for (int i = lane; i < rows * R; i += 64)
    if (i % R + 1 < R && pl[i + 1] > pl[i]) ok = false;
  int k = 0;
  if (__ballot(!ok) == 0) {
    double P = 1.0;                       // the node's priority (root: 1)
    int dep = 0, nr = 0;                  // the node's depth, its next child's rank
    uint64_t an = 0;                      // the node's ancestor mask
    double cand = lane == 0 ? pl[0] : -1.0;
    // requested ahead, so no step waits on LDS: the probability of the
    // candidate's next sibling, and lane d's rank-0 probability at depth d
    double pn = lane == 0 && R > 1 ? pl[1] : 0.0;
    const double p0 = lane < rows ? pl[lane * R] : 0.0;
    for (; k < N; ++k) {
      // lane l's candidate slot lies in [R l, R l + R): slot order is lane
      // order, so the smallest slot of the best priority is the lowest lane
      // holding it
      const double bp = wave_max(cand);
      if (bp < 0.0) break;   // no live candidate (uniform)
      const int w = __builtin_ctzll(__ballot(cand == bp));   // the winner's lane: its parent + 1
      const int rk = __builtin_amdgcn_readlane(nr, w);
      const int wdep = __builtin_amdgcn_readlane(dep, w);
      const uint64_t wan = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)an, w) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(an >> 32), w) << 32);
      const int ndp = wdep + 1;
      const uint64_t am = wan | (1ull << k);
      if (lane == w) {   // the parent's next child
        nr = rk + 1;
        cand = nr < R ? P * pn : -1.0;
        pn = nr + 1 < R ? pl[dep * R + nr + 1] : 0.0;
      }
      // rank-0 probability at the new node's depth (its first child's factor)
      const double f0 = read_lane(p0, min(ndp, 63));
      if (lane == k + 1) {   // node k and its first child
        P = bp;
        dep = ndp;
        an = am;
        nr = 0;
        cand = ndp < D ? bp * f0 : -1.0;
        pn = ndp < D && R > 1 ? pl[ndp * R + 1] : 0.0;
      }
      if (lane == 0) {
        ndep[k] = ndp;
        nanc[k] = am;
        npar[k] = w - 1;
        nrank[k] = rk;
        nprio[k] = bp;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  } else {
  for (; k < N; ++k) {
    double bp = -1.0;
    int bs = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (cp[j] > bp) {   // ascending slots: an equal later slot never wins
        bp = cp[j];
        bs = lane + 64 * j;
      }
    wave_argmax(bp, bs);
    if (bp < 0.0) break;   // no live candidate (uniform)
    const int par = bs < R ? -1 : (bs - R) / R;
    const int rk = bs < R ? bs : (bs - R) % R;
    const int dep = par < 0 ? 1 : ndep[par] + 1;
    const uint64_t am = (par < 0 ? 0ull : nanc[par]) | (1ull << k);
    // the winner's slot dies; node k's children take slots R + k R .. + R - 1,
    // at most one per lane since R <= 16 (the winner's slot lies below them)
    const int first = R + k * R;
    const int off = (lane - first) & 63;
    const bool add = dep < D && off < R;
    const int jn = (first + off) >> 6, jw = bs >> 6;
    const bool own = (bs & 63) == lane;
    const double val = add ? bp * pl[dep * R + off] : -1.0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (own && j == jw) cp[j] = -1.0;
      if (add && j == jn) cp[j] = val;
    }
    if (lane == 0) {
      ndep[k] = dep;
      nanc[k] = am;
      npar[k] = par;
      nrank[k] = rk;
      nprio[k] = bp;
    }
    // one wave: its LDS accesses complete in program order, so the next
    // step's reads see these writes; the clobber keeps the compiler's order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  }
  if (lane < k) {   // the nodes go out together, one per lane (N <= 64)
    parent[lane] = npar[lane];
    depth[lane] = ndep[lane];
    rank[lane] = nrank[lane];
    prio[lane] = nprio[lane];
    anc[lane] = nanc[lane];
  }
  if (lane == 0) *count = k;
}

__global__ __launch_bounds__(64) void tree_accept_kernel(const int32_t *parent, int N, const int32_t *draft,
                                                         const int32_t *argmax, int32_t *n_acc, int32_t *path,
                                                         int32_t *bonus) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int par = lane < N ? parent[lane] : -2;
  const int tok = lane < N ? draft[(size_t)b * N + lane] : 0;
  const int32_t *am = argmax + (size_t)b * (N + 1);
  int u = -1, len = 0;
  for (int step = 0; step < N; ++step) {
    const int target = am[u + 1];
    const unsigned long long m = __ballot(par == u && tok == target);
    if (!m) break;
    const int c = __ffsll((long long)m) - 1;
    if (lane == 0) path[(size_t)b * N + len] = c;
    ++len;
    u = c;
  }
  if (lane == 0) {
    n_acc[b] = len;
    bonus[b] = am[u + 1];
  }
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

}  // namespace

extern "C" nl_status nested_tree_build(const double *p, int32_t D, int32_t R, int32_t N, int32_t *parent,
                                       int32_t *depth, int32_t *rank, double *prio, uint64_t *anc, int32_t *count,
                                       void *stream) {
  if (D < 1) return fail("nested_tree_build: D must be >= 1 (got %d)", D);
  if (R < 1 || R > NL_TREE_MAX_RANKS) return fail("nested_tree_build: R must be in 1..%d (got %d)", NL_TREE_MAX_RANKS, R);
  if (N < 1 || N > NL_TREE_MAX_NODES) return fail("nested_tree_build: N must be in 1..%d (got %d)", NL_TREE_MAX_NODES, N);
  if (!p || !parent || !depth || !rank || !prio || !anc || !count)
    return fail("nested_tree_build: NULL pointer");
  hipLaunchKernelGGL(tree_build_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), p, D, R, N, parent,
                     depth, rank, prio, anc, count);
  return launched("nested_tree_build");
}

extern "C" nl_status nested_tree_accept(const int32_t *parent, int32_t N, int32_t B, const int32_t *draft,
                                        const int32_t *argmax, int32_t *n_acc, int32_t *path, int32_t *bonus,
                                        void *stream) {
  if (N < 1 || N > NL_TREE_MAX_NODES) return fail("nested_tree_accept: N must be in 1..%d (got %d)", NL_TREE_MAX_NODES, N);
  if (B < 1) return fail("nested_tree_accept: B must be >= 1 (got %d)", B);
  if (!parent || !draft || !argmax || !n_acc || !path || !bonus) return fail("nested_tree_accept: NULL pointer");
  hipLaunchKernelGGL(tree_accept_kernel, dim3((unsigned)B), dim3(64), 0, static_cast<hipStream_t>(stream), parent, N,
                     draft, argmax, n_acc, path, bonus);
  return launched("nested_tree_accept");
}
