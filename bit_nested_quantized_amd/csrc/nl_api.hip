// nl_api.hip -- the C ABI (include/nested_linear.h): validation, create-time
// repack, workspace layout, launch configuration.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/nested_linear.h"
#include "nl_fwd.h"
#include "nl_kernels.h"

using namespace nl;

static thread_local std::string g_err;

static nl_status fail(nl_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
static nl_status fail(nl_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

static nl_status ok() {
  g_err.clear();
  return NL_OK;
}

// The encoder's translation unit reports its errors through the same
// per-thread message (NL_OK clears it).
namespace nl {
__attribute__((visibility("hidden"))) nl_status api_error(nl_status st, const char *msg) {
  if (st == NL_OK) g_err.clear();
  else g_err = msg;
  return st;
}
}  // namespace nl

#define HIP_OR_FAIL(expr)                                                              \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(NL_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

static constexpr uint32_t kMagic = 0x4E4C4C31u;   // "NLL1"
static constexpr uint32_t kGroupMagic = 0x4E4C4731u;

struct nl_linear {
  uint32_t magic;
  int d_out, d_in, bits, G, n_tiles, n_chunks, b_in, b_out;
  bool has_sign_out;
  float level_err;
  void *mem;
  size_t mem_bytes;
  LinearDev dev;
};

struct nl_group {
  uint32_t magic;
  int n, d_out, d_in, bits, n_tiles, n_chunks, b_in, b_out;
  bool has_sign_out;
  LinearDev *dev_array;  // device copy of the experts' descriptors
};

static int block_size(int n) {  // POC section 1 "Block size" rule
  int b = 1;
  while (n % (2 * b) == 0 && 2 * b <= 4096) b *= 2;
  return b;
}

static int log2i(int b) {
  int l = 0;
  while ((1 << l) < b) ++l;
  return l;
}

// Rows per finish workgroup: one superblock of 256*E outputs, E in {2..16}.
static int finish_rows(bool sign_out, int b_out) {
  if (!sign_out) return 4096;
  return b_out > kChunk ? b_out : kChunk;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Round a float to the nearest fp16 (ties to even) and return its bits.
static uint16_t f2h_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  memcpy(&b, &h, 2);
  return b;
}

static float h_bits2f(uint16_t b) {
  _Float16 h;
  memcpy(&h, &b, 2);
  return (float)h;
}

// Largest relative error of a base level as the kernels hold it (create
// refuses levels beyond it).
constexpr float kMaxLevelRelErr = 2e-3f;

// Pick kappa so that fp16(kappa * levels[c]) is as close as possible to
// kappa * levels[c] for all four levels (relative error), then build the
// fp16x2 pair table used by the kernels' base unpack.
static void build_lut(const float levels[4], uint32_t lut[16], float *kinv, float *err_out) {
  float lmax = 0.f;
  for (int c = 0; c < 4; ++c) lmax = fmaxf(lmax, fabsf(levels[c]));
  double best_err = 1e30;
  double best_kappa = 1.0;
  if (lmax > 0.f) {
    // kappa * lmax spans one binade of fp16 in steps of 1/8 ulp.
    for (int n = 1024 * 8; n < 2048 * 8; ++n) {
      const double kappa = (n / 8.0) / (double)lmax;
      double e = 0.0;
      for (int c = 0; c < 4; ++c) {
        if (levels[c] == 0.f) continue;
        const double want = kappa * (double)levels[c];
        const double got = (double)h_bits2f(f2h_bits((float)want));
        e = fmax(e, fabs(got - want) / fabs(want));
      }
      if (e < best_err) {
        best_err = e;
        best_kappa = kappa;
      }
    }
  } else {
    best_err = 0.0;
  }
  uint16_t hb[4];
  for (int c = 0; c < 4; ++c) hb[c] = f2h_bits((float)(best_kappa * (double)levels[c]));
  for (int i = 0; i < 16; ++i) lut[i] = (uint32_t)hb[i & 3] | ((uint32_t)hb[i >> 2] << 16);
  *kinv = (float)(1.0 / best_kappa);
  *err_out = (float)best_err;
}

// Live handles, so that NULL, destroyed or foreign pointers are rejected
// without being dereferenced.
static std::mutex g_live_mu;
static std::unordered_set<const void *> g_live;

static void live_add(const void *p) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  g_live.insert(p);
}
static void live_del(const void *p) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  g_live.erase(p);
}
static bool live(const void *p) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.count(p) != 0;
}
static bool valid(const nl_linear *h) { return h && live(h) && h->magic == kMagic; }
static bool valid(nl_group_handle g) { return g && live(g) && g->magic == kGroupMagic; }

extern "C" const char *nested_linear_last_error(void) { return g_err.c_str(); }

extern "C" nl_status nested_linear_create(const nl_desc *d, nl_handle *out) {
  if (!d || !out) return fail(NL_EINVAL, "create: NULL desc or out");
  if (d->d_out < 1) return fail(NL_EINVAL, "create: d_out must be >= 1 (got %d)", d->d_out);
  if (d->d_in < NL_GROUP || d->d_in % NL_GROUP)
    return fail(NL_EINVAL, "create: d_in must be a positive multiple of 128 (got %d)", d->d_in);
  const int bits = d->residual_bits;
  if (bits != 0 && bits != 6 && bits != 7 && bits != 8)
    return fail(NL_EINVAL, "create: residual_bits must be 0, 6, 7 or 8 (got %d)", bits);
  if (!d->base_codes || !d->base_scales || !d->sign_in)
    return fail(NL_EINVAL, "create: base_codes, base_scales and sign_in are required");
  if (bits && (!d->resid_codes || !d->resid_scales))
    return fail(NL_EINVAL, "create: residual arrays are required when residual_bits > 0");
  if (!bits && (d->resid_codes || d->resid_scales))
    return fail(NL_EINVAL, "create: residual arrays given with residual_bits == 0");
  for (int c = 0; c < 4; ++c)
    if (!std::isfinite(d->levels[c])) return fail(NL_EINVAL, "create: level %d is not finite", c);
  {  // the kernels hold the levels as fp16 after one exact rescale: refuse
     // levels that fp16 cannot hold within the output tolerance
    uint32_t lut[16];
    float kinv, err;
    build_lut(d->levels, lut, &kinv, &err);
    if (!(err <= kMaxLevelRelErr))
      return fail(NL_EUNSUPPORTED,
                  "create: levels (%g, %g, %g, %g) span too wide a ratio for fp16 (relative error %.3g > %g)",
                  d->levels[0], d->levels[1], d->levels[2], d->levels[3], err, kMaxLevelRelErr);
  }

  // Signs: copied to the host once and checked to be +-1.
  std::vector<int8_t> si(d->d_in), so(d->sign_out ? d->d_out : 0);
  HIP_OR_FAIL(hipMemcpy(si.data(), d->sign_in, si.size(), hipMemcpyDeviceToHost));
  if (d->sign_out) HIP_OR_FAIL(hipMemcpy(so.data(), d->sign_out, so.size(), hipMemcpyDeviceToHost));
  for (size_t i = 0; i < si.size(); ++i)
    if (si[i] != 1 && si[i] != -1) return fail(NL_EINVAL, "create: sign_in[%zu] = %d is not +-1", i, si[i]);
  for (size_t i = 0; i < so.size(); ++i)
    if (so[i] != 1 && so[i] != -1) return fail(NL_EINVAL, "create: sign_out[%zu] = %d is not +-1", i, so[i]);

  nl_linear *h = new (std::nothrow) nl_linear();
  if (!h) return fail(NL_ENOMEM, "create: host allocation failed");
  h->d_out = d->d_out;
  h->d_in = d->d_in;
  h->bits = bits;
  h->G = d->d_in / NL_GROUP;
  h->n_tiles = (d->d_out + kTileRows - 1) / kTileRows;
  h->n_chunks = (d->d_in + kChunk - 1) / kChunk;
  h->b_in = block_size(d->d_in);
  h->b_out = block_size(d->d_out);
  h->has_sign_out = d->sign_out != nullptr;

  const size_t tcs = (size_t)h->n_tiles * h->n_chunks;
  const size_t o_base = 0;
  const size_t o_resid = align256(o_base + tcs * kBaseBlockBytes);
  const size_t o_bsc = align256(o_resid + (bits ? tcs * resid_block_bytes(bits) : 0));
  const size_t o_rsc = align256(o_bsc + tcs * kScaleBlockBytes);
  const size_t o_si = align256(o_rsc + (bits ? tcs * kScaleBlockBytes : 0));
  const size_t o_so = align256(o_si + d->d_in);
  const size_t o_lut = align256(o_so + (d->sign_out ? d->d_out : 0));
  const size_t total = align256(o_lut + 256 * sizeof(uint2));
  hipError_t e = hipMalloc(&h->mem, total);
  if (e != hipSuccess) {
    delete h;
    (void)hipGetLastError();
    return fail(NL_ENOMEM, "create: hipMalloc(%zu) failed: %s", total, hipGetErrorString(e));
  }
  h->mem_bytes = total;
  char *m = (char *)h->mem;
  LinearDev &L = h->dev;
  memset(&L, 0, sizeof L);
  L.base = (const uint4 *)(m + o_base);
  L.resid = bits ? (const uint4 *)(m + o_resid) : nullptr;
  L.bscale = (const uint2 *)(m + o_bsc);
  L.rscale = bits ? (const uint2 *)(m + o_rsc) : nullptr;
  L.sign_in = (const int8_t *)(m + o_si);
  L.sign_out = d->sign_out ? (const int8_t *)(m + o_so) : nullptr;
  build_lut(d->levels, L.lut, &L.kinv, &h->level_err);
  L.lut256 = (const uint2 *)(m + o_lut);
  uint2 lut256[256];
  for (int i = 0; i < 256; ++i) lut256[i] = make_uint2(L.lut[i & 15], L.lut[i >> 4]);

  RepackArgs ra;
  ra.base_codes = d->base_codes;
  ra.base_scales = d->base_scales;
  ra.resid_codes = d->resid_codes;
  ra.resid_scales = d->resid_scales;
  ra.base = (uint4 *)(m + o_base);
  ra.resid = bits ? (uint4 *)(m + o_resid) : nullptr;
  ra.bscale = (uint16_t *)(m + o_bsc);
  ra.rscale = bits ? (uint16_t *)(m + o_rsc) : nullptr;
  ra.d_out = h->d_out;
  ra.d_in = h->d_in;
  ra.G = h->G;
  ra.n_tiles = h->n_tiles;
  ra.n_chunks = h->n_chunks;
  e = launch_repack(ra, bits, nullptr);
  if (e == hipSuccess) e = hipMemcpy(m + o_si, si.data(), si.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && d->sign_out) e = hipMemcpy(m + o_so, so.data(), so.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(m + o_lut, lut256, sizeof lut256, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(h->mem);
    delete h;
    return fail(NL_EHIP, "create: repack failed: %s", hipGetErrorString(e));
  }
  h->magic = kMagic;
  live_add(h);
  *out = h;
  return ok();
}

extern "C" nl_status nested_linear_destroy(nl_handle h) {
  if (!valid(h)) return fail(NL_EINVAL, "destroy: invalid handle");
  live_del(h);
  h->magic = 0;
  hipError_t e = hipFree(h->mem);
  delete h;
  if (e != hipSuccess) return fail(NL_EHIP, "destroy: hipFree failed: %s", hipGetErrorString(e));
  return ok();
}

extern "C" nl_status nested_linear_info(nl_handle h, int32_t *d_out, int32_t *d_in, int32_t *bits,
                                        int32_t *block_in, int32_t *block_out, float *level_rel_err) {
  if (!valid(h)) return fail(NL_EINVAL, "info: invalid handle");
  if (d_out) *d_out = h->d_out;
  if (d_in) *d_in = h->d_in;
  if (bits) *bits = h->bits;
  if (block_in) *block_in = h->b_in;
  if (block_out) *block_out = h->b_out;
  if (level_rel_err) *level_rel_err = h->level_err;
  return ok();
}

// ---------------------------------------------------------------------------
// Launch plan and workspace layout of one call.
// ---------------------------------------------------------------------------
struct Plan {
  int rows;       // rows of x' (tokens, or pairs for a grouped call)
  int mt;         // 16-token MFMA tiles
  int tw;         // tile waves per contraction workgroup
  int n_rb;       // row blocks (16 x tile waves rows) per linear
  int S, cps;     // split-K count and chunks per split
  bool finish;    // the staged path needs a finish pass
  int mode;       // single launch: kOutDirect, kOutSplit or kOutTwoSided
  int n_sb, sb_rows;  // output superblocks per linear and their rows
  int n_ctr;      // counters at the start of the workspace
  bool local;     // single launch rotates x inside the contraction workgroups
  size_t o_xh, o_meta, o_part, o_ysum, total;
};

// Launch tuning knobs, read once: NL_WG_TARGET (workgroups the split-K aims
// for, default 256: one per CU) and NL_SPLITS (force the split count).
static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}
static const int g_wg_target = env_int("NL_WG_TARGET", 256);
static const int g_splits = env_int("NL_SPLITS", 0);
// Tile waves of the staged single launch at one to three token tiles: 4 (one
// per SIMD) or 8 (two per SIMD); 0 leaves the planner's choice.
static int g_t_stw = 0;

// tokens: rows of x per linear (T; a grouped call routes each token to an
// expert at most once).
static Plan make_plan(int d_out, int n_tiles, int n_chunks, bool sign_out, int b_out, int rows, int mt,
                      int n_linears, int tokens, int tw, int b_in) {
  Plan p;
  p.rows = rows;
  p.mt = mt;
  p.tw = tw;
  p.n_rb = (n_tiles + tw - 1) / tw;
  // Split K while the grid stays within one workgroup per CU (256 CUs).
  int S = g_wg_target / (p.n_rb * n_linears);
  S = S < 1 ? 1 : (S > n_chunks ? n_chunks : S);
  if (g_splits > 0) S = g_splits < n_chunks ? g_splits : n_chunks;
  p.cps = (n_chunks + S - 1) / S;
  p.S = (n_chunks + p.cps - 1) / p.cps;
  // In-workgroup rotation: a K-range inside one input superblock (SB/512
  // chunks) takes one transform pass, one that straddles two takes two.
  // Align the ranges to the superblocks when that keeps the split count.
  if (g_splits <= 0 && tw == 4 && mt == 1 && tokens <= kLocalTokens) {
    const int cpsb = std::max(b_in, kChunk) / kChunk;
    int c = p.cps;
    if (c < cpsb) {
      while (cpsb % c) ++c;  // a divisor of the superblock
    } else {
      c = (c + cpsb - 1) / cpsb * cpsb;  // whole superblocks
    }
    if (c != p.cps && (n_chunks + c - 1) / c == p.S) p.cps = c;
  }
  p.finish = sign_out || p.S > 1 || n_linears > 1;
  p.mode = sign_out ? kOutTwoSided : (p.S > 1 ? kOutSplit : kOutDirect);
  p.local = tw == 4 && mt == 1 && tokens <= kLocalTokens && p.cps <= kLocalChunks;
  if (p.local) p.mt = 0;
  p.sb_rows = finish_rows(sign_out, b_out);
  p.n_sb = (d_out + p.sb_rows - 1) / p.sb_rows;
  p.n_ctr = kCtrFixed + n_linears * p.n_rb + 2 * n_linears * p.n_sb;
  const size_t Kp = (size_t)n_chunks * kChunk;
  p.o_xh = kCtrBytes;
  p.o_meta = align256(p.o_xh + (size_t)rows * Kp * 2);
  p.o_part = align256(p.o_meta + (size_t)rows * n_chunks * 5 * 4);
  p.o_ysum = align256(p.o_part + (p.finish ? (size_t)p.S * rows * d_out * 4 : 0));
  p.total = align256(p.o_ysum + (sign_out ? (size_t)rows * d_out * 4 : 0));
  return p;
}

static int mt_for(int T) { return (T + 15) / 16; }

// Tile waves of the staged single launch (the three-launch form keeps
// tile_waves: its contraction kernel has one variant per token-tile count).
static int staged_tile_waves(int T) {
  const int mt = mt_for(T);
  if (g_t_stw == 8 && mt <= 3 && T > kLocalTokens) return 8;
  if (g_t_stw == 4 && mt <= 2) return 4;
  return tile_waves(mt);
}

static nl_status check_call(nl_handle h, const char *who, int verify, int32_t T, const void *ws,
                            size_t ws_bytes, Plan *plan, int tw) {
  if (!valid(h)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (verify && !h->bits) return fail(NL_EINVAL, "%s: the linear has no residual (draft only)", who);
  if (T < 1) return fail(NL_EINVAL, "%s: T must be >= 1 (got %d)", who, T);
  if (T > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T = %d exceeds %d", who, T, NL_MAX_T);
  if (!ws) return fail(NL_EINVAL, "%s: NULL workspace", who);
  if ((uintptr_t)ws & 255) return fail(NL_EINVAL, "%s: workspace must be 256-byte aligned", who);
  *plan = make_plan(h->d_out, h->n_tiles, h->n_chunks, h->has_sign_out, h->b_out, T, mt_for(T), 1, T, tw,
                    h->b_in);
  if (ws_bytes < plan->total)
    return fail(NL_EINVAL, "%s: workspace too small (%zu < %zu)", who, ws_bytes, plan->total);
  if (plan->n_ctr > kCtrLines)
    return fail(NL_EUNSUPPORTED, "%s: d_out = %d needs %d counters (> %d)", who, h->d_out, plan->n_ctr, kCtrLines);
  return NL_OK;
}

static RotInArgs rot_args(nl_handle h, const void *x, int T, char *ws, const Plan &p) {
  RotInArgs r;
  memset(&r, 0, sizeof r);
  r.x = (const uint16_t *)x;
  r.sign = h->dev.sign_in;
  r.x_rows = T;
  r.rows = T;
  r.lb = log2i(h->b_in);
  r.xh = (uint16_t *)(ws + p.o_xh);
  r.meta = (float *)(ws + p.o_meta);
  r.d_in = h->d_in;
  r.b = h->b_in;
  r.SB = h->b_in > kChunk ? h->b_in : kChunk;
  r.Kp = h->n_chunks * kChunk;
  r.Gp = h->n_chunks * 4;
  r.n_chunks = h->n_chunks;
  r.rsqrt_b = (float)(1.0 / std::sqrt((double)h->b_in));
  return r;
}

extern "C" nl_status nested_linear_prepare_input(nl_handle h, const void *x, int32_t T, void *ws,
                                                 size_t ws_bytes, void *stream) {
  Plan p;
  nl_status st = check_call(h, "prepare_input", 0, T, ws, ws_bytes, &p, tile_waves(mt_for(T)));
  if (st != NL_OK) return st;
  if (!x) return fail(NL_EINVAL, "prepare_input: NULL x");
  if ((uintptr_t)x & 15) return fail(NL_EINVAL, "prepare_input: x must be 16-byte aligned");
  RotInArgs r = rot_args(h, x, T, (char *)ws, p);
  HIP_OR_FAIL(launch_rotate_in(r, T, (hipStream_t)stream));
  return ok();
}

extern "C" nl_status nested_linear_contract(nl_handle h, int32_t verify, int32_t T, float *y,
                                            void *ws, size_t ws_bytes, void *stream) {
  Plan p;
  nl_status st = check_call(h, "contract", verify, T, ws, ws_bytes, &p, tile_waves(mt_for(T)));
  if (st != NL_OK) return st;
  if (!y && !p.finish) return fail(NL_EINVAL, "contract: NULL y");
  char *w = (char *)ws;
  GemmArgs g;
  memset(&g, 0, sizeof g);
  g.lin = h->dev;
  g.xh = (const uint16_t *)(w + p.o_xh);
  g.meta = (const float *)(w + p.o_meta);
  g.out = p.finish ? (float *)(w + p.o_part) : y;
  g.split_stride = (size_t)T * h->d_out;
  g.T = T;
  g.d_out = h->d_out;
  g.n_tiles = h->n_tiles;
  g.n_chunks = h->n_chunks;
  g.Kp = h->n_chunks * kChunk;
  g.Gp = h->n_chunks * 4;
  g.cps = p.cps;
  g.ldo = h->d_out;
  g.n_rb = p.n_rb;
  g.n_experts = 1;
  HIP_OR_FAIL(launch_gemm(g, verify ? h->bits : 0, mt_for(T), p.S, (hipStream_t)stream));
  return ok();
}

extern "C" nl_status nested_linear_finish(nl_handle h, int32_t T, float *y, void *ws, size_t ws_bytes,
                                          void *stream) {
  Plan p;
  nl_status st = check_call(h, "finish", 0, T, ws, ws_bytes, &p, tile_waves(mt_for(T)));
  if (st != NL_OK) return st;
  if (!y) return fail(NL_EINVAL, "finish: NULL y");
  if (!p.finish) return ok();
  FinishArgs f;
  memset(&f, 0, sizeof f);
  f.part = (const float *)((char *)ws + p.o_part);
  f.split_stride = (size_t)T * h->d_out;
  f.y = y;
  f.sign_out = h->dev.sign_out;
  f.T = T;
  f.d_out = h->d_out;
  f.S = p.S;
  f.b = h->b_out;
  f.lb = log2i(h->b_out);
  f.OB = finish_rows(h->has_sign_out, h->b_out);
  f.rsqrt_b = (float)(1.0 / std::sqrt((double)h->b_out));
  HIP_OR_FAIL(launch_finish(f, (hipStream_t)stream));
  return ok();
}

// Waits between workgroups: polls before a wait gives up, and extra tokens a
// wait asks for (set from the host so a lost hand-over can be shown).
static uint32_t g_spin_limit = 1u << 22;
static uint32_t g_wait_extra = 0;

// Counter bases, grid sizes and semaphore lines of one call.
static void fill_launch(FwdArgs &f, const Plan &p, int n_linears, char *ws, float *y, int d_out) {
  f.hv.ctr = (uint32_t *)ws;
  f.hv.y = y;
  f.hv.ysum = p.mode == kOutTwoSided ? (float *)(ws + p.o_ysum) : nullptr;
  f.hv.mode = p.mode;
  f.hv.S = p.S;
  f.hv.sb_rows = p.sb_rows;
  f.hv.n_sb = p.n_sb;
  f.hv.rb_base = kCtrFixed;
  f.hv.ob_base = kCtrFixed + n_linears * p.n_rb;
  f.hv.obr_base = f.hv.ob_base + n_linears * p.n_sb;
  // a rotation workgroup of 512 threads or more runs two transform groups
  f.rot.groups = 64 * (p.tw + 1) >= 512 ? 2 : 1;
  f.n_rot = p.local ? 0 : rotate_workgroups(p.rows, f.rot.Kp, f.rot.SB, f.rot.groups);
  // Contraction workgroups: one slot of them per linear, or, when that
  // halves the grid, one per linear that can have rows (each has one at
  // least, so at most rows of them do).  The slot's workgroups then find
  // their expert with a scan of the offsets, one memory round trip ahead of
  // the descriptor: that pays only where idle experts outnumber the rest.
  const int per = p.n_rb * p.S;
  const int cap = std::min(n_linears, p.rows);
  f.g.slots = n_linears > 1 && 2 * cap < n_linears;
  f.n_gemm = (f.g.slots ? cap : n_linears) * per;
  f.hv.n_rot = f.n_rot;
  f.hv.spin_limit = g_spin_limit;
  f.hv.wait_extra = g_wait_extra;
  f.g.out = p.mode == kOutDirect ? y : (float *)(ws + p.o_part);
  f.g.split_stride = (size_t)p.rows * d_out;
  f.fin.y = y;
  f.fin.T = p.rows;
  f.fin.d_out = d_out;
  f.fin.S = 1;
  f.fin.OB = p.sb_rows;
}

// ---------------------------------------------------------------------------
// Kernel timing: event pairs attached to the single launch of each call.
// ---------------------------------------------------------------------------
static struct {
  std::vector<hipEvent_t> ev;  // 2 per slot
  int used = 0;
  bool on = false;
} g_timing;

static void release_timing() {
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.used = 0;
  g_timing.on = false;
}

// The next free event pair, or nulls when timing is off, full, or the
// stream is being captured into a graph.
static void timing_slot(hipStream_t s, hipEvent_t *e0, hipEvent_t *e1) {
  *e0 = *e1 = nullptr;
  if (!g_timing.on || 2 * g_timing.used >= (int)g_timing.ev.size()) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  *e0 = g_timing.ev[2 * g_timing.used];
  *e1 = g_timing.ev[2 * g_timing.used + 1];
  ++g_timing.used;
}

extern "C" nl_status nested_linear_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t grid,
                                               void *stream) {
  if (!src || !sink) return fail(NL_EINVAL, "stream_read: NULL pointer");
  if (bytes == 0 || (bytes & 15) || ((uintptr_t)src & 15))
    return fail(NL_EINVAL, "stream_read: bytes must be a positive multiple of 16 and src 16-byte aligned");
  if (grid < 0 || grid > (1 << 20)) return fail(NL_EINVAL, "stream_read: grid must be in [0, 2^20]");
  HIP_OR_FAIL(launch_stream_read(src, bytes, sink, grid ? grid : 2048, (hipStream_t)stream));
  return ok();
}

extern "C" nl_status nested_linear_timing_begin(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return fail(NL_EINVAL, "timing_begin: capacity must be in [1, 2^20]");
  release_timing();
  g_timing.ev.assign(2 * (size_t)capacity, nullptr);
  for (hipEvent_t &e : g_timing.ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      release_timing();
      return fail(NL_EHIP, "timing_begin: %s", hipGetErrorString(r));
    }
  }
  g_timing.on = true;
  return ok();
}

extern "C" nl_status nested_linear_timing_end(float *us, int32_t capacity, int32_t *count) {
  if (!g_timing.on) return fail(NL_EINVAL, "timing_end: timing was not begun");
  if (!count || (capacity > 0 && !us)) {
    release_timing();
    return fail(NL_EINVAL, "timing_end: NULL us or count");
  }
  const int n = g_timing.used < capacity ? g_timing.used : capacity;
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(g_timing.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    if (r != hipSuccess) {
      release_timing();
      return fail(NL_EHIP, "timing_end: %s", hipGetErrorString(r));
    }
    us[i] = ms * 1000.f;
  }
  *count = n;
  release_timing();
  return ok();
}

// ---------------------------------------------------------------------------
// Single-launch forward (nl_fwd.hip): plan and workspace of one call over n
// linears that read the same x (n = 1 for nested_linear_verify / draft).
// ---------------------------------------------------------------------------
struct JobPlan {
  int rt, kw, S, cps, n_rb, n_sb;
  size_t o_xb, o_part, o_ysum;
  int ctr_split, ctr_sb;
};
struct Plan2 {
  int n, T, mt, nw, blob, tm, SB, OB;
  bool local, two;
  int n_rot, n_con, n_fin, n_ctr, rot_groups;
  size_t lds, total;
  JobPlan j[kMaxJobs];
};

// Tuning knobs (nested_linear_set_tuning): forced split count, row tiles and
// waves per tile (0 = planner's choice), the largest T of the local form, and
// the cost model's rates.
static int g_t_S = 0, g_t_rt = 0, g_t_kw = 0, g_t_local = 2, g_t_cus = 256, g_t_nw = 0;
static double g_t_lat_us = 2.0, g_t_hbm_gbs = 6500.0, g_t_split_us = 1.5, g_t_xdma_gbs = 100.0;
// Single-linear calls with T at or above this use the staged-x' launch
// (forward_kernel: x' passes through LDS a chunk at a time, so no split of K is
// forced by T), below it the single launch that holds the K-range's x' in LDS.
// Measured on the 7B/8B-class projections: the latter is ahead for verify up
// to T = 8, the former from T = 16 on and for the draft at every T.
static int g_t_staged_v = 9, g_t_staged_d = 1;
// Multi-linear calls whose linears share the shape take the staged launch's
// grouped form from these T on (verify, draft; 65: never).  Measured on gate
// and up of the 7B/8B-class layer (2 x 14336x4096): verify equal at T = 24-32
// and 24-28% faster at 48-64; draft 5% faster at 24 and 38% at 64; both
// slower at T = 16 and below.
static int g_t_ms_v = 33, g_t_ms_d = 24;

// One pass of the in-workgroup transform (4096 points per 256 threads) in
// the local form, us: it runs while the weight stream is queued (measured
// 2.6-4.8 us there, 1.4 us in a rotation workgroup of its own).
static const double kRotPassUs = 3.0;

// Bytes of one tile-chunk (16 rows x 512 columns) in a pass.
static double tc_bytes(int bits) { return 16.0 * 512.0 * (0.265625 + (bits ? bits / 8.0 + 1.0 / 64.0 : 0.0)); }

// Local form: transform passes a split [c_lo, c_hi) needs (at most 2).
static int local_passes(int T, int n_chunks, int cps, int SB, int G) {
  int np = 0;
  for (int c_lo = 0; c_lo < n_chunks; c_lo += cps) {
    const int c_hi = std::min(n_chunks, c_lo + cps);
    const int sb0 = (c_lo * kChunk) / SB, sb1 = (c_hi * kChunk + SB - 1) / SB;
    const int per = G * (4096 / SB);
    np = std::max(np, (T * (sb1 - sb0) + per - 1) / per);
  }
  return np;
}

// Split count, row tiles per workgroup and waves per tile of one linear, by a
// small cost model (microseconds).  A wave streams its chunks through a ring
// of ns register sets, so it spends about one memory round trip (lat) per ns
// chunks, or its compute if that is longer (the waves of a SIMD share it);
// the call takes about the larger of the slowest wave of each round of
// workgroups and the HBM time of all bytes, plus the split-K reduction and
// the x' copies into LDS.  Ties go to more active waves, then fewer splits.
static void choose_job(int n_tiles, int n_chunks, int T, int bits, int mt, int nw, int ns, bool two, bool local,
                       int SB, int blob, int lds_fixed, double cus, JobPlan &jp) {
  const int G = nw / 4;
  const int budget = 160 * 1024 - lds_fixed;
  const int kc_max = std::max(1, budget / blob);
  const double tcb = tc_bytes(bits);
  const double t_c = (bits ? 0.35 : 0.15) * (1.0 + 0.6 * (mt - 1));  // us per chunk, one wave on its SIMD
  const double total = (double)n_tiles * n_chunks * tcb;
  double best = 1e30;
  jp.S = jp.cps = jp.rt = jp.kw = 0;
  for (int cps0 = n_chunks; cps0 >= 1; --cps0) {
    const int S = (n_chunks + cps0 - 1) / cps0, cps = (n_chunks + S - 1) / S;
    if (cps != cps0) continue;  // each split count once
    if (cps > kc_max) continue;
    if (g_t_S > 0 && S != g_t_S) continue;
    if (local && local_passes(T, n_chunks, cps, SB, G) > 2) continue;
    for (int rt = 1; rt <= nw; ++rt) {
      if (two && (rt & (rt - 1))) continue;  // row blocks inside one output superblock
      if (g_t_rt > 0 && rt != g_t_rt) continue;
      for (int kw = 1; rt * kw <= nw && kw <= cps; ++kw) {
        if (g_t_kw > 0 && kw != g_t_kw) continue;
        const int n_rb = (n_tiles + rt - 1) / rt, n_wg = n_rb * S;
        const int rounds = (int)std::ceil(n_wg / cus);
        const int wc = (cps + kw - 1) / kw;               // chunks of the busiest wave
        const int active = rt * ((cps + wc - 1) / wc);    // waves that have chunks
        const double share = std::max(1.0, active / 4.0);  // waves per SIMD
        const double t_wave = wc * std::max(g_t_lat_us / std::min(ns, wc), t_c * share) + g_t_lat_us;
        const double xdma = local ? 0.0 : cps * (double)blob / (g_t_xdma_gbs * 1e3);
        // local form: each pass of the workgroup's transform precedes its contraction
        const double rot = local ? kRotPassUs * local_passes(T, n_chunks, cps, SB, G) : 0.0;
        const double split = S > 1 ? g_t_split_us + 2.0 * S * T * n_tiles * 16.0 * 4.0 / (g_t_hbm_gbs * 1e3) : 0.0;
        // the slowest wave chain and the HBM time overlap but not completely:
        // a smooth maximum (4-norm) keeps both in view
        const double a = rounds * (t_wave + xdma + rot), b = total / (g_t_hbm_gbs * 1e3);
        const double cost = std::pow(std::pow(a, 4.0) + std::pow(b, 4.0), 0.25) + split + 1e-3 * (nw - active) + 1e-4 * S;
        if (cost < best) {
          best = cost;
          jp.S = S;
          jp.cps = cps;
          jp.rt = rt;
          jp.kw = kw;
        }
      }
    }
  }
  if (jp.S == 0) {  // forced knobs that fit nothing: the plainest plan that fits
    jp.cps = std::min(kc_max, n_chunks);
    jp.S = (n_chunks + jp.cps - 1) / jp.cps;
    jp.cps = (n_chunks + jp.S - 1) / jp.S;
    jp.rt = 1;
    jp.kw = std::min(nw, jp.cps);
  }
  jp.n_rb = (n_tiles + jp.rt - 1) / jp.rt;
}

// The shape facts a plan depends on.
struct CallShape {
  int d_out, n_tiles, n_chunks, b_in, b_out;
  bool sign_out;
};
static CallShape shape_of(const nl_linear *h) {
  return CallShape{h->d_out, h->n_tiles, h->n_chunks, h->b_in, h->b_out, h->has_sign_out};
}

static Plan2 make_plan2(const CallShape *hs, int n, int T, int bits) {
  Plan2 p;
  memset(&p, 0, sizeof p);
  p.n = n;
  p.T = T;
  p.mt = mt_for(T);
  // one token tile: eight waves with a four-set ring for the draft (its sets
  // are small; the knob can ask for twelve), twelve for verify
  p.nw = p.mt != 1 ? fwd_waves(p.mt) : (bits == 0 && g_t_nw != 12) ? 8 : 12;
  p.blob = blob_bytes(T);
  p.tm = blob_tm(T);
  const CallShape *h0 = &hs[0];
  p.SB = std::max(h0->b_in, kChunk);
  p.two = h0->sign_out;
  p.OB = p.two ? std::max(h0->b_out, kChunk) : 0;
  const int G = p.nw / 4;
  const int n_chunks = h0->n_chunks;
  const int n_sbi = (n_chunks * kChunk) / p.SB;
  p.local = !p.two && p.mt == 1 && T <= g_t_local;
  if (p.local) {  // every linear's K must fit two transform passes at some split count
    for (int c = n_chunks; c >= 1; --c)
      if (local_passes(T, n_chunks, c, p.SB, G) <= 2) {
        if ((c * p.blob) > 160 * 1024 - kLdsX - G * kFwhtArea) p.local = false;
        break;
      }
  }
  const int lds_fixed = kLdsX + (p.local ? G * kFwhtArea + 16 : 0);
  // rotation: one 256-thread transform group per workgroup while that takes
  // at most 32 workgroups, more groups per workgroup beyond
  const int task_groups = (n * T * n_sbi + (4096 / p.SB) - 1) / (4096 / p.SB);
  p.rot_groups = std::min(G, std::max(1, (task_groups + 31) / 32));
  p.n_rot = p.local ? 0 : (task_groups + p.rot_groups - 1) / p.rot_groups;
  // the rotation workgroups hold their CUs until the hand-over
  const double cus_free = std::max(32.0, (double)g_t_cus - p.n_rot);
  double total_tc = 0;
  for (int i = 0; i < n; ++i) total_tc += (double)hs[i].n_tiles;
  size_t off = kCtrBytes;
  int ctr = kCtrFixed, con = 0, fin_tasks = 0;
  int lds_blob = 0;
  for (int i = 0; i < n; ++i) {
    const CallShape *h = &hs[i];
    JobPlan &jp = p.j[i];
    const double cus = std::max(1.0, cus_free * h->n_tiles / total_tc);
    choose_job(h->n_tiles, n_chunks, T, bits, p.mt, p.nw, fwd_ring_sets(bits, p.mt, p.local, p.nw), p.two, p.local, p.SB,
               p.blob, lds_fixed, cus, jp);
    jp.n_sb = p.two ? (h->d_out + p.OB - 1) / p.OB : 0;
    jp.o_xb = off;
    off = align256(off + (size_t)n_chunks * p.blob);
    jp.o_part = off;
    if (jp.S > 1) off = align256(off + (size_t)jp.S * T * h->d_out * 4);
    jp.o_ysum = off;
    if (p.two) off = align256(off + (size_t)T * h->d_out * 4);
    jp.ctr_split = ctr;
    if (jp.S > 1) ctr += jp.n_rb;
    jp.ctr_sb = ctr;
    if (p.two) ctr += 2 * jp.n_sb;
    con += jp.n_rb * jp.S;
    fin_tasks += T * jp.n_sb;
    lds_blob = std::max(lds_blob, jp.cps * p.blob);
  }
  p.n_ctr = ctr;
  p.n_con = con;
  p.n_fin = p.two ? (fin_tasks + G * (4096 / p.OB) - 1) / (G * (4096 / p.OB)) : 0;
  size_t lds = kLdsX + (size_t)std::max(p.nw * p.mt * 1024, ((lds_blob + 15) & ~15) + (p.local ? G * kFwhtArea : 0));
  if (p.n_rot || p.n_fin) lds = std::max(lds, (size_t)kLdsX + G * kFwhtArea);
  p.lds = lds;
  p.total = off;
  return p;
}

// ---------------------------------------------------------------------------
// Multi-linear calls of one shape (gate and up, say) at large T: the staged
// launch's grouped form.  Linear q is expert q and owns pair rows q*T .. q*T
// + T - 1 of x' (its own rotation of x with its own signs; pair q*T + t
// reads token t), and its rows go to its own y.  The expert array, the
// offsets and the pair tokens live at the end of the workspace, written by
// a small kernel on the same stream (a kernel, not a copy, so that the call
// can be captured into a graph).
// ---------------------------------------------------------------------------
struct MultiSetupArgs {
  LinearDev lin[kMaxJobs];
  int n, T;
  LinearDev *lins;
  int32_t *offsets, *pairs;
};
static_assert(kMaxJobs <= 4, "GemmArgs::ys holds four outputs");

__global__ __launch_bounds__(256) void multi_setup_kernel(const MultiSetupArgs s) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
#pragma unroll
    for (int q = 0; q < kMaxJobs; ++q)
      if (q < s.n) s.lins[q] = s.lin[q];
  }
  if (i <= s.n) s.offsets[i] = i * s.T;
  if (i < s.n * s.T) s.pairs[i] = i % s.T;
}

static bool multi_staged_route(const nl_linear *const *hs, int n, int verify, int T) {
  if (n < 2 || hs[0]->has_sign_out || T < (verify ? g_t_ms_v : g_t_ms_d)) return false;
  for (int i = 1; i < n; ++i)
    if (hs[i]->d_out != hs[0]->d_out || hs[i]->b_in != hs[0]->b_in || hs[i]->bits != hs[0]->bits) return false;
  return true;
}

struct MultiPlan {
  Plan p;
  size_t o_lins, o_off, o_pairs, total;
};
static MultiPlan multi_plan(const nl_linear *h0, int n, int T) {
  MultiPlan m;
  m.p = make_plan(h0->d_out, h0->n_tiles, h0->n_chunks, false, h0->b_out, n * T, mt_for(T), n, T,
                  tile_waves(mt_for(T)), h0->b_in);
  m.o_lins = align256(m.p.total);
  m.o_off = align256(m.o_lins + sizeof(LinearDev) * n);
  m.o_pairs = align256(m.o_off + sizeof(int32_t) * (n + 1));
  m.total = align256(m.o_pairs + sizeof(int32_t) * n * T);
  return m;
}

static nl_status forward_multi_staged(const nl_linear *const *hs, int n, int verify, const void *x, int32_t T,
                                      float *const *ys, void *ws, size_t ws_bytes, void *stream, const char *who) {
  const nl_linear *h0 = hs[0];
  const MultiPlan m = multi_plan(h0, n, T);
  const Plan &p = m.p;
  if (ws_bytes < m.total) return fail(NL_EINVAL, "%s: workspace too small (%zu < %zu)", who, ws_bytes, m.total);
  if (p.n_ctr > kCtrLines) return fail(NL_EUNSUPPORTED, "%s: the call needs %d counters (> %d)", who, p.n_ctr, kCtrLines);
  // the eight-tile-wave variants of one and two token tiles have no per-linear outputs
  if (p.tw == 8 && p.mt < 3) return fail(NL_EUNSUPPORTED, "%s: no staged multi-linear form at T = %d", who, T);
  char *w = (char *)ws;
  MultiSetupArgs sa;
  memset(&sa, 0, sizeof sa);
  for (int i = 0; i < n; ++i) sa.lin[i] = hs[i]->dev;
  sa.n = n;
  sa.T = T;
  sa.lins = (LinearDev *)(w + m.o_lins);
  sa.offsets = (int32_t *)(w + m.o_off);
  sa.pairs = (int32_t *)(w + m.o_pairs);
  hipLaunchKernelGGL(multi_setup_kernel, dim3((n * T + 256) / 256), dim3(256), 0, (hipStream_t)stream, sa);
  HIP_OR_FAIL(hipGetLastError());

  FwdArgs f;
  memset(&f, 0, sizeof f);
  RotInArgs &r = f.rot;
  r.x = (const uint16_t *)x;
  r.lins = sa.lins;
  r.pair_token = sa.pairs;
  r.offsets = sa.offsets;
  r.n_experts = n;
  r.x_rows = T;
  r.rows = n * T;
  r.lb = log2i(h0->b_in);
  r.xh = (uint16_t *)(w + p.o_xh);
  r.meta = (float *)(w + p.o_meta);
  r.d_in = h0->d_in;
  r.b = h0->b_in;
  r.SB = h0->b_in > kChunk ? h0->b_in : kChunk;
  r.Kp = h0->n_chunks * kChunk;
  r.Gp = h0->n_chunks * 4;
  r.n_chunks = h0->n_chunks;
  r.rsqrt_b = (float)(1.0 / std::sqrt((double)h0->b_in));
  GemmArgs &ga = f.g;
  ga.lins = sa.lins;
  ga.offsets = sa.offsets;
  ga.xh = (const uint16_t *)(w + p.o_xh);
  ga.meta = (const float *)(w + p.o_meta);
  ga.T = n * T;
  ga.d_out = h0->d_out;
  ga.n_tiles = h0->n_tiles;
  ga.n_chunks = h0->n_chunks;
  ga.Kp = r.Kp;
  ga.Gp = r.Gp;
  ga.cps = p.cps;
  ga.ldo = h0->d_out;
  ga.n_rb = p.n_rb;
  ga.n_experts = n;
  for (int i = 0; i < n; ++i) ga.ys[i] = ys[i];
  fill_launch(f, p, n, w, ys[0], h0->d_out);
  hipEvent_t e0, e1;
  timing_slot((hipStream_t)stream, &e0, &e1);
  HIP_OR_FAIL(launch_forward(f, verify ? h0->bits : 0, p.mt, p.tw, 0, (hipStream_t)stream, e0, e1));
  return ok();
}

static nl_status forward_n(const nl_linear *const *hs, int n, int verify, const void *x, int32_t T, float *const *ys,
                           void *ws, size_t ws_bytes, void *stream, const char *who) {
  if (n < 1 || n > kMaxJobs) return fail(NL_EINVAL, "%s: between 1 and %d linears per call (got %d)", who, kMaxJobs, n);
  for (int i = 0; i < n; ++i) {
    if (!valid(hs[i])) return fail(NL_EINVAL, "%s: linear %d is not a valid handle", who, i);
    if (verify && !hs[i]->bits) return fail(NL_EINVAL, "%s: linear %d has no residual (draft only)", who, i);
    if (hs[i]->d_in != hs[0]->d_in) return fail(NL_EINVAL, "%s: linear %d differs in d_in", who, i);
    if (verify && hs[i]->bits != hs[0]->bits)
      return fail(NL_EINVAL, "%s: linear %d differs in residual bits", who, i);
    if (hs[i]->has_sign_out != hs[0]->has_sign_out || (hs[0]->has_sign_out && hs[i]->b_out != hs[0]->b_out))
      return fail(NL_EINVAL, "%s: linear %d differs in the output rotation (presence or block)", who, i);
    if (!ys || !ys[i]) return fail(NL_EINVAL, "%s: NULL y", who);
  }
  if (T < 1) return fail(NL_EINVAL, "%s: T must be >= 1 (got %d)", who, T);
  if (T > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T = %d exceeds %d", who, T, NL_MAX_T);
  if (!x) return fail(NL_EINVAL, "%s: NULL x", who);
  if ((uintptr_t)x & 15) return fail(NL_EINVAL, "%s: x must be 16-byte aligned", who);
  if (!ws) return fail(NL_EINVAL, "%s: NULL workspace", who);
  if ((uintptr_t)ws & 255) return fail(NL_EINVAL, "%s: workspace must be 256-byte aligned", who);
  if (multi_staged_route(hs, n, verify, T)) return forward_multi_staged(hs, n, verify, x, T, ys, ws, ws_bytes, stream, who);
  const int bits = verify ? hs[0]->bits : 0;
  CallShape cs[kMaxJobs];
  for (int i = 0; i < n; ++i) cs[i] = shape_of(hs[i]);
  Plan2 p = make_plan2(cs, n, T, bits);
  if (ws_bytes < p.total) return fail(NL_EINVAL, "%s: workspace too small (%zu < %zu)", who, ws_bytes, p.total);
  if (p.n_ctr > kCtrLines) return fail(NL_EUNSUPPORTED, "%s: the call needs %d counters (> %d)", who, p.n_ctr, kCtrLines);
  if (p.total > 0x7FFFFFF0u) return fail(NL_EUNSUPPORTED, "%s: workspace layout beyond 2 GiB", who);
  char *w = (char *)ws;
  FwdArgs2 a;
  memset(&a, 0, sizeof a);
  a.x = (const uint16_t *)x;
  a.ws = w;
  a.T = T;
  a.d_in = hs[0]->d_in;
  a.n_chunks = hs[0]->n_chunks;
  a.Kp = hs[0]->n_chunks * kChunk;
  a.lb_in = log2i(hs[0]->b_in);
  a.SB = p.SB;
  a.rsqrt_in = (float)(1.0 / std::sqrt((double)hs[0]->b_in));
  a.lb_out = p.two ? log2i(hs[0]->b_out) : 0;
  a.OB = p.OB;
  a.rsqrt_out = p.two ? (float)(1.0 / std::sqrt((double)hs[0]->b_out)) : 0.f;
  a.blob = p.blob;
  a.tm = p.tm;
  a.n_jobs = n;
  a.n_rot = p.n_rot;
  a.n_con = p.n_con;
  a.n_fin = p.n_fin;
  a.rot_groups = p.rot_groups;
  a.spin_limit = g_spin_limit;
  a.wait_extra = g_wait_extra;
  int con = 0;
  for (int i = 0; i < n; ++i) {
    const JobPlan &jp = p.j[i];
    FwdJob &J = a.job[i];
    J.lin = hs[i]->dev;
    J.y = ys[i];
    J.part = (float *)(w + jp.o_part);
    J.ysum = p.two ? (float *)(w + jp.o_ysum) : nullptr;
    J.xb = (int)jp.o_xb;
    J.d_out = hs[i]->d_out;
    J.n_tiles = hs[i]->n_tiles;
    J.rt = jp.rt;
    J.kw = jp.kw;
    J.n_rb = jp.n_rb;
    J.S = jp.S;
    J.cps = jp.cps;
    J.con0 = con;
    J.ctr_split = jp.ctr_split;
    J.ctr_sb = jp.ctr_sb;
    J.n_sb = jp.n_sb;
    con += jp.n_rb * jp.S;
  }
  hipEvent_t e0, e1;
  timing_slot((hipStream_t)stream, &e0, &e1);
  HIP_OR_FAIL(launch_forward2(a, bits, p.mt, p.nw, p.local, p.lds, (hipStream_t)stream, e0, e1));
  return ok();
}

// The staged-x' launch of one linear (forward_kernel): rotation workgroups
// write x' to the workspace, contraction workgroups stage it through LDS one
// chunk at a time beside their weight stream.
static nl_status forward_staged(nl_handle h, int verify, const void *x, int32_t T, float *y, void *ws,
                                size_t ws_bytes, void *stream, const char *who) {
  Plan p;
  nl_status st = check_call(h, who, verify, T, ws, ws_bytes, &p, staged_tile_waves(T));
  if (st != NL_OK) return st;
  if (!x || !y) return fail(NL_EINVAL, "%s: NULL x or y", who);
  if ((uintptr_t)x & 15) return fail(NL_EINVAL, "%s: x must be 16-byte aligned", who);
  char *w = (char *)ws;
  FwdArgs f;
  memset(&f, 0, sizeof f);
  f.rot = rot_args(h, x, T, w, p);
  GemmArgs &g = f.g;
  g.lin = h->dev;
  g.xh = (const uint16_t *)(w + p.o_xh);
  g.meta = (const float *)(w + p.o_meta);
  g.T = T;
  g.d_out = h->d_out;
  g.n_tiles = h->n_tiles;
  g.n_chunks = h->n_chunks;
  g.Kp = h->n_chunks * kChunk;
  g.Gp = h->n_chunks * 4;
  g.cps = p.cps;
  g.ldo = h->d_out;
  g.n_rb = p.n_rb;
  g.n_experts = 1;
  f.fin.sign_out = h->dev.sign_out;
  f.fin.b = h->b_out;
  f.fin.lb = log2i(h->b_out);
  f.fin.rsqrt_b = (float)(1.0 / std::sqrt((double)h->b_out));
  fill_launch(f, p, 1, w, y, h->d_out);
  const int n_fin = p.mode == kOutTwoSided ? finish_workgroups(T, h->d_out, p.sb_rows) : 0;
  hipEvent_t e0, e1;
  timing_slot((hipStream_t)stream, &e0, &e1);
  HIP_OR_FAIL(launch_forward(f, verify ? h->bits : 0, p.mt, p.tw, n_fin, (hipStream_t)stream, e0, e1));
  return ok();
}

static bool use_staged(int verify, int T) { return T >= (verify ? g_t_staged_v : g_t_staged_d); }

static nl_status forward(nl_handle h, int verify, const void *x, int32_t T, float *y, void *ws,
                         size_t ws_bytes, void *stream, const char *who) {
  if (!valid(h)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (use_staged(verify, T) && T <= NL_MAX_T) return forward_staged(h, verify, x, T, y, ws, ws_bytes, stream, who);
  const nl_linear *hs[1] = {h};
  float *ys[1] = {y};
  return forward_n(hs, 1, verify, x, T, ys, ws, ws_bytes, stream, who);
}

// ---------------------------------------------------------------------------
// Forward without allocation: the workspace is a static device array, one per
// GPU, held until the process ends.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
static std::mutex g_scratch_mu;
static char *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of the array, looked up once per device
// with that device current (the array's name is a host-side stand-in).
static nl_status scratch_on_current_device(char **out) {
  int dev = 0;
  HIP_OR_FAIL(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(NL_EUNSUPPORTED, "forward_static: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(NL_EHIP, "forward_static: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = (char *)p;
  }
  *out = g_scratch_ptr[dev];
  return NL_OK;
}

// Zero the first n words (the counters a call uses; a fill kernel rather than
// a memset, so that the call can be captured into a graph).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

extern "C" nl_status nested_linear_forward_static(nl_handle h, int32_t verify, const void *x, int32_t T, float *y,
                                                  void *stream) {
  const char *who = "forward_static";
  if (!valid(h)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (verify && !h->bits) return fail(NL_EINVAL, "%s: the linear has no residual (draft only)", who);
  if (T < 1) return fail(NL_EINVAL, "%s: T must be >= 1 (got %d)", who, T);
  if (T > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T = %d exceeds %d", who, T, NL_MAX_T);
  size_t total;
  int n_ctr;
  if (use_staged(verify, T)) {
    const Plan p = make_plan(h->d_out, h->n_tiles, h->n_chunks, h->has_sign_out, h->b_out, T, mt_for(T), 1, T,
                             staged_tile_waves(T), h->b_in);
    total = p.total;
    n_ctr = p.n_ctr;
  } else {
    const CallShape cs[1] = {shape_of(h)};
    const Plan2 p = make_plan2(cs, 1, T, verify ? h->bits : 0);
    total = p.total;
    n_ctr = p.n_ctr;
  }
  if (total > kScratchBytes)
    return fail(NL_EUNSUPPORTED, "%s: the call needs %zu bytes of scratch, beyond the library's %zu", who, total,
                kScratchBytes);
  if (n_ctr > kCtrLines) return fail(NL_EUNSUPPORTED, "%s: the call needs %d counters (> %d)", who, n_ctr, kCtrLines);
  char *ws = nullptr;
  const nl_status st = scratch_on_current_device(&ws);
  if (st != NL_OK) return st;
  // the previous call on this GPU left its counters at zero unless a wait gave
  // up; clear them anyway so that no earlier failure carries over
  const int words = n_ctr * kCtrStride;
  hipLaunchKernelGGL(clear_words_kernel, dim3(std::min(64, (words + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (uint32_t *)ws, words);
  HIP_OR_FAIL(hipGetLastError());
  return forward(h, verify ? 1 : 0, x, T, y, ws, kScratchBytes, stream, who);
}

extern "C" nl_status nested_linear_describe_call(const int32_t *d_out, int32_t n, int32_t d_in, int32_t bits,
                                                 int32_t two_sided, int32_t T, int32_t *out, int32_t out_len) {
  if (!d_out || !out || n < 1 || n > kMaxJobs || T < 1 || T > NL_MAX_T || d_in < NL_GROUP || d_in % NL_GROUP ||
      (bits != 0 && bits != 6 && bits != 7 && bits != 8))
    return fail(NL_EINVAL, "describe_call: bad arguments");
  CallShape cs[kMaxJobs];
  for (int i = 0; i < n; ++i) {
    if (d_out[i] < 1) return fail(NL_EINVAL, "describe_call: d_out[%d] < 1", i);
    cs[i] = CallShape{d_out[i], (d_out[i] + kTileRows - 1) / kTileRows, (d_in + kChunk - 1) / kChunk, block_size(d_in),
                      block_size(d_out[i]), two_sided != 0};
  }
  const Plan2 p = make_plan2(cs, n, T, bits);
  int32_t v[8 + 6 * kMaxJobs] = {p.local, p.mt, p.nw, p.n_rot, p.n_con, p.n_fin, (int32_t)p.lds, p.blob};
  for (int i = 0; i < n; ++i) {
    const JobPlan &jp = p.j[i];
    const int32_t jv[6] = {jp.S, jp.cps, jp.rt, jp.kw, jp.n_rb, jp.n_sb};
    memcpy(v + 8 + 6 * i, jv, sizeof jv);
  }
  memcpy(out, v, sizeof(int32_t) * std::min<int>(out_len, 8 + 6 * n));
  return ok();
}

extern "C" nl_status nested_linear_verify_multi(const nl_handle *hs, int32_t n, const void *x, int32_t T,
                                                float *const *ys, void *ws, size_t ws_bytes, void *stream) {
  if (!hs) return fail(NL_EINVAL, "verify_multi: NULL handles");
  return forward_n((const nl_linear *const *)hs, n, 1, x, T, ys, ws, ws_bytes, stream, "verify_multi");
}

extern "C" nl_status nested_linear_draft_multi(const nl_handle *hs, int32_t n, const void *x, int32_t T,
                                               float *const *ys, void *ws, size_t ws_bytes, void *stream) {
  if (!hs) return fail(NL_EINVAL, "draft_multi: NULL handles");
  return forward_n((const nl_linear *const *)hs, n, 0, x, T, ys, ws, ws_bytes, stream, "draft_multi");
}

extern "C" nl_status nested_linear_multi_workspace_bytes(const nl_handle *hs, int32_t n, int32_t T_max,
                                                         size_t *bytes) {
  if (!hs || !bytes || n < 1 || n > kMaxJobs) return fail(NL_EINVAL, "multi_workspace_bytes: bad arguments");
  if (T_max < 1) return fail(NL_EINVAL, "multi_workspace_bytes: T_max must be >= 1");
  if (T_max > NL_MAX_T) return fail(NL_EUNSUPPORTED, "multi_workspace_bytes: T_max > %d", NL_MAX_T);
  for (int i = 0; i < n; ++i) {
    if (!valid(hs[i])) return fail(NL_EINVAL, "multi_workspace_bytes: linear %d is not a valid handle", i);
    if (hs[i]->d_in != hs[0]->d_in) return fail(NL_EINVAL, "multi_workspace_bytes: linear %d differs in d_in", i);
  }
  size_t mx = 0;
  CallShape cs[kMaxJobs];
  for (int i = 0; i < n; ++i) cs[i] = shape_of(hs[i]);
  // the staged grouped form of linears of one shape, at any T (its threshold is a tuning knob)
  bool one_shape = n >= 2 && !hs[0]->has_sign_out;
  for (int i = 1; i < n; ++i)
    one_shape = one_shape && hs[i]->d_out == hs[0]->d_out && hs[i]->b_in == hs[0]->b_in && hs[i]->bits == hs[0]->bits;
  for (int T = 1; T <= T_max; ++T) {
    for (int b = 0; b < 2; ++b) mx = std::max(mx, make_plan2(cs, n, T, b ? hs[0]->bits : 0).total);
    if (one_shape) mx = std::max(mx, multi_plan(hs[0], n, T).total);
  }
  *bytes = mx;
  return ok();
}

extern "C" nl_status nested_linear_workspace_bytes(nl_handle h, int32_t T_max, size_t *bytes) {
  if (!valid(h)) return fail(NL_EINVAL, "workspace_bytes: invalid handle");
  if (!bytes) return fail(NL_EINVAL, "workspace_bytes: NULL bytes");
  if (T_max < 1) return fail(NL_EINVAL, "workspace_bytes: T_max must be >= 1");
  if (T_max > NL_MAX_T) return fail(NL_EUNSUPPORTED, "workspace_bytes: T_max > %d", NL_MAX_T);
  size_t mx = 0;
  const CallShape hs[1] = {shape_of(h)};
  for (int T = 1; T <= T_max; ++T) {
    // the staged calls' layouts (every tile-wave count the staged launch can
    // take, so that a size taken before a tuning change stays valid) and the
    // single launch's, draft and verify
    for (int tw : {tile_waves(mt_for(T)), 4, 8}) {
      if (tw != tile_waves(mt_for(T)) && mt_for(T) > (tw == 8 ? 3 : 2)) continue;
      const Plan p = make_plan(h->d_out, h->n_tiles, h->n_chunks, h->has_sign_out, h->b_out, T, mt_for(T), 1, T, tw,
                               h->b_in);
      mx = std::max(mx, p.total);
    }
    mx = std::max(mx, make_plan2(hs, 1, T, 0).total);
    if (h->bits) mx = std::max(mx, make_plan2(hs, 1, T, h->bits).total);
  }
  *bytes = mx;
  return ok();
}

extern "C" nl_status nested_linear_set_tuning(int32_t knob, double value) {
  switch (knob) {
    case NL_TUNE_SPLITS: g_t_S = (int)value; break;
    case NL_TUNE_ROW_TILES: g_t_rt = (int)value; break;
    case NL_TUNE_WAVES_PER_TILE: g_t_kw = (int)value; break;
    case NL_TUNE_LOCAL_T: g_t_local = (int)value; break;
    case NL_TUNE_CUS: g_t_cus = value >= 1 ? (int)value : 256; break;
    case NL_TUNE_LAT_US: g_t_lat_us = value > 0 ? value : 2.0; break;
    case NL_TUNE_HBM_GBS: g_t_hbm_gbs = value > 0 ? value : 6500.0; break;
    case NL_TUNE_SPLIT_US: g_t_split_us = value >= 0 ? value : 1.5; break;
    case NL_TUNE_XDMA_GBS: g_t_xdma_gbs = value > 0 ? value : 100.0; break;
    case NL_TUNE_SPIN_LIMIT: g_spin_limit = value >= 1 ? (uint32_t)value : (1u << 22); break;
    case NL_TUNE_WAIT_EXTRA: g_wait_extra = value >= 0 ? (uint32_t)value : 0u; break;
    case NL_TUNE_WAVES: g_t_nw = ((int)value == 8 || (int)value == 12) ? (int)value : 0; break;
    case NL_TUNE_STAGED_T_VERIFY: g_t_staged_v = value > 0 ? (int)value : 9; break;
    case NL_TUNE_STAGED_T_DRAFT: g_t_staged_d = value > 0 ? (int)value : 1; break;
    case NL_TUNE_STAGED_WAVES: g_t_stw = ((int)value == 4 || (int)value == 8) ? (int)value : 0; break;
    case NL_TUNE_MULTI_STAGED_T_VERIFY: g_t_ms_v = value > 0 ? (int)value : 33; break;
    case NL_TUNE_MULTI_STAGED_T_DRAFT: g_t_ms_d = value > 0 ? (int)value : 24; break;
    default: return fail(NL_EINVAL, "set_tuning: unknown knob %d", knob);
  }
  return ok();
}

extern "C" nl_status nested_linear_workspace_status(void *ws, uint32_t *errors, int32_t clear, void *stream) {
  if (!ws || !errors) return fail(NL_EINVAL, "workspace_status: NULL workspace or errors");
  if ((uintptr_t)ws & 255) return fail(NL_EINVAL, "workspace_status: workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  HIP_OR_FAIL(hipStreamSynchronize(s));
  HIP_OR_FAIL(hipMemcpy(errors, ws, sizeof(uint32_t), hipMemcpyDeviceToHost));
  if (clear) {
    HIP_OR_FAIL(hipMemsetAsync(ws, 0, kCtrBytes, s));
    HIP_OR_FAIL(hipStreamSynchronize(s));
  }
  return ok();
}

extern "C" nl_status nested_linear_verify(nl_handle h, const void *x, int32_t T, float *y, void *ws,
                                          size_t ws_bytes, void *stream) {
  return forward(h, 1, x, T, y, ws, ws_bytes, stream, "verify");
}

extern "C" nl_status nested_linear_draft(nl_handle h, const void *x, int32_t T, float *y, void *ws,
                                         size_t ws_bytes, void *stream) {
  return forward(h, 0, x, T, y, ws, ws_bytes, stream, "draft");
}

extern "C" nl_status nested_linear_decode(nl_handle h, int32_t row0, int32_t nrows, uint8_t *base_idx,
                                          int8_t *resid, void *stream) {
  if (!valid(h)) return fail(NL_EINVAL, "decode: invalid handle");
  if (!base_idx) return fail(NL_EINVAL, "decode: NULL base_idx");
  if (row0 < 0 || nrows < 1 || row0 + nrows > h->d_out)
    return fail(NL_EINVAL, "decode: rows [%d, %d) outside [0, %d)", row0, row0 + nrows, h->d_out);
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.lin = h->dev;
  a.base_idx = base_idx;
  a.resid = h->bits ? resid : nullptr;
  a.d_in = h->d_in;
  a.n_chunks = h->n_chunks;
  a.row0 = row0;
  a.nrows = nrows;
  a.tile0 = row0 / kTileRows;
  const int tile1 = (row0 + nrows - 1) / kTileRows;
  HIP_OR_FAIL(launch_decode(a, h->bits, tile1 - a.tile0 + 1, (hipStream_t)stream));
  return ok();
}

// ---------------------------------------------------------------------------
// Grouped (mixture-of-experts) calls.
// ---------------------------------------------------------------------------
extern "C" nl_status nested_linear_group_create(const nl_handle *experts, int32_t n,
                                                nl_group_handle *out) {
  if (!experts || !out || n < 1) return fail(NL_EINVAL, "group_create: bad arguments");
  for (int i = 0; i < n; ++i)
    if (!valid(experts[i])) return fail(NL_EINVAL, "group_create: expert %d is not a valid handle", i);
  const nl_linear *e0 = experts[0];
  for (int i = 1; i < n; ++i) {
    const nl_linear *e = experts[i];
    if (e->d_out != e0->d_out || e->d_in != e0->d_in || e->bits != e0->bits ||
        e->has_sign_out != e0->has_sign_out)
      return fail(NL_EINVAL, "group_create: expert %d differs in shape, bits or sign_out", i);
  }
  std::vector<LinearDev> devs(n);
  for (int i = 0; i < n; ++i) devs[i] = experts[i]->dev;
  nl_group *g = new (std::nothrow) nl_group();
  if (!g) return fail(NL_ENOMEM, "group_create: host allocation failed");
  hipError_t e = hipMalloc(&g->dev_array, sizeof(LinearDev) * n);
  if (e != hipSuccess) {
    delete g;
    (void)hipGetLastError();
    return fail(NL_ENOMEM, "group_create: hipMalloc failed: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(g->dev_array, devs.data(), sizeof(LinearDev) * n, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(g->dev_array);
    delete g;
    return fail(NL_EHIP, "group_create: copy failed: %s", hipGetErrorString(e));
  }
  g->n = n;
  g->d_out = e0->d_out;
  g->d_in = e0->d_in;
  g->bits = e0->bits;
  g->n_tiles = e0->n_tiles;
  g->n_chunks = e0->n_chunks;
  g->b_in = e0->b_in;
  g->b_out = e0->b_out;
  g->has_sign_out = e0->has_sign_out;
  g->magic = kGroupMagic;
  live_add(g);
  *out = g;
  return ok();
}

extern "C" nl_status nested_linear_group_destroy(nl_group_handle g) {
  if (!valid(g)) return fail(NL_EINVAL, "group_destroy: invalid handle");
  live_del(g);
  g->magic = 0;
  hipError_t e = hipFree(g->dev_array);
  delete g;
  if (e != hipSuccess) return fail(NL_EHIP, "group_destroy: hipFree failed: %s", hipGetErrorString(e));
  return ok();
}

static Plan group_plan(nl_group_handle g, int P, int T) {
  // short experts (K of at most two chunks): eight tile waves, half the
  // workgroups; longer ones keep the deeper register ring of four
  const int tw = T > kLocalTokens && g->n_chunks <= 2 && mt_for(T) < 4 ? 8 : tile_waves(mt_for(T));
  return make_plan(g->d_out, g->n_tiles, g->n_chunks, g->has_sign_out, g->b_out, P, mt_for(T), g->n, T, tw,
                   g->b_in);
}

extern "C" nl_status nested_linear_group_workspace_bytes(nl_group_handle g, int32_t P_max,
                                                         size_t *bytes) {
  if (!valid(g)) return fail(NL_EINVAL, "group_workspace_bytes: invalid handle");
  if (!bytes || P_max < 1) return fail(NL_EINVAL, "group_workspace_bytes: bad arguments");
  // the two tile-wave counts give different split counts: the larger plan
  const size_t a = group_plan(g, P_max, 1).total, b = group_plan(g, P_max, NL_MAX_T).total;
  *bytes = a > b ? a : b;
  return ok();
}

static nl_status grouped(nl_group_handle g, int verify, const int32_t *pair_token,
                         const int32_t *offsets, int32_t P, const void *x, int32_t x_rows, int32_t T, float *y,
                         void *ws, size_t ws_bytes, void *stream, const char *who) {
  if (!valid(g)) return fail(NL_EINVAL, "%s: invalid handle", who);
  if (verify && !g->bits) return fail(NL_EINVAL, "%s: the experts have no residual", who);
  if (!pair_token || !offsets || !x || !y || !ws) return fail(NL_EINVAL, "%s: NULL pointer", who);
  if ((uintptr_t)x & 15) return fail(NL_EINVAL, "%s: x must be 16-byte aligned", who);
  if (P < 1 || T < 1 || x_rows < 1) return fail(NL_EINVAL, "%s: P, x_rows and T must be >= 1", who);
  if (T > NL_MAX_T) return fail(NL_EUNSUPPORTED, "%s: T = %d exceeds %d", who, T, NL_MAX_T);
  if ((uintptr_t)ws & 255) return fail(NL_EINVAL, "%s: workspace must be 256-byte aligned", who);
  Plan p = group_plan(g, P, T);
  if (ws_bytes < p.total) return fail(NL_EINVAL, "%s: workspace too small (%zu < %zu)", who, ws_bytes, p.total);
  if (p.n_ctr > kCtrLines)
    return fail(NL_EUNSUPPORTED, "%s: %d experts of d_out = %d need %d counters (> %d)", who, g->n, g->d_out,
                p.n_ctr, kCtrLines);
  char *w = (char *)ws;
  FwdArgs f;
  memset(&f, 0, sizeof f);
  RotInArgs &r = f.rot;
  r.x = (const uint16_t *)x;
  r.lins = g->dev_array;
  r.pair_token = pair_token;
  r.offsets = offsets;
  r.n_experts = g->n;
  r.x_rows = x_rows;
  r.rows = P;
  r.lb = log2i(g->b_in);
  r.xh = (uint16_t *)(w + p.o_xh);
  r.meta = (float *)(w + p.o_meta);
  r.d_in = g->d_in;
  r.b = g->b_in;
  r.SB = g->b_in > kChunk ? g->b_in : kChunk;
  r.Kp = g->n_chunks * kChunk;
  r.Gp = g->n_chunks * 4;
  r.n_chunks = g->n_chunks;
  r.rsqrt_b = (float)(1.0 / std::sqrt((double)g->b_in));

  GemmArgs &ga = f.g;
  ga.lins = g->dev_array;
  ga.offsets = offsets;
  ga.xh = (const uint16_t *)(w + p.o_xh);
  ga.meta = (const float *)(w + p.o_meta);
  ga.T = P;
  ga.d_out = g->d_out;
  ga.n_tiles = g->n_tiles;
  ga.n_chunks = g->n_chunks;
  ga.Kp = r.Kp;
  ga.Gp = r.Gp;
  ga.cps = p.cps;
  ga.ldo = g->d_out;
  ga.n_rb = p.n_rb;
  ga.n_experts = g->n;

  FinishArgs &fa = f.fin;
  fa.lins = g->has_sign_out ? g->dev_array : nullptr;
  fa.offsets = offsets;
  fa.n_experts = g->n;
  fa.b = g->b_out;
  fa.lb = log2i(g->b_out);
  fa.rsqrt_b = (float)(1.0 / std::sqrt((double)g->b_out));
  fill_launch(f, p, g->n, w, y, g->d_out);
  const int n_fin = p.mode == kOutTwoSided ? finish_workgroups(P, g->d_out, p.sb_rows) : 0;
  hipEvent_t e0, e1;
  timing_slot((hipStream_t)stream, &e0, &e1);
  HIP_OR_FAIL(launch_forward(f, verify ? g->bits : 0, p.mt, p.tw, n_fin, (hipStream_t)stream, e0, e1));
  return ok();
}

extern "C" nl_status nested_linear_verify_grouped(nl_group_handle g, const int32_t *pair_token,
                                                  const int32_t *offsets, int32_t P, const void *x,
                                                  int32_t x_rows, int32_t T, float *y, void *ws,
                                                  size_t ws_bytes, void *stream) {
  return grouped(g, 1, pair_token, offsets, P, x, x_rows, T, y, ws, ws_bytes, stream, "verify_grouped");
}

extern "C" nl_status nested_linear_draft_grouped(nl_group_handle g, const int32_t *pair_token,
                                                 const int32_t *offsets, int32_t P, const void *x,
                                                 int32_t x_rows, int32_t T, float *y, void *ws,
                                                 size_t ws_bytes, void *stream) {
  return grouped(g, 0, pair_token, offsets, P, x, x_rows, T, y, ws, ws_bytes, stream, "draft_grouped");
}
