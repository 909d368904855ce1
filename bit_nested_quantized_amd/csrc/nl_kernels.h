// nl_kernels.h -- argument blocks and host launchers of the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nl_layout.h"

namespace nl {

struct RepackArgs {
  const uint8_t *base_codes;
  const uint16_t *base_scales;
  const uint8_t *resid_codes;
  const uint16_t *resid_scales;
  uint4 *base;
  uint4 *resid;
  uint16_t *bscale;
  uint16_t *rscale;
  int d_out, d_in, G, n_tiles, n_chunks;
};

struct DecodeArgs {
  LinearDev lin;
  uint8_t *base_idx;
  int8_t *resid;
  int d_in, n_chunks, row0, nrows, tile0;
};

// Input rotation.  Grid (tokens, superblocks of SB columns); for a grouped
// call token t of the grid is pair t, its activation row is pair_token[t]
// and its signs those of its expert.
struct RotInArgs {
  const uint16_t *x;        // [T][d_in] bf16
  const int8_t *sign;       // [d_in] (single linear)
  const LinearDev *lins;    // expert array (grouped) or null
  const int32_t *pair_token;
  const int32_t *offsets;
  int n_experts;
  int x_rows;               // rows of x (bounds for pair_token)
  uint16_t *xh;             // fp16 in the contraction's run layout (see xa_index)
  float *meta;              // [n_chunks][5][rows]: 4 group sums of xh, then 2^-s / sqrt(b)
  int rows;                 // rows of x' (tokens, or pairs of a grouped call)
  int d_in, b, lb, SB, Kp, Gp, n_chunks;
  float rsqrt_b;
  int groups;               // 256-thread transform groups per workgroup (0 or 1: one)
};

struct GemmArgs {
  LinearDev lin;            // single linear
  const LinearDev *lins;    // expert array (grouped) or null
  const int32_t *offsets;   // grouped: [n_experts + 1]
  const uint16_t *xh;
  const float *meta;
  float *out;               // [split][rows][ldo]
  size_t split_stride;
  int T;                    // rows of x' (tokens or pairs)
  int d_out, n_tiles, n_chunks, Kp, Gp, cps, ldo, n_rb, n_experts;
  int slots;                // grouped: grid slots map to the experts with rows (else slot = expert)
  float *ys[4];             // one-sided multi-linear form (experts = linears of one x, all rows of
                            // each): expert e's row t goes to row t of ys[e]; else null
};

struct FinishArgs {
  const float *part;        // [S][rows][d_out]
  size_t split_stride;
  float *y;                 // [rows][d_out]
  const int8_t *sign_out;   // single linear (or null)
  const LinearDev *lins;    // grouped: per-pair expert sign_out
  const int32_t *offsets;
  int n_experts;
  int T, d_out, S, b, lb, OB;   // OB = 256*E rows per workgroup
  float rsqrt_b;
};

// Counters of the single-launch forward: 32-bit words, one per 64-byte
// line, in a region of fixed size at the start of every workspace (so calls
// of any shape can share a workspace).  Fixed slots, then per linear the
// row-block arrival counters (split-K) and per output superblock the arrival
// counters and finish tokens (two-sided form).  Every rotation workgroup adds
// one to each of the 8 ready lines once its x' is stored; a contraction
// workgroup that has rows to compute polls one line until it reads n_rot,
// and counts itself on that line's exit counter when done.  The line's
// target (active linears x its workgroups per linear) is published by the
// first rotation workgroup; the last exit clears the line's three words.
constexpr int kCtrStride = 16;  // words
constexpr int kCtrLines = 16384;
constexpr size_t kCtrBytes = (size_t)kCtrLines * kCtrStride * 4;  // 1 MiB
enum : int {
  kCtrErr = 0,       // waits that hit the spin limit (diagnostic; stays zero)
  kCtrReady = 1,     // 8 ready lines: rotation workgroups done
  kCtrExit = 9,      // 8 lines: waiting contraction workgroups done
  kCtrActive = 17,   // 8 lines: linears with rows (1, or the active experts)
  kCtrFixed = 25,
};
constexpr uint32_t kSpinLimit = 1u << 22;  // default of Handover::spin_limit

enum : int { kOutDirect = 0, kOutSplit = 1, kOutTwoSided = 2 };

// Calls with at most kLocalTokens rows per linear and at most kLocalChunks
// chunks per split rotate x inside each contraction workgroup (no rotation
// workgroups, no hand-over); they launch with MT = 0.  (Each extra row costs
// the workgroup one more 4096-point transform pass, so the limit is small.)
constexpr int kLocalRows = 4;   // rows of the resident x' layout (>= kLocalTokens)
constexpr int kLocalTokens = 2;
constexpr int kLocalChunks = 8;

// What a contraction workgroup of the single launch does with its result.
struct Handover {
  uint32_t *ctr;
  float *y;           // [rows][d_out] output
  float *ysum;        // two-sided: [rows][d_out] split sums before H_o
  int mode;           // kOutDirect, kOutSplit or kOutTwoSided
  int S;              // splits
  int sb_rows;        // rows per output superblock (two-sided)
  int n_sb;           // output superblocks per linear
  int rb_base, ob_base, obr_base;  // first counter of each kind
  int line;           // ready line of the workgroup (set per workgroup)
  int n_rot;          // rotation workgroups of the launch
  uint32_t spin_limit;  // polls before a wait gives up
  uint32_t wait_extra;  // added to every wait target (> 0: the waits give up; a test hook)
};

struct FwdArgs {
  RotInArgs rot;
  GemmArgs g;         // g.out = y (direct) or the split partials
  FinishArgs fin;
  Handover hv;
  int n_rot, n_gemm;
};

// Tile waves (16 output rows each) of a contraction workgroup, plus one x'
// loader wave: eight for three or more 16-token tiles, whose chunks are long
// enough that two tile waves per SIMD pay, else four.  Grouped calls (more
// than kLocalTokens tokens) whose experts span at most two chunks of K take
// eight at any tile count: their workgroups are short, and half as many of
// them pay more than the register ring they give up.
// Tile waves per workgroup of the staged kernels by token tiles: four up to
// two tiles; eight for three (168 registers each); seven for four, whose
// accumulators and unpacked operands need the 256 registers of an
// eight-wave workgroup.
constexpr int tile_waves(int mt) { return mt >= 4 ? 7 : (mt == 3 ? 8 : 4); }
constexpr int wg_threads(int mt) { return 64 * (tile_waves(mt) + 1); }

int rotate_workgroups(int rows, int Kp, int SB, int groups = 1);
int finish_workgroups(int rows, int d_out, int OB);

hipError_t launch_repack(const RepackArgs &a, int bits, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int bits, int ntiles, hipStream_t s);
hipError_t launch_rotate_in(const RotInArgs &a, int rows, hipStream_t s);
hipError_t launch_gemm(const GemmArgs &a, int bits, int mt, int splits, hipStream_t s);
hipError_t launch_finish(const FinishArgs &a, hipStream_t s);
// Streaming-read reference (nl_stream.hip): reads bytes (a multiple of 16)
// from src once; sink holds one word per workgroup of the grid.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int grid, hipStream_t s);
// ev0/ev1 (optional): events that record the kernel's own start and end
// (attached to the dispatch, not queued beside it).
hipError_t launch_forward(const FwdArgs &f, int bits, int mt, int tw, int n_fin, hipStream_t s,
                          hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

}  // namespace nl
