// nl_fwd.h -- argument block and launcher of the single-launch forward of one
// or more nested linears that read the same activations (draft and verify).
//
// One launch per call.  Its workgroups take one of three roles by index:
//   [0, n_rot)                rotation: x' = H_i S_i x of every linear, one
//                             (linear, token, superblock) task per 256 threads,
//                             stored as fp16 "blobs" (below) with agent-scope
//                             stores, then counted on 8 ready lines;
//   [n_rot, n_rot + n_con)    contraction: a panel of rt row tiles (16 rows
//                             each) x one K-range (split) of a linear.  Its
//                             waves issue their first weight loads, wait for
//                             the ready line, copy the K-range's blobs into
//                             LDS, then stream and contract their own chunks
//                             with no further barrier; kw waves share a row
//                             tile and add their sums in LDS at the end;
//   [n_rot + n_con, ...)      finish (two-sided form): y = S_o H_o y~.
// With few tokens (local form) each contraction workgroup rotates its own
// K-range of x into LDS and there are no rotation workgroups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nl_layout.h"

namespace nl {

constexpr int kMaxJobs = 4;  // linears of one call

// x' of one 512-column chunk for T token rows (a "blob"):
//   activations [group 4][step 4][quarter 4][T][8] fp16: the MFMA A operand
//               of (group, step) for the lanes of quarter q is the 8 columns
//               128 g + 32 q + 8 s .. + 8 of token t (T KiB in all);
//   sums        [4][tm] fp32, tm = T rounded up to 4: per group and token the
//               sum of the group's fp16 activations (they remove the residual
//               operands' offset);
//   scale       [tm] fp32: 2^-e / sqrt(b) per token, where 2^e scaled the
//               chunk's largest magnitude into [2^14, 2^15) before the fp16
//               rounding.
__host__ __device__ constexpr int blob_tm(int T) { return (T + 3) & ~3; }
__host__ __device__ constexpr int blob_bytes(int T) { return T * 1024 + 20 * blob_tm(T); }

// LDS layout of a workgroup (bytes): byte table, flag word, then the blobs of
// the K-range (contraction) and the transform areas (rotation / local form).
constexpr int kLdsLut = 0;
constexpr int kLdsFlag = 2048;
constexpr int kLdsX = 2304;
constexpr int kFwhtArea = (4096 + 256) * 4;  // one 256-thread transform area

struct FwdJob {
  LinearDev lin;      // weights, signs, byte table (read with scalar loads)
  float *y;           // [T][d_out] output
  float *part;        // [S][T][d_out] split partials (S > 1)
  float *ysum;        // [T][d_out] sums before the output rotation (two-sided)
  int xb;             // byte offset of the job's blobs [n_chunks][blob] in the workspace
  int d_out, n_tiles;
  int rt, kw;         // row tiles per workgroup, waves per row tile
  int n_rb, S, cps;   // row blocks, splits of K, chunks per split
  int con0;           // first contraction workgroup of the job (among contraction workgroups)
  int ctr_split;      // counter of the job's first row block (split arrivals)
  int ctr_sb;         // two-sided: first superblock arrival counter, then n_sb token counters
  int n_sb;           // two-sided: output superblocks
  int fin0;           // two-sided: first finish task of the job
  int pad_[3];
};

struct FwdArgs2 {
  const uint16_t *x;  // [T][d_in] bf16
  char *ws;           // workspace: counters from byte 0, blobs at FwdJob::xb
  int T, d_in, n_chunks, Kp;
  int lb_in, SB;      // log2 of the input block, superblock = max(block, 512)
  float rsqrt_in;     // 1 / sqrt(input block)
  int lb_out, OB;     // two-sided: log2 of the output block, rows per finish task
  float rsqrt_out;
  int blob, tm;
  int n_jobs, n_rot, n_con, n_fin;
  int rot_groups;     // 256-thread transform groups used per rotation workgroup
  uint32_t spin_limit;  // polls before a wait gives up
  uint32_t wait_extra;  // added to every wait target (> 0: the waits give up; a test hook)
  FwdJob job[kMaxJobs];
};

// Waves per workgroup of the contraction by 16-token tiles: twelve (three per
// SIMD, at most 168 registers each) up to two tiles, eight beyond; one token
// tile also has an eight-wave form with a deeper ring.
__host__ __device__ constexpr int fwd_waves(int mt) { return mt <= 2 ? 12 : 8; }

// Register sets in a wave's weight ring (within 168 registers for twelve
// waves, 256 for eight; verify at three or four token tiles keeps one, its
// registers going to the next tile's activations).  In the local form the
// waves that rotate x request their sets only after the transform, so no
// wave holds both.
__host__ __device__ constexpr int fwd_ring_sets(int bits, int mt, bool local, int nw) {
  return (void)local, nw == 8 && mt == 1 ? 4 : (mt == 1 ? (bits == 0 ? 4 : 2) : (bits == 0 ? 3 : (mt >= 3 ? 1 : 2)));
}

hipError_t launch_forward2(const FwdArgs2 &a, int bits, int mt, int nw, bool local, size_t lds, hipStream_t s,
                           hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

}  // namespace nl
