// nl_layout.h -- internal packed layout of a nested linear on gfx950 and the
// device routines that unpack it into MFMA operands.
//
// Work unit: a "tile-chunk" = 16 output rows x 512 input columns (4 scale
// groups of 128).  One wave64 contracts a tile-chunk with
// v_mfma_f32_16x16x32_f16: the weights are the B operand (N = 16 rows), the
// activations the A operand (M = 16 tokens).  Lane l owns row (l & 15) and
// the 32 consecutive columns [32*(l >> 4), +32) of every group; MFMA step s
// (0..3) of a group feeds the lane's columns 8s..8s+7, which matches the A
// operand lane that reads x'[token][32*(l >> 4) + 8s .. +8] from LDS.  Within
// a group the contraction order is therefore a fixed permutation of k, the
// same on both operands.
//
// Every lane's bytes of a tile-chunk are split into 16-byte pieces; piece i of
// all 64 lanes is one contiguous 1 KiB run, so each global_load_dwordx4 of a
// wave reads 1 KiB of consecutive memory.
//   base   2 pieces / lane  (2048 B per tile-chunk, 2 bits per weight)
//   resid  b pieces / lane  (1024*b B per tile-chunk, b bits per weight)
//   scales [16 rows][4 groups] fp16 per tile-chunk and per kind (128 B)
// Tile-chunks are stored tile-major, chunk-minor, so a wave streaming one row
// tile over K reads one contiguous range per plane.
//
// Per lane and group the 32 codes of each plane become 16 "pairs": pair P is
// the lane's columns (2P, 2P+1), packed as one fp16x2 dword of the B operand
// (MFMA step P >> 2, dword P & 3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nl {

constexpr int kGroup = 128;
constexpr int kChunkGroups = 4;
constexpr int kChunk = kGroup * kChunkGroups;  // 512 columns
constexpr int kTileRows = 16;
constexpr int kBasePieces = 2;
constexpr int kBaseBlockBytes = 64 * 16 * kBasePieces;   // 2048
constexpr int kScaleBlockBytes = kTileRows * kChunkGroups * 2;  // 128

__host__ __device__ constexpr int resid_block_bytes(int bits) { return 64 * 16 * bits; }


// Device-side description of one linear (also an element of a grouped
// launch's expert array).
struct LinearDev {
  const uint4 *base;        // [n_tiles][n_chunks][2][64] uint4
  const uint4 *resid;       // [n_tiles][n_chunks][bits][64] uint4 (or null)
  const uint2 *bscale;      // [n_tiles][n_chunks][16] (4 x fp16 each)
  const uint2 *rscale;      // [n_tiles][n_chunks][16]
  const int8_t *sign_in;    // [d_in]
  const int8_t *sign_out;   // [d_out] or null
  uint32_t lut[16];         // fp16x2 {kappa*L[i & 3], kappa*L[i >> 2]}
  float kinv;               // 1 / kappa
  int32_t pad_;
  const uint2 *lut256;      // [256] byte-indexed base table (two fp16x2 per byte of codes)
};
static_assert(sizeof(LinearDev) == 128, "descriptor size");

// ---------------------------------------------------------------------------
// Residual unpack: the lane's `bits` dwords of one group -> 16 fp16x2 pairs,
// each half = 1024 + u.  The packings were chosen so that most pairs cost one
// v_and_or_b32 (6/7-bit) or one v_perm_b32 (8-bit); they are produced by the
// repack kernel and inverted by the decode kernel through these same routines.
//
// 8-bit: dword w holds columns 4w..4w+3 as bytes.
// 6-bit: dword d (0..5) holds pair d in bits [0,6) / [16,22) and pair 6+d in
//   bits [6,12) / [22,28); the spare nibbles [12,16) / [28,32) of dwords 0..3
//   hold the low 4 bits of pairs 12..15, and those of dwords 4 (pairs 12, 13)
//   and 5 (pairs 14, 15) hold their top 2 bits, two bits per pair.
// 7-bit: dword d (0..6) holds pair d in bits [0,7) / [16,23) and pair 7+d in
//   [7,14) / [23,30); the 2-bit spares [14,16) / [30,32) of the seven dwords
//   hold pairs 14 (bits 0-1 in dword 0, 2-3 in 1, 4-5 in 2, 6 in dword 3 bit
//   14) and 15 (bit 0 in dword 3 bit 15, 1-2 in 4, 3-4 in 5, 5-6 in 6).
// ---------------------------------------------------------------------------
// A constant the optimiser cannot fold into literals: materialised once in an
// SGPR, so (a & m) | o selects a single v_and_or_b32 (GFX9 VOP3 encodings
// take no literal operands) while the compiler still schedules the VALU work
// and its MFMA hazards itself.
__device__ __forceinline__ uint32_t sconst(uint32_t c) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(c));
  return r;
}

// The or-constant of and_or lives in a VGPR (one SGPR read per VOP3).  Only
// VALU instructions read it, so the asm's VGPR write needs no MFMA hazard
// handling.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return (a & sconst(m)) | o;
}

// SUB: the halves are the fp16 subnormals u * 2^-24 instead (exact; no
// exponent bits are set), for a contraction that removes the smaller offset
// 2^(b-1) * 2^-24 with the activations' group sums.
template <int BITS, bool SUB = false>
__device__ __forceinline__ void unpack_resid(const uint32_t *d, uint32_t *out) {
  const uint32_t K = SUB ? 0u : vconst(0x64006400u);
  if constexpr (BITS == 8) {
    const uint32_t K8 = SUB ? 0u : 0x64646464u;
#pragma unroll
    for (int P = 0; P < 16; ++P)
      out[P] = SUB ? __builtin_amdgcn_perm(0u, d[P >> 1], (P & 1) ? 0x0c030c02u : 0x0c010c00u)
                   : __builtin_amdgcn_perm(K8, d[P >> 1], (P & 1) ? 0x04030402u : 0x04010400u);
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int P = 0; P < 6; ++P) out[P] = and_or(d[P], 0x003F003Fu, K);
#pragma unroll
    for (int P = 0; P < 6; ++P) out[6 + P] = and_or(d[P] >> 6, 0x003F003Fu, K);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[12 + j] = and_or(d[j] >> 12, 0x000F000Fu,
                           and_or(d[4 + (j >> 1)] >> (8 + 2 * (j & 1)), 0x00300030u, K));
  } else if constexpr (BITS == 7) {
#pragma unroll
    for (int P = 0; P < 7; ++P) out[P] = and_or(d[P], 0x007F007Fu, K);
#pragma unroll
    for (int P = 0; P < 7; ++P) out[7 + P] = and_or(d[P] >> 7, 0x007F007Fu, K);
    out[14] = and_or(d[3] >> 8, 0x00400040u,
                     and_or(d[2] >> 10, 0x00300030u,
                            and_or(d[1] >> 12, 0x000C000Cu, and_or(d[0] >> 14, 0x00030003u, K))));
    out[15] = and_or(d[6] >> 9, 0x00600060u,
                     and_or(d[5] >> 11, 0x00180018u,
                            and_or(d[4] >> 13, 0x00060006u, and_or(d[3] >> 15, 0x00010001u, K))));
  }
}

// Inverse of unpack_resid: 32 unsigned values (u < 2^BITS) of one lane-group
// -> BITS dwords.  Used only by the create-time repack.
template <int BITS>
__device__ __forceinline__ void pack_resid(const uint32_t *v, uint32_t *d) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) d[i] = 0;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int w = 0; w < 8; ++w)
      d[w] = v[4 * w] | (v[4 * w + 1] << 8) | (v[4 * w + 2] << 16) | (v[4 * w + 3] << 24);
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int P = 0; P < 6; ++P) d[P] |= v[2 * P] | (v[2 * P + 1] << 16);
#pragma unroll
    for (int P = 0; P < 6; ++P) d[P] |= (v[2 * (6 + P)] << 6) | (v[2 * (6 + P) + 1] << 22);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = v[2 * (12 + j)], hi = v[2 * (12 + j) + 1];
      d[j] |= ((lo & 15u) << 12) | ((hi & 15u) << 28);
      int sh = 2 * (j & 1);
      d[4 + (j >> 1)] |= ((lo >> 4) << (12 + sh)) | ((hi >> 4) << (28 + sh));
    }
  } else if constexpr (BITS == 7) {
#pragma unroll
    for (int P = 0; P < 7; ++P) d[P] |= v[2 * P] | (v[2 * P + 1] << 16);
#pragma unroll
    for (int P = 0; P < 7; ++P) d[P] |= (v[2 * (7 + P)] << 7) | (v[2 * (7 + P) + 1] << 23);
    {  // pair 14: columns 28 (low half) and 29 (high half)
      uint32_t lo = v[28], hi = v[29];
      d[0] |= ((lo & 3u) << 14) | ((hi & 3u) << 30);
      d[1] |= (((lo >> 2) & 3u) << 14) | (((hi >> 2) & 3u) << 30);
      d[2] |= (((lo >> 4) & 3u) << 14) | (((hi >> 4) & 3u) << 30);
      d[3] |= (((lo >> 6) & 1u) << 14) | (((hi >> 6) & 1u) << 30);
    }
    {  // pair 15: columns 30 and 31
      uint32_t lo = v[30], hi = v[31];
      d[3] |= ((lo & 1u) << 15) | ((hi & 1u) << 31);
      d[4] |= (((lo >> 1) & 3u) << 14) | (((hi >> 1) & 3u) << 30);
      d[5] |= (((lo >> 3) & 3u) << 14) | (((hi >> 3) & 3u) << 30);
      d[6] |= (((lo >> 5) & 3u) << 14) | (((hi >> 5) & 3u) << 30);
    }
  }
}

// ---------------------------------------------------------------------------
// Base unpack: the lane's 2 dwords of one group (code j of the lane's 32 at
// bits 2*(j & 15) of dword j >> 4) -> 16 fp16x2 pairs.  Each byte of the
// codes (4 codes = 2 pairs) indexes a 256-entry LDS table of two fp16x2
// dwords, so one ds_read_b64 yields two B-operand dwords.  The table holds
// the levels scaled by a per-linear constant kappa chosen so that fp16
// represents them (nearly) exactly; 1/kappa is folded into the base scale.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack_base(const uint32_t *b, const uint2 *lut_lds, uint32_t *out) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint2 e = lut_lds[(b[w] >> (8 * q)) & 0xFFu];
      out[8 * w + 2 * q] = e.x;
      out[8 * w + 2 * q + 1] = e.y;
    }
  }
}

// Entry i of the byte-indexed table from the 16-entry pair table.
__device__ __forceinline__ uint2 base_table_entry(const uint32_t *lut16, int i) {
  return make_uint2(lut16[i & 15], lut16[i >> 4]);
}

}  // namespace nl
