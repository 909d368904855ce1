/*
 * nested_w4w8.h -- C ABI of the BitNest W4/W8 dual-plane linear on MI355X
 * (gfx950), in the same library as nested_linear.h.
 *
 * Source: "BitNest: Bit-Nested Speculative Decoding for Memory-Efficient LLM
 * Inference Acceleration" (page 2 of the source pages).  A W4 base q4 in
 * [-8, 7] with one scale s4 per 128-weight group (section 3.2, appendix A.1
 * eq. 5-6) and a 4-bit refinement q_r read with s_ref = s4 / 16 (eq. 8-10),
 * stored as two separate planes of N/2 bytes (section 3.3, "Dual-Plane
 * Weight Storage"):
 *
 *     draft:   y = W_draft  x,  W_draft  = q4 s4
 *     verify:  y = W_target x,  W_target = (16 q4 + q_r) s4 / 16
 *
 * for a batch of T draft-tree tokens x[t] (bf16).  The rotations the paper
 * folds into the weights are part of them: there is no online transform.
 * The draft reads only the base plane and the scales.
 *
 * Conventions as in nested_linear.h (nl_status results, the message from
 * nested_linear_last_error(), device pointers unless marked "host",
 * asynchronous calls on the given hipStream_t).
 */
#ifndef NESTED_W4W8_H
#define NESTED_W4W8_H

#include "nested_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nl_w4w8 *nl_w4w8_handle;   /* one W4/W8 linear, opaque */

/*
 * Canonical arrays (G = d_in / 128):
 *   base_plane [d_out][d_in/2] bytes: two's-complement q4 nibbles, weight k
 *              of a row in byte k/2, the low nibble for even k;
 *   ref_plane  [d_out][d_in/2] bytes: q_r in the same layout, or NULL for a
 *              draft-only linear.  Composites 16 q4 + q_r must lie in
 *              [-128, 127] (the eq. 9 boundary rule: q_r >= 0 where q4 = -8);
 *              they are not checked;
 *   scales     [d_out][G] fp16 bit patterns (s4).
 */
typedef struct {
  int32_t d_out;               /* >= 1 */
  int32_t d_in;                /* >= 128 and a multiple of 128 */
  const uint8_t *base_plane;
  const uint8_t *ref_plane;    /* may be NULL */
  const uint16_t *scales;
} nl_w4w8_desc;

/*
 * Copy the arrays into library-owned device memory, repacked tile-major
 * (16 rows x one 128-column group per 1 KiB block, rows padded to a multiple
 * of 128 with zeros) so the kernels stream contiguous memory.  The caller
 * may free its arrays when this returns.  Synchronises the device.  Errors: NL_EINVAL (shape, NULL pointer),
 * NL_ENOMEM, NL_EHIP.  *out is set only on success.
 */
nl_status nested_w4w8_create(const nl_w4w8_desc *desc, nl_w4w8_handle *out);

/* Free a linear.  The caller ensures no call on it is still running. */
nl_status nested_w4w8_destroy(nl_w4w8_handle h);

/*
 * Workspace bytes for calls with up to T_max tokens (host *bytes).  The
 * workspace is caller-owned, 256-byte aligned, zero-filled once before its
 * first use (its first words are the split-K tickets; every call leaves them
 * at zero), and not shared by calls that may overlap.
 */
nl_status nested_w4w8_workspace_bytes(nl_w4w8_handle h, int32_t T_max, size_t *bytes);

/*
 * Verify forward y = W_target x (eq. 10) and draft forward y = W_draft x
 * (eq. 6).  x [T][d_in] bf16 bit patterns, 16-byte aligned; y [T][d_out]
 * fp32 (must not overlap x or ws).  One kernel launch per call.  Where K is
 * split across workgroups, the workgroup of a row block that finishes last
 * sums the split-K partials in split order; for small T * d_in the waves of
 * one workgroup split K and add their sums in wave order.  Either way
 * results do not depend on timing.
 * Errors: NL_EINVAL (NULL pointer, T < 1, misaligned x, small or misaligned
 * ws, verify on a draft-only linear), NL_EUNSUPPORTED (T > 64), NL_EHIP.
 */
nl_status nested_w4w8_verify(nl_w4w8_handle h, const void *x_bf16, int32_t T, float *y, void *ws,
                             size_t ws_bytes, void *hip_stream);
nl_status nested_w4w8_draft(nl_w4w8_handle h, const void *x_bf16, int32_t T, float *y, void *ws,
                            size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NESTED_W4W8_H */
