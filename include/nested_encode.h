/*
 * nested_encode.h -- C ABI of the round-to-nearest encoder that produces the
 * canonical planes of a bit-nested linear (include/nested_linear.h) from a
 * dense weight matrix, and of the Lloyd-Max fitter of its four base levels.
 *
 * Source: the forum post "bit-nested" (page 1 of the source pages), POC
 * recipe:
 *   section 1  W~ = H_o S_o W S_i H_i, H the normalised Sylvester-Hadamard
 *              matrix applied block-diagonally (block = largest power of two
 *              dividing the dimension, at most 4096);
 *   section 2  base scale per (row, 128-group) = RMS of the block rounded to
 *              fp16; code = nearest of the 4 levels times that scale; the
 *              levels are fitted on RMS-normalised rotated weights from the
 *              quantiles 0.125/0.375/0.625/0.875 by Lloyd iterations (60 in
 *              the post) and then symmetrised;
 *   section 3  residual R~ = W~ - Q_base quantised uniformly to b bits,
 *              integers -qm..qm (qm = 2^(b-1) - 1), scale = max|block|/qm
 *              in fp16.
 * The post's GPTQ/LDLQ variant needs calibration activations; this is the
 * plain round-to-nearest quantiser.
 *
 * Arithmetic (the same on every call and GPU): the rotation runs in fp64,
 * butterflies over strides 1, 2, 4, ... and then a multiplication of each
 * block by 1/sqrt(b), the input side before the output side.  Scales are
 * rounded from fp64 straight to fp16 (nearest, ties to even; beyond 65504
 * they saturate to 65504).  A weight goes to the nearest reconstruction point
 * levels[c] * scale, decided exactly (midpoints between points are exact in
 * fp64); a weight on a midpoint takes the level of smaller magnitude, and of
 * two equal magnitudes the larger level; with a zero scale that same rule
 * picks the code.  Residual integers are round-half-even of R~/scale clamped
 * to [-qm, qm], and 0 where the residual scale is 0.
 *
 * Conventions as in nested_linear.h: every call returns an nl_status and
 * never aborts; nested_linear_last_error() has the message; pointers are
 * device pointers unless marked "host"; calls are asynchronous on the given
 * hipStream_t (void*, NULL = null stream) except where stated.  Inputs must be
 * finite and signs +-1 (neither is checked on the device).  Outputs must not
 * overlap inputs.
 */
#ifndef NESTED_ENCODE_H
#define NESTED_ENCODE_H

#include "nested_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Where the encoder writes one linear's canonical arrays (layouts as in
 * nl_desc): base_codes [d_out][G][32], base_scales [d_out][G],
 * resid_codes [d_out][G][16*b] and resid_scales [d_out][G] (both NULL iff
 * residual_bits == 0), G = d_in / 128. */
typedef struct {
  int32_t d_out;              /* >= 1 */
  int32_t d_in;               /* >= 128 and a multiple of 128 */
  int32_t residual_bits;      /* 0, 6, 7 or 8 */
  float levels[4];            /* host: the base levels, finite, strictly ascending */
  uint8_t *base_codes;
  uint16_t *base_scales;
  uint8_t *resid_codes;
  uint16_t *resid_scales;
} nl_codes;

/*
 * Rotate a dense matrix (section 1): wt = H_o S_o W S_i H_i, or W S_i H_i
 * when sign_out is NULL.  w [d_out][d_in] fp32 row-major, sign_in [d_in],
 * sign_out [d_out] or NULL, wt [d_out][d_in] fp64 output.
 * Errors: NL_EINVAL (shape, NULL pointer, overlap of w and wt), NL_EHIP.
 */
nl_status nested_encode_rotate(int32_t d_out, int32_t d_in, const float *w, const int8_t *sign_in,
                               const int8_t *sign_out, double *wt, void *hip_stream);

/*
 * Quantise a rotated matrix (sections 2 and 3): wt [d_out][d_in] fp64 ->
 * the canonical arrays of *out (its d_out, d_in give wt's shape).
 * Errors: NL_EINVAL (shape, bits, NULL or extra pointer, levels), NL_EHIP.
 */
nl_status nested_encode_quantize(const double *wt, const nl_codes *out, void *hip_stream);

/*
 * Device workspace of nested_encode (host output *bytes): 0 for the
 * one-sided form (sign_out NULL), which is one fused launch, else
 * 8 * d_out * d_in bytes for the rotated matrix.
 */
nl_status nested_encode_workspace_bytes(int32_t d_out, int32_t d_in, int32_t two_sided, size_t *bytes);

/*
 * The whole encoder: rotate w (as nested_encode_rotate) and quantise (as
 * nested_encode_quantize) into *out.  ws: 256-byte aligned, ws_bytes >=
 * nested_encode_workspace_bytes(...) (may be NULL/0 when that is 0).
 * Errors: as the two calls above, and NL_EINVAL for a small workspace.
 */
nl_status nested_encode(const float *w, const int8_t *sign_in, const int8_t *sign_out,
                        const nl_codes *out, void *ws, size_t ws_bytes, void *hip_stream);

/*
 * The level fitter's samples (section 2): v = wt / s with s the fp16 RMS
 * scale of the weight's (row, 128-group); 0 where s is 0.  wt and v are
 * [d_out][d_in] fp64 and must not overlap.
 * Errors: NL_EINVAL (shape, NULL pointer, overlap), NL_EHIP.
 */
nl_status nested_encode_normalize(int32_t d_out, int32_t d_in, const double *wt, double *v,
                                  void *hip_stream);

/* Device workspace of nested_encode_fit_levels for n samples (host *bytes). */
nl_status nested_encode_fit_workspace_bytes(int64_t n, size_t *bytes);

/*
 * Fit four levels to the samples v[0..n) (fp64, finite) as section 2
 * describes: start at the quantiles 0.125, 0.375, 0.625, 0.875 (linear
 * interpolation between order statistics at q (n - 1), found exactly by a
 * radix select), then `iters` Lloyd iterations (every level moves to the
 * mean of the samples nearest to it, ties as for the codes; a level with no
 * samples stays), then symmetrise to (-a1, -a0, a0, a1) with
 * a0 = (l2 - l1)/2, a1 = (l3 - l0)/2.  levels: host double[4] output.
 * The fp64 cell sums are added in a fixed order, so repeated calls agree.
 * Synchronises the stream (the levels are copied to the host).
 * ws: 256-byte aligned, ws_bytes >= nested_encode_fit_workspace_bytes(n);
 * no clearing needed.
 * Errors: NL_EINVAL (n < 1, iters outside 0..100000, NULL pointer, small or
 * misaligned ws), NL_EHIP.
 */
nl_status nested_encode_fit_levels(const double *v, int64_t n, int32_t iters, double *levels,
                                   void *ws, size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NESTED_ENCODE_H */
