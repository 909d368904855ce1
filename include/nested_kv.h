/*
 * nested_kv.h -- C ABI of the nested KV cache (KV4 base + 4-bit refinement)
 * and of the tree-masked attention that reads it, on MI355X (gfx950), in
 * the same library as nested_linear.h.
 *
 * Source: "BitNest: Bit-Nested Speculative Decoding for Memory-Efficient LLM
 * Inference Acceleration" (page 2 of the source pages), section 3.4 and
 * appendix A.2.  On write, each (token, KV head) vector x of d = 128 is
 * quantised: s = max|x| / 7, q4 = clip(round(x / s), -8, 7) (eq. 11),
 * q_r = clip(round((x - q4 s) / (s / 16)), -8, 7) (eq. 13).  The draft reads
 * KV4, x = q4 s (eq. 12); verification reads KV8, x = (16 q4 + q_r) s / 16
 * (eq. 14).  The attention is the verify pass's over a draft tree: token t
 * attends to the L context positions and to the tree nodes set in its
 * ancestor mask anc[t] (itself included; nested_tree.h produces the masks).
 *
 * Cache layout: row = position * H_kv + kv_head, positions 0 .. L-1 the
 * context and L .. L+T-1 the tree tokens; per row 64 bytes of each plane
 * (two's-complement nibbles, dimension k in byte k/2, low nibble for even k)
 * and one fp32 scale.  The quantiser works in fp32 (correctly rounded
 * divisions, round half to even, the residual x - q4 s formed exactly and
 * rounded once); a zero vector stores scale 0 and zero codes.
 *
 * Conventions as in nested_linear.h.  All arrays are device pointers.
 */
#ifndef NESTED_KV_H
#define NESTED_KV_H

#include "nested_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

#define NL_KV_HEAD_DIM 128
#define NL_KV_MAX_ROWS 256   /* query rows per KV head: T * (H_q / H_kv) */

/*
 * Quantise n vectors x [n][128] (bf16 bit patterns) into cache rows row[n]
 * of the planes base [rows][64], ref [rows][64] and the scales scale[rows].
 * Errors: NL_EINVAL (n < 1, NULL pointer), NL_EHIP.
 */
nl_status nested_kv_write(const void *x_bf16, int32_t n, const int32_t *row, uint8_t *base, uint8_t *ref,
                          float *scale, void *hip_stream);

/* Workspace bytes of nested_kv_attention for these sizes (host *bytes). */
nl_status nested_kv_attention_workspace_bytes(int32_t T, int32_t H_q, int32_t H_kv, int32_t L, size_t *bytes);

/*
 * out [T][H_q][128] fp32 = softmax(q . k / sqrt(128)) v over the visible
 * keys, with q [T][H_q][128] bf16 and query head j reading KV head
 * j / (H_q / H_kv).  verify != 0 reads KV8 (k_ref and v_ref required),
 * verify == 0 KV4 (the refinement planes are not read and may be NULL).
 * anc [T] uint64 ancestor masks.  ws: 256-byte aligned, at least
 * nested_kv_attention_workspace_bytes(...).  Two launches: the positions
 * are split into spans of 64-position sub-chunks (at most 64 spans per KV
 * head), each span's partial softmax state is written to ws, then the spans
 * are combined.  Both products run on fp16 matrix cores with exact integer
 * K/V codes and fp32 accumulation; the result is held to within 5e-4 of
 * max|v| of the exact attention over the dequantised cache.
 * Errors: NL_EINVAL (T outside 1..64, H_kv < 1, H_q not a multiple of H_kv,
 * T * H_q / H_kv > 256, L < 0, NULL pointer, small or misaligned ws),
 * NL_EHIP.
 */
nl_status nested_kv_attention(const void *q_bf16, int32_t T, int32_t H_q, int32_t H_kv, int32_t L,
                              const uint8_t *k_base, const uint8_t *k_ref, const float *k_scale,
                              const uint8_t *v_base, const uint8_t *v_ref, const float *v_scale,
                              const uint64_t *anc, int32_t verify, float *out, void *ws, size_t ws_bytes,
                              void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NESTED_KV_H */
