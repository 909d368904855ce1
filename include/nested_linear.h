/*
 * nested_linear.h -- C ABI of the bit-nested quantized linear for AMD MI355X
 * (gfx950).
 *
 * The layer is the verifier Linear of the forum post "bit-nested" (page 1 of
 * the source pages), POC recipe section 4: for a batch of T draft-tree
 * tokens x[t] (bf16),
 *
 *     x'  = H_i S_i x                      (section 1: randomized Hadamard)
 *     y~  = (Q_base + Q_resid) x'          (sections 2 and 3)
 *     y   = S_o H_o y~                     (section 1, output side)
 *
 * where Q_base[r,k] = levels[c(r,k)] * s_base[r, k/128] is the 2-bit
 * Lloyd-Max base and Q_resid[r,k] = q(r,k) * s_resid[r, k/128] the uniform
 * b-bit residual (b = 6, 7 or 8), both in the rotated basis.  The draft
 * forward drops the Q_resid term and nothing else (section 4); it reads only
 * the base planes, the dual-plane
 * principle of the BitNest paper (page 2, section 3.3 "Dual-Plane Weight
 * Storage").  H is the normalised Sylvester-Hadamard matrix applied
 * block-diagonally with block b = the largest power of two dividing the
 * dimension, capped at 4096 (section 1, "Block size").
 *
 * All calls return an nl_status and never abort or throw.  On failure
 * nested_linear_last_error() returns a message for the calling thread.
 * Pointers are DEVICE pointers unless marked "host".  Compute calls are
 * asynchronous on the given hipStream_t (passed as void*, NULL = the null
 * stream); they never synchronise the host.  Faults inside kernels surface at
 * the caller's next synchronisation.
 */
#ifndef NESTED_LINEAR_H
#define NESTED_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nl_linear *nl_handle;      /* one nested linear, opaque */
typedef struct nl_group *nl_group_handle; /* experts of one MoE projection, opaque */

typedef enum {
  NL_OK = 0,
  NL_EINVAL = 1,        /* bad argument: shape, pointer, T, bits, workspace */
  NL_ENOMEM = 2,        /* device allocation failed */
  NL_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
  NL_EUNSUPPORTED = 4   /* valid request outside this library's range (T > 64) */
} nl_status;

#define NL_MAX_T 64       /* largest draft tree per call (prefill is out of scope) */
#define NL_GROUP 128      /* weights per scale group along d_in */

/*
 * Canonical packed input of one linear (W is d_out x d_in, G = d_in / 128):
 *   base_codes   [d_out][G][32] bytes: bytes 0..15 = bit 0 of the group's
 *                128 codes, bytes 16..31 = bit 1; code j at bit (j & 7) of
 *                byte (j >> 3) (POC section 2: "2 bit-planes").  Code c
 *                selects levels[c].
 *   base_scales  [d_out][G] fp16 bit patterns (one scale per row and 128-group).
 *   resid_codes  [d_out][G][16*b] bytes: 128 b-bit two's-complement fields,
 *                field j at bits [j*b, j*b + b) of the group's little-endian
 *                bit string (POC section 3: the residual grid is uniform and symmetric).
 *   resid_scales [d_out][G] fp16 bit patterns.
 *   sign_in      [d_in] int8, each +1 or -1 (S_i).
 *   sign_out     [d_out] int8 (S_o), or NULL: the output then stays in the
 *                rotated basis, y = y~ (the one-sided form).
 * All arrays are device pointers; they are read only during create.
 */
typedef struct {
  int32_t d_out;              /* >= 1 */
  int32_t d_in;               /* >= 128 and a multiple of 128 */
  int32_t residual_bits;      /* 0 (draft-only linear), 6, 7 or 8 */
  const uint8_t *base_codes;
  const uint16_t *base_scales;
  const uint8_t *resid_codes;   /* NULL iff residual_bits == 0 */
  const uint16_t *resid_scales; /* NULL iff residual_bits == 0 */
  const int8_t *sign_in;
  const int8_t *sign_out;       /* may be NULL */
  float levels[4];              /* host values of the 4 base levels, finite */
} nl_desc;

/*
 * Build a linear from the canonical arrays (POC sections 2-3 storage).
 * Copies and repacks everything into library-owned device memory laid out
 * for the gfx950 kernels; the caller may free its arrays when this returns.
 * Synchronises the device.  Errors: NL_EINVAL (shape, bits, NULL pointer,
 * a sign not +-1, non-finite level), NL_EUNSUPPORTED (levels whose fp16
 * copy, after the one common rescale that create searches for, errs by more
 * than 2e-3 relative: a nonzero level some 1e10 times smaller than the
 * largest falls below fp16's subnormal range), NL_ENOMEM, NL_EHIP.  *out is
 * set only on success.  A handle is immutable after create: concurrent calls on
 * different streams are safe when each uses its own workspace.
 */
nl_status nested_linear_create(const nl_desc *desc, nl_handle *out);

/* Free a linear.  The caller ensures no call on it is still running. */
nl_status nested_linear_destroy(nl_handle h);

/*
 * Bytes of workspace a draft or verify call with up to T_max tokens needs
 * (host output *bytes).  The workspace is caller-owned device memory,
 * 256-byte aligned, and must not be shared by calls that may run
 * concurrently.  It must be zero-filled once before its first use: its
 * first 1 MiB holds the counters through which the workgroups of one launch
 * hand work to each other, and every call leaves them at zero again, so later
 * calls (of any linear, any T) need no clearing.
 *
 * Ordering assumption.  Inside one launch a workgroup only ever waits for
 * workgroups of lower index (the activation rotation, split partial sums, the
 * output rotation's inputs), and the GPU dispatches the workgroups of a
 * launch in index order, so every awaited workgroup is running or done.
 * Each wait is still bounded by a spin limit (about a tenth of a second).  A
 * wait that gives up adds one to the workspace's first 32-bit word (the error
 * word), the outputs it would have fed are written as NaN, and the launch
 * ends normally; such a workspace must be reset with
 * nested_linear_workspace_status(..., clear = 1) before its next use.
 */
nl_status nested_linear_workspace_bytes(nl_handle h, int32_t T_max, size_t *bytes);

/*
 * Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * verify (verify != 0) or draft forward of nested_linear_verify / _draft, with
 * the workspace taken from a static device array inside the library instead of
 * a caller's buffer.  The array is 32 MiB per GPU, held from the library's
 * load until the process ends; a call whose plan needs more (a very large
 * d_out with large T, two-sided) fails with NL_EUNSUPPORTED and must use the
 * workspace form.  Each call first clears the counters it uses with a small
 * kernel (two launches per call, both capturable), so a wait that gave up in
 * an earlier call carries over nothing; such a call's outputs are NaN (this
 * form has no readable error word).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.  Arguments and other errors are
 * those of nested_linear_verify.  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.
 */
nl_status nested_linear_forward_static(nl_handle h, int32_t verify, const void *x_bf16, int32_t T, float *y,
                                       void *hip_stream);

/*
 * Verify forward (POC section 4): y = S_o H_o ((Q_base + Q_resid) H_i S_i x)
 * for T tokens, or the rotated-basis y~ when the linear has no sign_out.
 *   x   [T][d_in] bf16 bit patterns (row-major), 16-byte aligned (rows are
 *       read 16 bytes at a time); y [T][d_out] fp32 output, must not
 *       overlap x or ws.
 *   ws  workspace of ws_bytes >= nested_linear_workspace_bytes(h, T).
 * Weight bytes are streamed from HBM once per call for all T tokens.  One
 * kernel launch, of one of two designs chosen by T (NL_TUNE_STAGED_T_*):
 * either each contraction workgroup holds its K-range of x' in LDS (rotated
 * by itself for T <= 2, else by rotation workgroups and handed over through
 * the workspace), or rotation workgroups write x' and contraction workgroups
 * stage it through LDS a chunk at a time.  Hand-overs wait on workspace
 * counters after the weights are requested; the last workgroups (two-sided
 * form only) apply S_o H_o.
 * Errors: NL_EINVAL (NULL pointer, T < 1, x not 16-byte aligned, small or
 * misaligned ws, linear without a residual), NL_EUNSUPPORTED (T > 64, or d_out beyond what the
 * counter region serves: about 16000 row blocks of 64 or 128 rows), NL_EHIP
 * (launch failure).
 */
nl_status nested_linear_verify(nl_handle h, const void *x_bf16, int32_t T, float *y,
                               void *ws, size_t ws_bytes, void *hip_stream);

/*
 * Draft forward (POC section 4: the verifier without its residual term): as
 * verify with Q_resid omitted; only the base planes and base scales are read.
 */
nl_status nested_linear_draft(nl_handle h, const void *x_bf16, int32_t T, float *y,
                              void *ws, size_t ws_bytes, void *hip_stream);

/*
 * Verify / draft of n linears (1 <= n <= 4) that read the same activations,
 * in one launch: y_i = linear i applied to x (for instance the q, k and v
 * projections of an attention block, or the gate and up projections of an
 * MLP).  The linears share d_in, the residual bits (verify), and the output
 * rotation's presence and block; each keeps its own signs, planes, scales and
 * levels, and each output ys[i] is [T][d_out_i] fp32.  ys is a host array of n
 * device pointers.  The workspace must hold
 * nested_linear_multi_workspace_bytes(hs, n, T) bytes; the other rules are
 * those of nested_linear_verify.  Each linear's arithmetic is that of a
 * separate call; the split count of K (and with it the order in which the
 * split partial sums are added) may differ.  Linears of one shape without the
 * output rotation (gate and up, say) take, from T = 33 for verify and T = 24
 * for the draft (NL_TUNE_MULTI_STAGED_T_*), the staged-x' launch in its
 * grouped form: each linear is an expert that takes all T rows; that form
 * keeps its expert descriptors and row maps in the workspace and writes them
 * with a small kernel on the same stream before the launch.
 */
nl_status nested_linear_verify_multi(const nl_handle *hs /* host array */, int32_t n, const void *x_bf16,
                                     int32_t T, float *const *ys /* host array */, void *ws, size_t ws_bytes,
                                     void *hip_stream);
nl_status nested_linear_draft_multi(const nl_handle *hs, int32_t n, const void *x_bf16, int32_t T,
                                    float *const *ys, void *ws, size_t ws_bytes, void *hip_stream);
nl_status nested_linear_multi_workspace_bytes(const nl_handle *hs, int32_t n, int32_t T_max, size_t *bytes);

/*
 * Host query of the launch plan a verify or draft call would use (no device
 * work, no handle needed): n linears of d_out[i] x d_in read by one call,
 * bits = their residual bits for verify or 0 for the draft, two_sided != 0
 * when they carry sign_out, T tokens.  out[0 .. 8 + 6 n) receives (truncated
 * to out_len): local form (0/1), 16-token tiles, waves per workgroup,
 * rotation / contraction / finish workgroups, LDS bytes per workgroup, bytes
 * per x' chunk blob; then per linear: splits of K, chunks per split, row
 * tiles per workgroup, waves per row tile, row blocks, output superblocks.
 * Errors: NL_EINVAL.
 */
nl_status nested_linear_describe_call(const int32_t *d_out /* host array */, int32_t n, int32_t d_in, int32_t bits,
                                      int32_t two_sided, int32_t T, int32_t *out /* host */, int32_t out_len);

/*
 * Reads the error word of a workspace (waits that gave up, see
 * nested_linear_workspace_bytes) into *errors after synchronising hip_stream;
 * with clear != 0 it then zeroes the workspace's counter region (its first
 * MiB) and synchronises again, which makes a workspace usable after a call
 * that reported errors.  Not for use inside graph capture (it synchronises).
 * Errors: NL_EINVAL (NULL or misaligned pointers), NL_EHIP.
 */
nl_status nested_linear_workspace_status(void *ws, uint32_t *errors /* host */, int32_t clear, void *hip_stream);

/*
 * Tuning hook of the launch planner and the waits (process-wide, not
 * thread-safe; results do not depend on it beyond the summation order of
 * split-K partial sums).  value <= 0 restores a knob's default where a
 * default exists.
 */
typedef enum {
  NL_TUNE_SPLITS = 1,          /* force the split count of K (0: planner) */
  NL_TUNE_ROW_TILES = 2,       /* force 16-row tiles per workgroup (0: planner) */
  NL_TUNE_WAVES_PER_TILE = 3,  /* force waves sharing a row tile (0: planner) */
  NL_TUNE_LOCAL_T = 4,         /* largest T rotated inside each workgroup (default 2; 0 disables) */
  NL_TUNE_CUS = 5,             /* compute units the planner fills (default 256) */
  NL_TUNE_LAT_US = 6,          /* planner: memory round trip under load, us (default 2) */
  NL_TUNE_HBM_GBS = 7,         /* planner: HBM stream rate, GB/s (default 6500) */
  NL_TUNE_SPLIT_US = 8,        /* planner: cost of a split-K reduction, us (default 1.5) */
  NL_TUNE_XDMA_GBS = 9,        /* planner: per-CU rate of the x' copy into LDS, GB/s (default 100) */
  NL_TUNE_SPIN_LIMIT = 10,     /* polls before a wait gives up (default 2^22) */
  NL_TUNE_WAIT_EXTRA = 11,     /* test hook: added to every wait target, > 0 makes the waits give up */
  NL_TUNE_WAVES = 12,          /* draft waves per workgroup up to 16 tokens: 0 or 8 (default), 12 */
  NL_TUNE_STAGED_T_VERIFY = 13, /* single-linear verify with T at or above this uses the staged-x' launch
                                   (default 9; 65 never) */
  NL_TUNE_STAGED_T_DRAFT = 14,  /* the same for the draft (default 1: always) */
  NL_TUNE_STAGED_WAVES = 15,    /* tile waves per workgroup of the staged launch at 3..48 tokens: 4 or 8
                                   (0: planner) */
  NL_TUNE_MULTI_STAGED_T_VERIFY = 16, /* *_multi verify of linears of one shape (one-sided) with T at or
                                         above this takes the staged launch's grouped form (default 33;
                                         65 never) */
  NL_TUNE_MULTI_STAGED_T_DRAFT = 17   /* the same for the draft (default 24) */
} nl_tuning;
nl_status nested_linear_set_tuning(int32_t knob, double value);

/*
 * The three stages of a draft/verify call as separate kernel launches, for
 * callers that time them apart or run their own work in between (draft and
 * verify fuse them into one launch).  They must run in this order, on one
 * stream, with one workspace and the same T; they leave the workspace
 * counters untouched:
 *   prepare_input  x' = H_i S_i x into ws (POC section 1: the activation
 *                  is rotated a single time per linear and call);
 *   contract       y~ = Q x' from the packed planes (verify != 0 adds the
 *                  residual); writes partial sums into ws, or y directly
 *                  when the linear is one-sided and needs no reduction;
 *   finish         sums the partials and applies y = S_o H_o y~ (a no-op
 *                  when contract already wrote y).
 * Arguments and errors are those of nested_linear_verify.
 */
nl_status nested_linear_prepare_input(nl_handle h, const void *x_bf16, int32_t T,
                                      void *ws, size_t ws_bytes, void *hip_stream);
nl_status nested_linear_contract(nl_handle h, int32_t verify, int32_t T, float *y,
                                 void *ws, size_t ws_bytes, void *hip_stream);
nl_status nested_linear_finish(nl_handle h, int32_t T, float *y, void *ws, size_t ws_bytes,
                               void *hip_stream);

/*
 * Grouped forward of a mixture-of-experts projection (DFlash write-up,
 * "The verify's own cost": tokens sorted by expert, one grouped launch per
 * projection instead of a per-expert loop).  All experts share d_out, d_in,
 * residual_bits and the presence of sign_out; each keeps its own planes,
 * scales, levels and signs.  group_create copies the experts' device
 * descriptors; the expert handles must outlive the group.
 */
nl_status nested_linear_group_create(const nl_handle *experts /* host array */, int32_t n,
                                     nl_group_handle *out);
nl_status nested_linear_group_destroy(nl_group_handle g);
nl_status nested_linear_group_workspace_bytes(nl_group_handle g, int32_t P_max,
                                              size_t *bytes);
/*
 * Pair p (0 <= p < P) applies expert e, the one with
 * expert_offsets[e] <= p < expert_offsets[e+1], to row pair_token[p] of x;
 * pairs are sorted by expert.  x holds either one row per token (gate / up
 * projections: an expert receives each token at most once) or one row per
 * pair (the down projection, whose input is each pair's own activation:
 * pair_token[p] = p and x_rows = P).
 *   pair_token     [P] int32 device, values in [0, x_rows); a value outside
 *                  reads as a zero row
 *   expert_offsets [n+1] int32 device, non-decreasing, [0] = 0, [n] = P
 *   x              [x_rows][d_in] bf16 device
 *   T              at most this many pairs go to any one expert (1..64; the
 *                  tokens of the block); rows of an expert past the first
 *                  16 * ceil(T / 16) are not computed
 *   y              [P][d_out] fp32, row p = expert e's forward of x row
 *                  pair_token[p].
 * Offsets and tokens stay on the device: experts with no pairs cost no
 * weight traffic and the host never synchronises.  The offsets and tokens
 * are trusted to satisfy the rules above (they are not validated on the
 * device); offsets that break them can leave the launch waiting until the
 * spin limit.  The workspace rules are those of nested_linear_workspace_bytes.
 * Errors: NL_EINVAL, NL_EUNSUPPORTED (T > 64), NL_EHIP.
 */
nl_status nested_linear_verify_grouped(nl_group_handle g, const int32_t *pair_token,
                                       const int32_t *expert_offsets, int32_t P,
                                       const void *x_bf16, int32_t x_rows, int32_t T, float *y,
                                       void *ws, size_t ws_bytes, void *hip_stream);
nl_status nested_linear_draft_grouped(nl_group_handle g, const int32_t *pair_token,
                                      const int32_t *expert_offsets, int32_t P,
                                      const void *x_bf16, int32_t x_rows, int32_t T, float *y,
                                      void *ws, size_t ws_bytes, void *hip_stream);

/*
 * Test hook: decode rows [row0, row0 + nrows) of the library's internal
 * packed layout back to integers through the same unpack code the kernels
 * use.  base_idx [nrows][d_in] uint8 receives the level index 0..3;
 * resid [nrows][d_in] int8 the residual integer (may be NULL; ignored for a
 * draft-only linear).  Asynchronous on hip_stream.
 */
nl_status nested_linear_decode(nl_handle h, int32_t row0, int32_t nrows, uint8_t *base_idx,
                               int8_t *resid, void *hip_stream);

/* Host queries: shape, residual bits, the split of d_in into rotation
 * blocks, and the largest relative error of the base levels as the kernels
 * hold them (fp16 after a per-linear exact rescale; 0 when exact). */
nl_status nested_linear_info(nl_handle h, int32_t *d_out, int32_t *d_in, int32_t *bits,
                             int32_t *block_in, int32_t *block_out, float *level_rel_err);

/*
 * Kernel timing, a profiling aid that changes no result.  Between
 * nested_linear_timing_begin(capacity) and nested_linear_timing_end(), the
 * single kernel launch of each verify / draft call (single or grouped) is
 * made with a pair of HIP events attached to the dispatch itself, so the
 * pair brackets the kernel's execution (not the queue around it), for the
 * first `capacity` such launches of the process; launches into a stream that
 * is being captured into a graph are not recorded.  timing_end waits for the
 * recorded launches, writes their durations in microseconds, in launch
 * order, to us[0 .. min(recorded, capacity)), stores that number in *count
 * and releases the events.  begin allocates 2 * capacity HIP events (host
 * objects, no device memory); a second begin discards the first.  Not
 * thread-safe.  Errors: NL_EINVAL (capacity outside [1, 2^20], end without
 * begin, NULL pointers), NL_EHIP (event creation or query failed).
 */
nl_status nested_linear_timing_begin(int32_t capacity);
nl_status nested_linear_timing_end(float *us, int32_t capacity, int32_t *count);

/*
 * Measurement aid: the streaming-read reference.  One launch reads every
 * byte of [src, src + bytes) once from device memory with 16-byte
 * nontemporal loads (the load kind the forward streams its weights with) and
 * computes nothing else, so bytes / duration is the read rate this GPU
 * reaches in practice, the measured ceiling set beside the nominal peak.
 *   src   device, 16-byte aligned; bytes a positive multiple of 16
 *   sink  device, at least `grid` 32-bit words (practically never written)
 *   grid  workgroups of 256 threads (0: 2048)
 * Asynchronous on hip_stream.  Errors: NL_EINVAL, NL_EHIP.
 */
nl_status nested_linear_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t grid,
                                    void *hip_stream);

/* Message of the last failed call on this thread ("" if none). */
const char *nested_linear_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NESTED_LINEAR_H */
