/*
 * nested_tree.h -- C ABI of the draft tree for the bit-nested verifier on
 * MI355X (gfx950), in the same library as nested_linear.h.
 *
 * Source: the forum post "bit-nested" (page 1 of the source pages), POC
 * recipe section 6, "Building the draft tree".  p_d(r) is how often the
 * verifier's token has rank r in the draft's logits at draft depth d; a
 * path (r_1 .. r_k) has priority prod_d p_d(r_d); the tree is grown
 * best-first (pop the best path, push its children) to N nodes; greedy
 * acceptance follows the verifier's argmax down the tree and accepts the
 * longest matching prefix plus one bonus token.
 *
 * Readings: the root (the last verified token) is not a node; priorities are
 * fp64 products in depth order, and among equal priorities the path pushed
 * first is popped first (children are pushed in rank order when their
 * parent is popped); a node's draft token is the draft's rank-r token at its
 * parent, so siblings carry distinct tokens (if several children match,
 * the lowest node index is taken).
 *
 * Conventions as in nested_linear.h.  All arrays are device pointers.
 */
#ifndef NESTED_TREE_H
#define NESTED_TREE_H

#include "nested_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

#define NL_TREE_MAX_NODES 64   /* one tree fits one verify call (NL_MAX_T) */
#define NL_TREE_MAX_RANKS 16

/*
 * Grow the tree from p [D][R] fp64 (values in [0, 1], finite; not checked on
 * the device).  Outputs, in pop order, for n <= N nodes: parent[n] (-1 for
 * a child of the root), depth[n] (1-based), rank[n], prio[n] (fp64), and
 * anc[n], the node's ancestor mask (bit j set when node j is an ancestor or
 * the node itself: the tree-attention mask of the verify pass); *count = n
 * (a device int32; n < N only when fewer paths exist).  One workgroup.
 * Errors: NL_EINVAL (D < 1, R outside 1..16, N outside 1..64, NULL pointer),
 * NL_EHIP.
 */
nl_status nested_tree_build(const double *p, int32_t D, int32_t R, int32_t N, int32_t *parent, int32_t *depth,
                            int32_t *rank, double *prio, uint64_t *anc, int32_t *count, void *hip_stream);

/*
 * Greedy acceptance for B sequences sharing one tree of N nodes:
 * draft_token [B][N] (token of each node), argmax [B][N+1] (the verifier's
 * argmax after the root at index 0 and after node i at index 1 + i).
 * Outputs: n_accepted[B] (length of the accepted chain), path [B][N] (its
 * node indices from the root down; entries past n_accepted are left as
 * they were), bonus[B] (the verifier's token after the last accepted node).
 * One wave per sequence.  Errors: NL_EINVAL (N outside 1..64, B < 1, NULL
 * pointer), NL_EHIP.
 */
nl_status nested_tree_accept(const int32_t *parent, int32_t N, int32_t B, const int32_t *draft_token,
                             const int32_t *argmax, int32_t *n_accepted, int32_t *path, int32_t *bonus,
                             void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NESTED_TREE_H */
