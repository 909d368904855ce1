"""CPU oracle of the draft tree: best-first construction from rank statistics
and greedy acceptance.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product package never does.

Source: the forum post "bit-nested" (page 1 of the source pages), POC
recipe section 6, "Building the draft tree":
  * p_d(r) is the frequency of the verifier's token having rank r in the
    draft's logits at draft depth d (r < 16);
  * the priority of a path (r_1 .. r_k) is the product of p_d(r_d); the tree
    is grown best-first: pop the best path, push its children, stop at N
    nodes;
  * greedy acceptance follows the verifier's argmax down the tree: the
    longest matching prefix is accepted, plus one bonus token from the
    verifier.

Readings (listed with the design notes):
  * the root (the last verified token) is not a node; its children are the
    depth-1 paths; a path of depth D (the number of depths with statistics)
    has no children;
  * priorities are fp64 products taken in depth order; among equal
    priorities the path pushed first is popped first (a heap with an
    insertion counter), and a parent pushes its children in rank order;
  * a node's draft token is the draft's rank-r token at its parent; siblings
    therefore carry distinct tokens, and at most one child matches.
"""
from __future__ import annotations

import heapq

import numpy as np


def build(p, N: int) -> dict:
    """Best-first tree of at most N nodes from p[D][R] (fp64).  Returns
    parent (-1 = root), depth (1-based), rank, prio and anc (bit j set when
    node j is an ancestor of the node or the node itself), in pop order."""
    p = np.asarray(p, np.float64)
    D, R = p.shape
    heap, counter = [], 0
    for r in range(R):
        heapq.heappush(heap, (-p[0, r], counter, -1, 1, r, p[0, r]))
        counter += 1
    parent, depth, rank, prio, anc = [], [], [], [], []
    while heap and len(parent) < N:
        _, _, par, d, r, pr = heapq.heappop(heap)
        k = len(parent)
        parent.append(par)
        depth.append(d)
        rank.append(r)
        prio.append(pr)
        anc.append((anc[par] if par >= 0 else 0) | (1 << k))
        if d < D:
            for rr in range(R):
                cp = pr * p[d, rr]
                heapq.heappush(heap, (-cp, counter, k, d + 1, rr, cp))
                counter += 1
    return {"parent": np.array(parent, np.int32), "depth": np.array(depth, np.int32),
            "rank": np.array(rank, np.int32), "prio": np.array(prio, np.float64),
            "anc": np.array(anc, np.uint64), "n": len(parent)}


def accept(parent, draft_token, argmax):
    """Greedy acceptance.  argmax[0] is the verifier's token after the root,
    argmax[1 + i] after node i.  Returns (accepted nodes root-down, bonus
    token)."""
    parent = np.asarray(parent)
    u, path = -1, []
    while True:
        target = argmax[u + 1]
        hit = [c for c in range(len(parent)) if parent[c] == u and draft_token[c] == target]
        if not hit:
            break
        u = hit[0]
        path.append(u)
    return path, int(argmax[u + 1])
