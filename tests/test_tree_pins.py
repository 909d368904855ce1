"""Pins of the draft-tree oracle (oracle/tree.py) to the forum post's POC
section 6: with distinct path priorities the best-first tree is exactly the
N highest-priority paths (brute force over every path), ties pop in push
order, ancestor masks match the parent chain, and greedy acceptance is
checked against hand-made trees and its defining properties."""
import itertools

import numpy as np
import pytest

import synth
from oracle import tree


def all_paths(p):
    D, R = p.shape
    out = []
    for k in range(1, D + 1):
        for rs in itertools.product(range(R), repeat=k):
            pr = 1.0
            for d, r in enumerate(rs):
                pr *= p[d, r]
            out.append((pr, rs))
    return out


@pytest.mark.parametrize("D,R,N", [(3, 4, 10), (4, 3, 20), (2, 5, 12), (3, 4, 64), (2, 3, 64)])
def test_best_first_is_top_n_paths(D, R, N):
    p = np.random.default_rng(D * 10 + R).uniform(0.01, 0.9, (D, R))
    t = tree.build(p, N)
    # paths of the built nodes
    paths = []
    for k in range(t["n"]):
        rs, u = [], k
        while u >= 0:
            rs.append(int(t["rank"][u]))
            u = int(t["parent"][u])
        paths.append(tuple(reversed(rs)))
    brute = sorted(all_paths(p), key=lambda x: -x[0])[:N]
    assert paths == [rs for _, rs in brute]
    assert t["n"] == min(N, len(brute))


def test_ties_pop_in_push_order():
    # every rank equally likely: all depth-1 paths tie, then all depth-2 ones
    p = np.full((2, 3), 0.5)
    t = tree.build(p, 6)
    assert t["parent"].tolist() == [-1, -1, -1, 0, 0, 0]
    assert t["rank"].tolist() == [0, 1, 2, 0, 1, 2]


def test_ancestor_masks_follow_parents():
    p = synth.make_rank_stats(D=8, R=16, cfg=70)
    t = tree.build(p, 64)
    for k in range(t["n"]):
        m, u = 0, k
        while u >= 0:
            m |= 1 << u
            u = int(t["parent"][u])
        assert int(t["anc"][k]) == m
        assert t["depth"][k] == bin(m).count("1")
    # a parent is always popped before its children; priorities never increase
    assert all(t["parent"][k] < k for k in range(t["n"]))
    assert np.all(np.diff(t["prio"]) <= 0)


def test_acceptance_by_hand():
    #            root
    #           /    \
    #         0(a)   1(b)
    #         |  \
    #       2(c) 3(d)
    parent = np.array([-1, -1, 0, 0])
    draft = np.array([10, 11, 12, 13])
    assert tree.accept(parent, draft, [10, 13, 0, 0, 0]) == ([0, 3], 0)      # root->a, a->d, bonus after d
    assert tree.accept(parent, draft, [11, 5, 6, 7, 8]) == ([1], 6)          # root->b, bonus 6
    assert tree.accept(parent, draft, [99, 1, 2, 3, 4]) == ([], 99)          # nothing matches: bonus only
    assert tree.accept(parent, draft, [10, 12, 0, 7, 0]) == ([0, 2], 7)


def test_acceptance_properties():
    p = synth.make_rank_stats(cfg=71)
    t = tree.build(p, 32)
    draft, argmax = synth.make_tree_tokens(t["parent"], 20, cfg=71)
    for b in range(20):
        path, bonus = tree.accept(t["parent"], draft[b], argmax[b])
        u = -1
        for c in path:                      # a chain down from the root, each step the argmax
            assert t["parent"][c] == u and draft[b, c] == argmax[b, u + 1]
            u = c
        kids = [c for c in range(32) if t["parent"][c] == u]
        assert all(draft[b, c] != argmax[b, u + 1] for c in kids)   # maximal
        assert bonus == argmax[b, u + 1]
