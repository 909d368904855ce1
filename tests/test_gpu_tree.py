"""Parity of the HIP draft tree (include/nested_tree.h) with the oracle
(oracle/tree.py): structure, fp64 priorities and ancestor masks bit-exact,
acceptance exact for every sequence of a batch."""
import numpy as np
import pytest

import synth
from oracle import tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.fixture(scope="module")
def nl(torch_cuda):
    import bit_nested_quantized_amd as m
    m.lib()
    return m


def gpu_build(nl, torch, p, N):
    out = nl.tree_build(torch.from_numpy(np.ascontiguousarray(p, np.float64)).cuda(), N)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


CASES = [("stats-8x16-64", synth.make_rank_stats(8, 16, cfg=80), 64),
         ("stats-8x16-16", synth.make_rank_stats(8, 16, cfg=81), 16),
         ("stats-4x4-50", synth.make_rank_stats(4, 4, cfg=82), 50),
         ("ties", np.full((3, 4), 0.5), 40),
         ("zeros", np.r_[[[0.6, 0.3, 0.0, 0.0]], [[0.5, 0.0, 0.5, 0.0]]], 20),   # fewer live paths than N
         ("chain", np.full((70, 1), 0.9), 64),
         ("short", np.array([[0.7, 0.2, 0.1]]), 10),
         # rows non-increasing in rank (the one-candidate-per-node path), with
         # ties and zeros; and the same statistics with one row out of order
         # (the path that keeps every candidate)
         ("sorted-ties-zeros", np.array([[0.5, 0.5, 0.25, 0.0], [1.0, 0.5, 0.5, 0.0], [0.25, 0.25, 0.0, 0.0]]), 64),
         ("sorted-random", -np.sort(-np.random.default_rng(7).uniform(0, 1, (9, 16)) ** 3, axis=1), 64),
         ("unsorted-row", synth.make_rank_stats(8, 16, cfg=80)[:, [0, 1, 2, 3, 5, 4] + list(range(6, 16))], 64)]


@pytest.mark.parametrize("name,p,N", CASES, ids=[c[0] for c in CASES])
def test_build_matches_oracle(nl, torch_cuda, name, p, N):
    got = gpu_build(nl, torch_cuda, p, N)
    want = tree.build(p, N)
    n = want["n"]
    assert int(got["count"][0]) == n
    for k in ("parent", "depth", "rank"):
        np.testing.assert_array_equal(got[k][:n], want[k], err_msg=k)
    np.testing.assert_array_equal(got["prio"][:n], want["prio"])
    np.testing.assert_array_equal(got["anc"][:n].view(np.uint64), want["anc"])


@pytest.mark.parametrize("N,B", [(64, 300), (16, 7), (1, 5)])
def test_accept_matches_oracle(nl, torch_cuda, N, B):
    t = tree.build(synth.make_rank_stats(8, 16, cfg=83), N)
    draft, argmax = synth.make_tree_tokens(t["parent"], B, cfg=83 + N)
    d = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    n, path, bonus = nl.tree_accept(d(t["parent"]), d(draft), d(argmax))
    n, path, bonus = n.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy()
    for b in range(B):
        want_path, want_bonus = tree.accept(t["parent"], draft[b], argmax[b])
        assert n[b] == len(want_path), b
        assert path[b, :n[b]].tolist() == want_path, b
        assert bonus[b] == want_bonus, b
    assert n.max() >= min(3, N)  # the generator makes long chains happen
