"""Parity of the nested KV cache and its tree-masked attention
(include/nested_kv.h) with the oracle (oracle/kv.py).

The writer's codes and scales are integer/fp32 decisions taken the same way
on both sides (correctly rounded fp32 divisions, round half to even, the
residual formed exactly), so the planes are compared byte for byte.  The
attention runs on fp16 matrix cores against the fp64 oracle: the query is
widened to fp16 exactly (a power of two per row), the K/V codes are exact
fp16 integers whose products land exactly in fp32 accumulators, a score is
an fp32 sum of 128 terms (relative error ~1e-5 at worst), the softmax
weights times the V scales travel as an fp16 pair hi + lo (~22 bits), and
the output is an fp32 sum over at most a few thousand keys, so
|dO| <= 5e-4 * max|v_hat| holds with a wide margin.
"""
import numpy as np
import pytest

import synth
from oracle import kv, tree

pytestmark = pytest.mark.gpu
TOL = 5e-4


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


def vectors(rng, n, spread=True):
    x = rng.standard_normal((n, 128)).astype(np.float32)
    if spread:
        x *= np.exp(rng.normal(0, 1.5, (n, 1))).astype(np.float32)
    return synth.f32_to_bf16_bits(x)


def write(nl, torch, xb, rows, n_rows):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    base = torch.zeros((n_rows, 64), dtype=torch.uint8, device="cuda")
    ref = torch.zeros((n_rows, 64), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(n_rows, dtype=torch.float32, device="cuda")
    nl.nested_kv_write(d(xb.view(np.int16)), len(rows), d(np.asarray(rows, np.int32)), base, ref, sc)
    return base, ref, sc


def test_write_matches_oracle(nl, torch_cuda):
    rng = np.random.default_rng(1)
    n = 1000
    xb = vectors(rng, n)
    xf = kv.bf16_to_f32(xb).reshape(n, 128)
    xb = xb.reshape(n, 128)
    xb[0] = 0                                          # zero vector
    xb[1] = synth.f32_to_bf16_bits(xf[1] * 1e-30)      # tiny
    xb[2] = synth.f32_to_bf16_bits(xf[2] * 1e30)       # huge
    rows = rng.permutation(1200)[:n]                   # scattered destinations
    base, ref, sc = write(nl, torch_cuda, xb, rows, 1200)
    q4, qr, s = kv.quantize(xb)
    np.testing.assert_array_equal(base.cpu().numpy()[rows], synth.pack_nibbles(q4))
    np.testing.assert_array_equal(ref.cpu().numpy()[rows], synth.pack_nibbles(qr))
    np.testing.assert_array_equal(sc.cpu().numpy()[rows], s)


# (T, H_q, H_kv, L): a single row; GQA with a ragged sub-chunk; the 8B-class
# heads; 256 query rows per KV head (four row blocks); 80 rows (a partial
# second row block); positions ending exactly on a sub-chunk boundary; a
# context that spans several 64-key sub-chunks per workgroup; 32 rows (two of
# the four waves of a row block hold live rows)
CASES = [(1, 8, 8, 0), (5, 6, 2, 64), (16, 32, 8, 1000), (64, 4, 1, 300), (16, 32, 8, 4096), (3, 2, 2, 127),
         (20, 8, 2, 777), (16, 4, 4, 2032), (2, 4, 1, 9000), (8, 12, 3, 500)]


@pytest.mark.parametrize("T,H_q,H_kv,L", CASES, ids=[f"T{a}-Hq{b}-Hkv{c}-L{d}" for a, b, c, d in CASES])
def test_attention_matches_oracle(nl, torch_cuda, T, H_q, H_kv, L):
    rng = np.random.default_rng(T * 1000 + L)
    P = L + T
    kx, vx = vectors(rng, P * H_kv), vectors(rng, P * H_kv, spread=False)
    q = vectors(rng, T * H_q).reshape(T, H_q, 128)
    anc = tree.build(synth.make_rank_stats(8, 4, cfg=T), T)["anc"]
    assert len(anc) == T
    kb, kr, ks = write(nl, torch_cuda, kx, np.arange(P * H_kv), P * H_kv)
    vb, vr, vs = write(nl, torch_cuda, vx, np.arange(P * H_kv), P * H_kv)
    d = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = torch_cuda.empty(nl.nested_kv_attention_workspace_bytes(T, H_q, H_kv, L), dtype=torch_cuda.uint8,
                          device="cuda")
    out = torch_cuda.empty((T, H_q, 128), dtype=torch_cuda.float32, device="cuda")
    qk4, qkr, sk = kv.quantize(kx)
    qv4, qvr, sv = kv.quantize(vx)
    for verify in (True, False):
        nl.nested_kv_attention(d(q.view(np.int16)), T, H_q, H_kv, L, kb, kr, ks, vb, vr, vs,
                               d(anc.view(np.int64)), verify, out, ws)
        got = out.cpu().numpy().astype(np.float64)
        kh = kv.dequant(qk4, qkr, sk, verify).reshape(P, H_kv, 128)
        vh = kv.dequant(qv4, qvr, sv, verify).reshape(P, H_kv, 128)
        want = kv.attention(q, kh, vh, L, anc, H_kv)
        assert np.isfinite(got).all()
        err = np.abs(got - want).max() / np.abs(vh).max()
        assert err <= TOL, (verify, err)


def test_draft_reads_no_refinement(nl, torch_cuda):
    # KV4 attention must not depend on the refinement planes: pass none
    rng = np.random.default_rng(9)
    T, H_q, H_kv, L = 4, 4, 2, 50
    P = L + T
    kx, vx = vectors(rng, P * H_kv), vectors(rng, P * H_kv)
    q = vectors(rng, T * H_q).reshape(T, H_q, 128)
    anc = tree.build(synth.make_rank_stats(8, 4, cfg=9), T)["anc"]
    kb, _, ks = write(nl, torch_cuda, kx, np.arange(P * H_kv), P * H_kv)
    vb, _, vs = write(nl, torch_cuda, vx, np.arange(P * H_kv), P * H_kv)
    d = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = torch_cuda.empty(nl.nested_kv_attention_workspace_bytes(T, H_q, H_kv, L), dtype=torch_cuda.uint8,
                          device="cuda")
    out = torch_cuda.empty((T, H_q, 128), dtype=torch_cuda.float32, device="cuda")
    nl.nested_kv_attention(d(q.view(np.int16)), T, H_q, H_kv, L, kb, None, ks, vb, None, vs, d(anc.view(np.int64)),
                           False, out, ws)
    qk4, qkr, sk = kv.quantize(kx)
    qv4, qvr, sv = kv.quantize(vx)
    want = kv.attention(q, kv.dequant(qk4, qkr, sk, False).reshape(P, H_kv, 128),
                        kv.dequant(qv4, qvr, sv, False).reshape(P, H_kv, 128), L, anc, H_kv)
    assert np.abs(out.cpu().numpy() - want).max() <= TOL * np.abs(want).max() * 4
    with pytest.raises(nl.NLError):
        nl.nested_kv_attention(d(q.view(np.int16)), T, H_q, H_kv, L, kb, None, ks, vb, None, vs,
                               d(anc.view(np.int64)), True, out, ws)


def test_attention_scale_extremes(nl, torch_cuda):
    # V scales spread over ~e^+-6 and zero K and V vectors: the kernel's
    # per-sub-chunk V-scale normalisation and its zero-scale guards
    rng = np.random.default_rng(17)
    T, H_q, H_kv, L = 16, 8, 2, 700
    P = L + T
    kx = vectors(rng, P * H_kv).reshape(P * H_kv, 128)
    vx = synth.f32_to_bf16_bits(rng.standard_normal((P * H_kv, 128)).astype(np.float32)
                                * np.exp(rng.normal(0, 2.0, (P * H_kv, 1))).astype(np.float32))
    kx[rng.choice(P * H_kv, 40, replace=False)] = 0
    vx[rng.choice(P * H_kv, 40, replace=False)] = 0
    vx[2 * 64 * H_kv:3 * 64 * H_kv] = 0                 # a whole sub-chunk of zero values
    q = vectors(rng, T * H_q).reshape(T, H_q, 128)
    anc = tree.build(synth.make_rank_stats(8, 4, cfg=17), T)["anc"]
    kb, kr, ks = write(nl, torch_cuda, kx, np.arange(P * H_kv), P * H_kv)
    vb, vr, vs = write(nl, torch_cuda, vx, np.arange(P * H_kv), P * H_kv)
    d = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = torch_cuda.empty(nl.nested_kv_attention_workspace_bytes(T, H_q, H_kv, L), dtype=torch_cuda.uint8,
                          device="cuda")
    out = torch_cuda.empty((T, H_q, 128), dtype=torch_cuda.float32, device="cuda")
    qk4, qkr, sk = kv.quantize(kx)
    qv4, qvr, sv = kv.quantize(vx)
    for verify in (True, False):
        nl.nested_kv_attention(d(q.view(np.int16)), T, H_q, H_kv, L, kb, kr, ks, vb, vr, vs,
                               d(anc.view(np.int64)), verify, out, ws)
        got = out.cpu().numpy().astype(np.float64)
        kh = kv.dequant(qk4, qkr, sk, verify).reshape(P, H_kv, 128)
        vh = kv.dequant(qv4, qvr, sv, verify).reshape(P, H_kv, 128)
        want = kv.attention(q, kh, vh, L, anc, H_kv)
        assert np.isfinite(got).all()
        # each output is held to the largest |v_hat| of its own KV head
        for h in range(H_kv):
            js = slice(h * (H_q // H_kv), (h + 1) * (H_q // H_kv))
            err = np.abs(got[:, js] - want[:, js]).max() / np.abs(vh[:, h]).max()
            assert err <= TOL, (verify, h, err)
