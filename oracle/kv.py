"""CPU oracle of the nested KV cache (KV4 base + 4-bit refinement) and of the
tree-masked attention that reads it.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product package never does.

Source: "BitNest: Bit-Nested Speculative Decoding for Memory-Efficient LLM
Inference Acceleration" (page 2 of the source pages), appendix A.2:
  eq. 11  per (token, KV head) vector x of d = 128: s = max|x| / 7,
          q4 = clip(round(x / s), -8, 7);
  eq. 12  x_draft = q4 s (KV4);
  eq. 13  q_r = clip(round((x - q4 s) / (s / 16)), -8, 7);
  eq. 14  x_target = (16 q4 + q_r) s / 16 (KV8);
the draft reads only the base, verification both planes (section 3.4).
The attention is the verify pass's: each draft-tree token attends to the
whole context and to its ancestors in the tree (itself included), the
tree-attention mask of the forum post's POC section 6 tree.

Readings (listed with the design notes):
  * the quantiser runs in fp32 on bf16 inputs: s = fp32(max|x| / 7), the
    quotients are correctly rounded fp32 divisions, round() is
    round-half-even, and the residual x - q4 s is formed exactly and rounded
    once to fp32 (eq. 13 is stated over the reals; forming it exactly is the
    plainest fp32 rendering, and it is what a fused multiply-add computes);
    a zero vector stores s = 0 and zero codes;
  * planes are two's-complement nibbles, dimension k in byte k/2 (low nibble
    for even k), 64 bytes per (position, KV head) row; the scale is fp32;
  * attention scores are q . k_hat / sqrt(d); query head j reads KV head
    j / (H_q / H_kv).
"""
from __future__ import annotations

import numpy as np

D = 128


def bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(x_bf16):
    """Eq. 11-13 on rows of 128 bf16 values.  Returns q4 int8 [n][128],
    q_r int8 [n][128], s float32 [n]."""
    x = bf16_to_f32(x_bf16).reshape(-1, D)
    m = np.max(np.abs(x), axis=1)
    s = (m / np.float32(7.0)).astype(np.float32)
    sc = s[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q4 = np.where(sc > 0, np.clip(np.rint(x / sc), -8, 7), 0).astype(np.float32)
        # exact in fp64 (a 4-bit integer times an fp32 scale, then a difference
        # of nearby values), rounded once to fp32
        r = (x.astype(np.float64) - q4.astype(np.float64) * sc.astype(np.float64)).astype(np.float32)
        qr = np.where(sc > 0, np.clip(np.rint(r / (sc / np.float32(16.0))), -8, 7), 0)
    return q4.astype(np.int8), qr.astype(np.int8), s


def dequant(q4, qr, s, verify: bool):
    """KV4 (eq. 12) or KV8 (eq. 14) in fp64."""
    s = np.asarray(s, np.float32).astype(np.float64)[:, None]
    if verify:
        return (16.0 * q4.astype(np.float64) + qr.astype(np.float64)) * s / 16.0
    return q4.astype(np.float64) * s


def attention(q_bf16, k_hat, v_hat, L: int, anc, H_kv: int):
    """O[t][j] = softmax_over_keys(q[t][j] . k_hat / sqrt(d)) v_hat for T tree
    tokens.  q [T][H_q][128]; k_hat, v_hat [(L + T)][H_kv][128] fp64 (position
    major); key position p < L is context, p = L + i is tree node i, visible
    to token t when bit i of anc[t] is set.  fp64 [T][H_q][128]."""
    q = bf16_to_f32(q_bf16).astype(np.float64)
    T, H_q, _ = q.shape
    g = H_q // H_kv
    out = np.zeros((T, H_q, D))
    for t in range(T):
        vis = np.array([True] * L + [bool((int(anc[t]) >> i) & 1) for i in range(T)])
        for j in range(H_q):
            h = j // g
            sc = k_hat[:, h, :] @ q[t, j] / np.sqrt(D)
            sc = np.where(vis, sc, -np.inf)
            w = np.exp(sc - sc.max())
            w /= w.sum()
            out[t, j] = w @ v_hat[:, h, :]
    return out
