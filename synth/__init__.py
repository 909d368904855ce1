"""Seeded synthetic inputs for the bit-nested quantized linear.

This module only draws random numbers and lays them out in the canonical
storage format that the C-ABI and the oracle both accept.  It holds none of
the method's arithmetic (no rotation, no dequantisation, no contraction):
both the oracle and the HIP path consume what it produces.

Canonical storage format (per linear, W is d_out x d_in, G = ceil(d_in/128)
groups of 128 consecutive input columns per output row; the "bit-nested"
forum post, POC recipe sections 2 and 3):

* base_codes  uint8 [d_out][G][32]: two bit-planes of 16 bytes each.  Bytes
  0..15 hold bit 0 of every 2-bit code, bytes 16..31 bit 1.  Code j of the
  group sits at bit (j & 7) of byte (j >> 3) of each plane (LSB first).
  Code c selects levels[c]; levels are ascending.
* base_scales uint16 [d_out][G]: IEEE fp16 bit patterns.
* resid_codes uint8 [d_out][G][16*b]: the group's 128 b-bit two's-complement
  fields, field j at bits [j*b, (j+1)*b) of the group's little-endian bit
  string.
* resid_scales uint16 [d_out][G]: fp16 bit patterns.
* sign_in int8 [d_in], sign_out int8 [d_out] (or None): +-1.
* x uint16 [T][d_in]: bf16 bit patterns.

A ragged last group (d_in not a multiple of 128; only the oracle accepts it)
keeps the full-size byte block with the unused fields zero.

Seeds: every array is a pure function of SeedSequence([20261008, cfg,
linear_idx, stream]) with numpy's PCG64, so the host regenerates one linear
at a time.  Stream ids: 0 sign_in, 1 sign_out, 2 base codes, 3 base scales,
4 residual codes, 5 residual scales, 6 x, 7 router logits, 8 dense weights
(the encoder's input), 9-11 the W4 codes, refinement codes and scales of the
W4/W8 dual-plane format, 12-13 draft-tree rank statistics and tokens.
"""
from __future__ import annotations

import sys

import numpy as np

SEED0 = 20261008
GROUP = 128

# The four base levels of the synthetic workloads: the Gaussian 4-level
# Lloyd-Max quantiser, as fitted in the forum post's POC section 2 (its
# fitted values are within 0.5% of these).
LEVELS = np.array([-1.5104, -0.4528, 0.4528, 1.5104], dtype=np.float32)

STREAM_SIGN_IN, STREAM_SIGN_OUT, STREAM_BASE, STREAM_BASE_SCALE = 0, 1, 2, 3
STREAM_RESID, STREAM_RESID_SCALE, STREAM_X, STREAM_ROUTER = 4, 5, 6, 7
STREAM_DENSE = 8
STREAM_W4, STREAM_W4_REF, STREAM_W4_SCALE = 9, 10, 11
STREAM_TREE = 12


def rng(cfg: int, linear_idx: int, stream: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED0, cfg, linear_idx, stream])))


def groups(d_in: int) -> int:
    return (d_in + GROUP - 1) // GROUP


def qmax(bits: int) -> int:
    return (1 << (bits - 1)) - 1


def resid_sigma(bits: int) -> float:
    """Spread of the synthetic residual codes: N(0, 20) for 8-bit, scaled by
    qm/127 for narrower grids, so every width uses the same share of its
    range."""
    return 20.0 * qmax(bits) / 127.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def _pad_cols(a: np.ndarray, d_in: int) -> np.ndarray:
    g = groups(d_in)
    if g * GROUP == d_in:
        return a
    out = np.zeros(a.shape[:-1] + (g * GROUP,), dtype=a.dtype)
    out[..., :d_in] = a
    return out


def pack_base(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [d_out][d_in] in 0..3 -> canonical [d_out][G][32] bytes."""
    d_out, d_in = codes.shape
    c = _pad_cols(codes.astype(np.uint8), d_in).reshape(d_out, groups(d_in), GROUP)
    p0 = np.packbits(c & 1, axis=-1, bitorder="little")          # [d_out][G][16]
    p1 = np.packbits((c >> 1) & 1, axis=-1, bitorder="little")
    return np.ascontiguousarray(np.concatenate([p0, p1], axis=-1))


def pack_resid(q: np.ndarray, bits: int) -> np.ndarray:
    """q int [d_out][d_in] in [-2^(b-1), 2^(b-1)-1] -> canonical
    [d_out][G][16*b] bytes of LSB-first b-bit two's-complement fields.

    Eight consecutive fields fill exactly b bytes: they are combined into one
    little-endian 64-bit word whose low b bytes are the packed bytes."""
    assert sys.byteorder == "little"
    d_out, d_in = q.shape
    g = groups(d_in)
    u = _pad_cols(q.astype(np.int64), d_in).reshape(d_out, g, GROUP // 8, 8)
    u = (u & ((1 << bits) - 1)).astype(np.uint64)
    w = np.zeros(u.shape[:-1], np.uint64)
    for i in range(8):
        w |= u[..., i] << np.uint64(bits * i)
    by = w[..., None].view(np.uint8).reshape(d_out, g, GROUP // 8, 8)[..., :bits]
    return np.ascontiguousarray(by.reshape(d_out, g, 16 * bits))


def make_signs(n: int, cfg: int, idx: int, stream: int) -> np.ndarray:
    return (rng(cfg, idx, stream).integers(0, 2, size=n, dtype=np.int8) * 2 - 1).astype(np.int8)


def make_scales(d_out: int, d_in: int, cfg: int, idx: int, stream: int,
                lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    s = rng(cfg, idx, stream).uniform(lo, hi, size=(d_out, groups(d_in)))
    return np.ascontiguousarray(s.astype(np.float16).view(np.uint16))


def make_base_codes(d_out: int, d_in: int, cfg: int, idx: int) -> np.ndarray:
    return rng(cfg, idx, STREAM_BASE).integers(0, 4, size=(d_out, d_in), dtype=np.uint8)


def make_resid_codes(d_out: int, d_in: int, bits: int, cfg: int, idx: int) -> np.ndarray:
    """clip(rint(N(0, sigma_b))) drawn row-major; in row blocks (the same
    stream as one draw) so the float temporaries stay small."""
    qm = qmax(bits)
    g = rng(cfg, idx, STREAM_RESID)
    out = np.empty((d_out, d_in), np.int8)
    for r in range(0, d_out, 4096):
        v = g.normal(0.0, resid_sigma(bits), size=(min(4096, d_out - r), d_in))
        out[r:r + v.shape[0]] = np.clip(np.rint(v), -qm, qm)
    return out


def make_dense_weights(d_out: int, d_in: int, cfg: int = 0, idx: int = 0, sigma: float = 0.02,
                       outlier_frac: float = 0.01, outlier_gain: float = 8.0) -> np.ndarray:
    """A dense fp32 weight matrix [d_out][d_in] shaped like a trained
    Linear's: N(0, sigma^2) entries, a lognormal gain per output row (log-sd
    0.3) and a few input columns (outlier_frac of them, at least one) scaled
    by outlier_gain, the outlier channels the rotation is meant to spread.
    Drawn in row blocks of 4096 from one stream."""
    g = rng(cfg, idx, STREAM_DENSE)
    row_gain = np.exp(g.normal(0.0, 0.3, size=d_out)) * sigma
    col_gain = np.ones(d_in)
    col_gain[g.choice(d_in, max(1, int(d_in * outlier_frac)), replace=False)] = outlier_gain
    out = np.empty((d_out, d_in), np.float32)
    for r in range(0, d_out, 4096):
        n = min(4096, d_out - r)
        z = g.standard_normal(size=(n, d_in), dtype=np.float32)
        out[r:r + n] = z * row_gain[r:r + n, None].astype(np.float32) * col_gain[None, :].astype(np.float32)
    return out


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """[d_out][d_in] values in [-8, 7] -> [d_out][d_in/2] uint8 of
    two's-complement nibbles, weight 2i in the low nibble of byte i."""
    u = (np.asarray(q, np.int16) & 0x0F).astype(np.uint8)
    return np.ascontiguousarray(u[:, 0::2] | (u[:, 1::2] << 4))


def make_w4w8_linear(d_out: int, d_in: int, cfg: int = 0, idx: int = 0, keep_codes: bool = False) -> dict:
    """One synthetic BitNest W4/W8 linear (page 2, section 3.3 dual planes):
    base codes clip(rint(N(0, 3^2)), -8, 7), refinement codes uniform in
    [-8, 7] except [0, 7] where the base code is -8 (the boundary rule of
    eq. 9), fp16 scales U(0.005, 0.02) per (row, 128-group)."""
    assert d_in % GROUP == 0 and d_in % 2 == 0
    q4 = np.clip(np.rint(rng(cfg, idx, STREAM_W4).normal(0.0, 3.0, size=(d_out, d_in))), -8, 7).astype(np.int8)
    qr = rng(cfg, idx, STREAM_W4_REF).integers(-8, 8, size=(d_out, d_in), dtype=np.int8)
    qr = np.where(q4 == -8, np.abs(qr) % 8, qr).astype(np.int8)
    lin = {"d_out": d_out, "d_in": d_in, "base_plane": pack_nibbles(q4), "ref_plane": pack_nibbles(qr),
           "scales": make_scales(d_out, d_in, cfg, idx, STREAM_W4_SCALE)}
    if keep_codes:
        lin["q4"], lin["qr"] = q4, qr
    return lin


def make_rank_stats(D: int = 8, R: int = 16, cfg: int = 0, idx: int = 0) -> np.ndarray:
    """Synthetic rank statistics p[D][R]: at depth d the verifier's token has
    draft rank r with probability proportional to exp(-r / tau_d) (tau
    shrinking with depth: the draft gets worse further out), scaled by a
    per-depth acceptance mass a_d decaying from 0.8; rows sum to a_d <= 1.
    A little noise keeps products distinct."""
    g = rng(cfg, idx, STREAM_TREE)
    out = np.zeros((D, R))
    for d in range(D):
        tau = 1.5 / (1.0 + 0.25 * d)
        w = np.exp(-np.arange(R) / tau) * g.uniform(0.9, 1.1, R)
        out[d] = 0.8 * (0.95 ** d) * w / w.sum()
    return out


def make_tree_tokens(parent: np.ndarray, B: int, vocab: int = 32000, p_match: float = 0.7, cfg: int = 0,
                     idx: int = 0):
    """Draft tokens of a tree's nodes for B sequences (siblings distinct) and
    the verifier's argmax after the root and after each node: with
    probability p_match the argmax is the token of one of the node's
    children (if it has any), else a token no child carries."""
    g = rng(cfg, idx, STREAM_TREE + 1)
    N = len(parent)
    draft = np.zeros((B, N), np.int32)
    argmax = np.zeros((B, N + 1), np.int32)
    kids = [[c for c in range(N) if parent[c] == u] for u in range(-1, N)]
    for b in range(B):
        for u in range(-1, N):
            ks = kids[u + 1]
            toks = g.choice(vocab - 1, size=len(ks) + 1, replace=False).astype(np.int32)
            for c, tkn in zip(ks, toks[:-1]):
                draft[b, c] = tkn
            if ks and g.random() < p_match:
                argmax[b, u + 1] = draft[b, ks[g.integers(len(ks))]]
            else:
                argmax[b, u + 1] = toks[-1]
    return draft, argmax


def make_linear(d_out: int, d_in: int, bits: int, cfg: int = 0, idx: int = 0,
                two_sided: bool = True, keep_codes: bool = False) -> dict:
    """One synthetic nested linear in the canonical format.

    bits = 0 gives a draft-only linear (no residual arrays)."""
    lin = {
        "d_out": d_out, "d_in": d_in, "bits": bits,
        "levels": LEVELS.copy(),
        "sign_in": make_signs(d_in, cfg, idx, STREAM_SIGN_IN),
        "sign_out": make_signs(d_out, cfg, idx, STREAM_SIGN_OUT) if two_sided else None,
    }
    codes = make_base_codes(d_out, d_in, cfg, idx)
    lin["base_codes"] = pack_base(codes)
    lin["base_scales"] = make_scales(d_out, d_in, cfg, idx, STREAM_BASE_SCALE)
    if keep_codes:
        lin["base_idx"] = codes
    if bits:
        q = make_resid_codes(d_out, d_in, bits, cfg, idx)
        lin["resid_codes"] = pack_resid(q, bits)
        lin["resid_scales"] = make_scales(d_out, d_in, cfg, idx, STREAM_RESID_SCALE)
        if keep_codes:
            lin["resid_q"] = q
    else:
        lin["resid_codes"] = None
        lin["resid_scales"] = None
    return lin


def make_x(T: int, d_in: int, cfg: int = 0, idx: int = 0, scale: float = 1.0) -> np.ndarray:
    """bf16 activations N(0, scale^2) as uint16 bit patterns [T][d_in]."""
    v = rng(cfg, idx, STREAM_X).standard_normal(size=(T, d_in)).astype(np.float32) * scale
    return f32_to_bf16_bits(v)


def router_topk(T: int, n_experts: int, k: int, rho: float, cfg: int = 4, idx: int = 0):
    """Router logits for a block of T tokens: every logit is marginally N(0,1);
    tokens of the block share a common component with correlation rho
    (rho = 0 is iid routing).  Returns (experts [T][k] int32, sorted pairs).

    The pairs are (token, expert) sorted by expert, then token; returns
    pair_token int32 [P], expert_offsets int32 [n_experts+1]."""
    r = rng(cfg, idx, STREAM_ROUTER)
    g = r.standard_normal(n_experts)
    z = r.standard_normal((T, n_experts))
    logits = np.sqrt(rho) * g[None, :] + np.sqrt(1.0 - rho) * z
    top = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    pairs = sorted((int(e), t) for t in range(T) for e in top[t])
    pair_token = np.array([t for _, t in pairs], dtype=np.int32)
    counts = np.bincount(np.array([e for e, _ in pairs], dtype=np.int64), minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return top, pair_token, offsets


def bytes_per_weight(bits: int) -> float:
    """Streamed bytes per weight of one pass: codes plus fp16 group scales."""
    b = (2 * GROUP + 16) / 8 / GROUP            # 2-bit base + fp16 scale
    if bits:
        b += (bits * GROUP + 16) / 8 / GROUP
    return b
