"""fp64 CPU oracle of the BitNest W4/W8 dual-plane linear.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product package never does.

Source: "BitNest: Bit-Nested Speculative Decoding for Memory-Efficient LLM
Inference Acceleration" (page 2 of the source pages):
  section 3.2 / appendix A.1, eq. 5-6   W4 base: q4 in [-8, 7] with a scale s4
                                        per 128-weight group, W_draft = q4 s4;
  eq. 7-9                               refinement of the fixed base: the error
                                        dW = W' - W_draft, s_ref = s4 / 16,
                                        q_r = clip(round(dW / s_ref), lo, 7) with
                                        lo = 0 where q4 = -8, else -8;
  eq. 10                                W_target = q4 s4 + q_r s_ref
                                                 = (16 q4 + q_r) s_ref;
  section 3.3 (dual-plane storage)      base and refinement codes in two
                                        separate 4-bit planes of N/2 bytes.
The rotations the paper folds into W' are part of the weights: the layer
computes y = W x with no online transform.

Readings (listed with the design notes):
  * a plane holds two's-complement nibbles, weight k of a row in byte k/2,
    the low nibble for even k;
  * s4 is an fp16 value per (row, 128-column group); s_ref is not stored;
  * round() in eq. 9 is round-half-even of the fp64 quotient (dW / s_ref,
    with s_ref = s4 / 16 exact), and q_r = 0 where s4 = 0;
  * the W4 base of the tests is round-to-nearest with s4 = fp16(max|W'| / 7)
    (the paper's is GPTQ, which needs calibration data).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def unpack_nibbles(plane: np.ndarray, d_in: int) -> np.ndarray:
    """[d_out][d_in/2] uint8 -> [d_out][d_in] int8 two's-complement values."""
    p = np.asarray(plane, np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    out = np.empty((p.shape[0], d_in), np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out[out >= 8] -= 16
    return out.astype(np.int8)


def dequant(lin: dict, verify: bool, rows=None) -> np.ndarray:
    """W_draft = q4 s4 (eq. 6) or W_target = (16 q4 + q_r) s4 / 16 (eq. 10),
    fp64, for rows [r0, r1)."""
    d_out, d_in = lin["d_out"], lin["d_in"]
    r0, r1 = (0, d_out) if rows is None else rows
    q4 = unpack_nibbles(lin["base_plane"][r0:r1], d_in).astype(np.float64)
    s4 = np.asarray(lin["scales"][r0:r1], np.uint16).view(np.float16).astype(np.float64)
    s = np.repeat(s4, GROUP, axis=1)
    if not verify:
        return q4 * s
    qr = unpack_nibbles(lin["ref_plane"][r0:r1], d_in).astype(np.float64)
    return (16.0 * q4 + qr) * (s / 16.0)


def forward(lin: dict, x_bf16: np.ndarray, verify: bool, rows=None) -> np.ndarray:
    """y[t] = W x[t] for T tokens, x given as bf16 bit patterns; fp64
    [T][rows]."""
    x = (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x @ dequant(lin, verify, rows).T


def rtn_base(W: np.ndarray):
    """Round-to-nearest W4 base: s4 = fp16(max|group| / 7), q4 =
    clip(rint(W / s4), -8, 7) (0 where s4 = 0).  Returns (q4 int8, s4
    float16)."""
    W = np.asarray(W, np.float64)
    d_out, d_in = W.shape
    g = W.reshape(d_out, d_in // GROUP, GROUP)
    s4 = (np.max(np.abs(g), axis=2) / 7.0).astype(np.float16)
    sd = s4.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sd > 0, np.clip(np.rint(g / sd), -8, 7), 0.0)
    return q.astype(np.int8).reshape(d_out, d_in), s4


def refine(W: np.ndarray, q4: np.ndarray, s4: np.ndarray) -> np.ndarray:
    """Eq. 7-9: the 4-bit refinement of a fixed W4 base."""
    W = np.asarray(W, np.float64)
    d_out, d_in = W.shape
    s = np.repeat(np.asarray(s4, np.float16).astype(np.float64), GROUP, axis=1)
    dW = W - q4.astype(np.float64) * s                  # eq. 7
    s_ref = s / 16.0                                    # eq. 8 (exact)
    lo = np.where(q4 == -8, 0.0, -8.0)                  # eq. 9 boundary rule
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s_ref > 0, np.clip(np.rint(dW / s_ref), lo, 7.0), 0.0)
    return q.astype(np.int8)
