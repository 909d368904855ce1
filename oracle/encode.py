"""fp64 CPU oracle of the round-to-nearest encoder and the Lloyd-Max level
fitter: the offline step that turns a dense W into the canonical planes.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product package never does.

Everything follows the forum post "bit-nested" (page 1 of the source pages),
POC recipe:
  section 1  W~ = H_o S_o W S_i H_i, block-diagonal normalised Hadamard;
  section 2  base scale = RMS of the (row, 128-group) block rounded to fp16,
             code = nearest of 4 Lloyd-Max levels times that scale; levels
             fitted on RMS-normalised rotated weights from the quantiles
             0.125/0.375/0.625/0.875, 60 Lloyd iterations, then symmetrised;
  section 3  R~ = W~ - Q_base on an evenly spaced b-bit grid centred on 0,
             levels -qm..qm,
             qm = 2^(b-1) - 1, scale = max|block| / qm in fp16.
GPTQ/LDLQ (the post's calibrated variant of sections 2-3) needs calibration
data and is not modelled: this is the plain round-to-nearest quantiser.

Readings of points the post leaves open (each is a choice, listed with the
design notes):
  * rounding to fp16 is round-to-nearest-even straight from fp64; a value
    beyond the fp16 range saturates to 65504;
  * "nearest" is decided exactly: the boundary between two reconstruction
    points is their midpoint, computed without rounding in fp64 (products of
    an fp32 level and an fp16 scale are exact and so is their sum for levels
    within a factor 2^17 of each other); a value on a boundary takes the
    level of smaller magnitude, and of two equal magnitudes the larger level;
    a zero scale makes every point 0, so the same rule picks the code;
  * the residual integer is round-half-even of R~/s, clamped to [-qm, qm];
    a zero residual scale gives zeros;
  * a quantile is the linear interpolation between order statistics at
    position q (n - 1) (numpy's and torch's default);
  * a Lloyd cell with no samples keeps its level;
  * "symmetrise" is the closest symmetric set: a0 = (l2 - l1)/2,
    a1 = (l3 - l0)/2, levels (-a1, -a0, a0, a1);
  * the fitter's samples are rotated weights divided by their group's fp16
    scale (the normalisation the codes see); a group with a zero scale gives
    zeros.
"""
from __future__ import annotations

import numpy as np

from . import fwht

GROUP = 128
F16_MAX = 65504.0
QUANTILES = (0.125, 0.375, 0.625, 0.875)


def rot_fwd(W, sign_in, sign_out=None) -> np.ndarray:
    """W~ = H_o S_o W S_i H_i in fp64 (POC section 1, "Rotation"):
    the input side first (each row times S_i, then the block Hadamard along
    d_in), then, in the two-sided form, the output side (each row times its
    S_o sign, then the block Hadamard along d_out)."""
    W = np.asarray(W, np.float64)
    Wt = fwht(W * np.asarray(sign_in, np.float64)[None, :])
    if sign_out is not None:
        Wt = fwht((Wt * np.asarray(sign_out, np.float64)[:, None]).T).T
    return np.ascontiguousarray(Wt)


def rot_inv(Wt, sign_in, sign_out=None) -> np.ndarray:
    """W = S_o H_o W~ H_i S_i (POC section 1, the exact inverse): H is its own
    inverse, so the Hadamards are applied again and the signs after them."""
    X = np.asarray(Wt, np.float64)
    if sign_out is not None:
        X = fwht(X.T).T * np.asarray(sign_out, np.float64)[:, None]
    return fwht(X) * np.asarray(sign_in, np.float64)[None, :]


def to_f16(x) -> np.ndarray:
    """Round fp64 values to fp16 (nearest, ties to even), saturating at
    +-65504.  Returns float16."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    over = np.isinf(h) & np.isfinite(x)
    return np.where(over, np.copysign(np.float16(F16_MAX), x).astype(np.float16), h)


def _groups(A: np.ndarray) -> np.ndarray:
    d_out, d_in = A.shape
    assert d_in % GROUP == 0
    return A.reshape(d_out, d_in // GROUP, GROUP)


def base_scales(Wt) -> np.ndarray:
    """Per (row, 128-group) scale: sqrt(mean of squares), rounded to fp16
    (POC section 2, "Scale").  float16 [d_out][G]."""
    g = _groups(np.asarray(Wt, np.float64))
    return to_f16(np.sqrt(np.sum(g * g, axis=2) / GROUP))


def _tie_up(levels: np.ndarray) -> np.ndarray:
    """For each boundary k (between levels k and k+1): True if a value on it
    goes to level k+1 (|l_{k+1}| <= |l_k|)."""
    return np.abs(levels[1:]) <= np.abs(levels[:-1])


def nearest_codes(Wt, scales, levels) -> np.ndarray:
    """Index of the nearest reconstruction point levels[c] * scale for every
    weight (POC section 2, "Codes"); uint8 [d_out][d_in].  levels: 4
    ascending fp32 values."""
    L = np.asarray(levels, np.float32).astype(np.float64)
    assert L.shape == (4,) and np.all(np.diff(L) > 0)
    g = _groups(np.asarray(Wt, np.float64))
    s = np.asarray(scales, np.float16).astype(np.float64)[:, :, None]
    up = _tie_up(L)
    codes = np.zeros(g.shape, np.uint8)
    for k in range(3):
        mid = (L[k] * s + L[k + 1] * s) * 0.5
        codes += ((g > mid) | ((g == mid) & up[k])).astype(np.uint8)
    # zero scale: every point is 0, the boundary rule picks the smallest |level|
    zero = np.broadcast_to(s == 0.0, g.shape)
    order = sorted(range(4), key=lambda c: (abs(L[c]), -c))
    codes[zero] = order[0]
    return codes.reshape(np.asarray(Wt).shape)


def qmax(bits: int) -> int:
    return (1 << (bits - 1)) - 1


def residual(Wt, codes, scales, levels) -> np.ndarray:
    """R~ = W~ - Q_base in fp64 (POC section 3)."""
    L = np.asarray(levels, np.float32).astype(np.float64)
    g = _groups(np.asarray(Wt, np.float64))
    s = np.asarray(scales, np.float16).astype(np.float64)[:, :, None]
    return (g - L[_groups(np.asarray(codes))] * s).reshape(np.asarray(Wt).shape)


def residual_quantize(R, bits: int):
    """Uniform symmetric b-bit quantiser (POC section 3): scale = max|block|
    / qm in fp16, integer = round(R/scale) clamped to [-qm, qm].  Returns
    (int8 [d_out][d_in], float16 [d_out][G])."""
    qm = qmax(bits)
    g = _groups(np.asarray(R, np.float64))
    s = to_f16(np.max(np.abs(g), axis=2) / qm)
    sd = s.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sd > 0, np.clip(np.rint(g / sd), -qm, qm), 0.0)
    return q.astype(np.int8).reshape(np.asarray(R).shape), s


def quantize_rotated(Wt, bits: int, levels) -> dict:
    """Codes and scales of a rotated weight matrix (POC sections 2-3).
    Returns base_idx uint8 [d_out][d_in], base_scales fp16 bits, and for
    bits > 0 resid int8 [d_out][d_in] and resid_scales fp16 bits."""
    Wt = np.asarray(Wt, np.float64)
    s = base_scales(Wt)
    c = nearest_codes(Wt, s, levels)
    out = {"base_idx": c, "base_scales": s.view(np.uint16)}
    if bits:
        q, rs = residual_quantize(residual(Wt, c, s, levels), bits)
        out["resid"] = q
        out["resid_scales"] = rs.view(np.uint16)
    return out


def encode(W, sign_in, sign_out, bits: int, levels) -> dict:
    """The whole round-to-nearest encoder: rotate (section 1), then quantise
    (sections 2-3)."""
    return quantize_rotated(rot_fwd(W, sign_in, sign_out), bits, levels)


def normalized(Wt) -> np.ndarray:
    """Rotated weights divided by their group's fp16 scale (the fitter's
    samples, POC section 2); zeros where the scale is 0."""
    g = _groups(np.asarray(Wt, np.float64))
    s = base_scales(Wt).astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, g / s, 0.0)
    return v.reshape(np.asarray(Wt).shape)


def quantile_start(v) -> np.ndarray:
    """The four starting levels: order statistics of the sorted sample,
    linearly interpolated at position q (n - 1) for q in 0.125, 0.375,
    0.625, 0.875 (POC section 2)."""
    x = np.sort(np.asarray(v, np.float64).ravel())
    n = x.size
    assert n >= 1
    out = np.zeros(4)
    for i, q in enumerate(QUANTILES):
        pos = q * (n - 1)
        lo = int(np.floor(pos))
        hi = min(lo + 1, n - 1)
        t = pos - lo
        out[i] = x[lo] + (x[hi] - x[lo]) * t
    return out


def assign_cells(v, L) -> np.ndarray:
    """Nearest of four ascending levels for every sample; a sample on a
    midpoint goes to the level of smaller magnitude (the larger level if the
    magnitudes are equal)."""
    v = np.asarray(v, np.float64).ravel()
    up = _tie_up(np.asarray(L, np.float64))
    c = np.zeros(v.size, np.int64)
    for k in range(3):
        mid = (L[k] + L[k + 1]) * 0.5
        c += (v > mid) | ((v == mid) & up[k])
    return c


def lloyd_max_fit(v, iters: int = 60, symmetrize: bool = True) -> np.ndarray:
    """Four-level Lloyd-Max quantiser of the sample v (POC section 2): start
    at the quantiles, then `iters` times move every level to the mean of the
    samples nearest to it; finally symmetrise.  fp64 levels, ascending."""
    v = np.asarray(v, np.float64).ravel()
    L = quantile_start(v)
    for _ in range(iters):
        c = assign_cells(v, L)
        for k in range(4):
            m = c == k
            cnt = int(np.count_nonzero(m))
            if cnt:
                L[k] = np.sum(v[m]) / cnt
    if symmetrize:
        a0 = (L[2] - L[1]) * 0.5
        a1 = (L[3] - L[0]) * 0.5
        L = np.array([-a1, -a0, a0, a1])
    return L
