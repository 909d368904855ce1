"""Pins of the encoder oracle (oracle/encode.py) to what the forum post and the
mathematics fix, independent of the oracle's own formulas: a dense Sylvester
product for the rotation, exact rational arithmetic for fp16 rounding and for
"nearest level", closed forms of the RMS and of the uniform quantiser's error,
the textbook Gaussian 4-level Lloyd-Max quantiser (levels and distortion),
numpy's quantile, a four-cluster sample with a known fixed point, and a round
trip through the pinned decoder of the canonical planes.
"""
from bisect import bisect_left
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import encode as enc

LEV = synth.LEVELS


def sylvester(b: int) -> np.ndarray:
    H = np.ones((1, 1))
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(b)


def block_h(n: int, b: int) -> np.ndarray:
    H = np.zeros((n, n))
    for s in range(0, n, b):
        H[s:s + b, s:s + b] = sylvester(b)
    return H


# --- rotation (POC section 1) -------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,two", [(96, 640, True), (8, 4096, False), (256, 384, True)])
def test_rot_fwd_equals_dense_product(orc, d_out, d_in, two):
    # W~ = H_o S_o W S_i H_i with H grown by the Sylvester recursion and the
    # block sizes of the block-size rule (640 -> 128, 96 -> 32, 384 -> 128).
    rng = np.random.default_rng(d_out + d_in)
    W = rng.standard_normal((d_out, d_in))
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8) if two else None
    ref = W @ np.diag(si.astype(float)) @ block_h(d_in, orc.block_size(d_in)).T
    if two:
        ref = block_h(d_out, orc.block_size(d_out)) @ np.diag(so.astype(float)) @ ref
    np.testing.assert_allclose(enc.rot_fwd(W, si, so), ref, rtol=0, atol=1e-12)


def test_rot_inv_undoes_rot_fwd():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((160, 1536))           # blocks 32 and 512
    si = rng.choice([-1, 1], 1536).astype(np.int8)
    so = rng.choice([-1, 1], 160).astype(np.int8)
    np.testing.assert_allclose(enc.rot_inv(enc.rot_fwd(W, si, so), si, so), W, rtol=0, atol=1e-12)
    np.testing.assert_allclose(enc.rot_inv(enc.rot_fwd(W, si), si), W, rtol=0, atol=1e-12)


# --- fp16 rounding ------------------------------------------------------------------

def _f16_table():
    pats = np.arange(0, 0x7C00, dtype=np.uint16)           # +0 .. largest finite
    vals = pats.view(np.float16).astype(np.float64)
    return [Fraction(float(v)) for v in vals], pats


def test_to_f16_is_nearest_even_in_exact_arithmetic():
    fr, pats = _f16_table()
    rng = np.random.default_rng(2)
    x = np.concatenate([np.exp(rng.uniform(np.log(2.0 ** -27), np.log(7e4), 4000)),
                        # exact midpoints between neighbouring fp16 values
                        [float((fr[i] + fr[i + 1]) / 2) for i in rng.integers(1, len(fr) - 1, 300)]])
    got = enc.to_f16(x).view(np.uint16)
    for xi, g in zip(x, got):
        X = Fraction(float(xi))
        if X >= fr[-1] + (fr[-1] - fr[-2]) / 2:
            assert g == 0x7BFF                               # saturates
            continue
        i = bisect_left(fr, X)
        if i < len(fr) and fr[i] == X:
            assert g == pats[i]
            continue
        lo, hi = i - 1, i
        dl, dh = X - fr[lo], fr[hi] - X
        want = lo if dl < dh else hi if dh < dl else (lo if pats[lo] % 2 == 0 else hi)
        assert g == pats[want], (xi, g, pats[want])


# --- base quantiser (POC section 2) ------------------------------------------

def test_scale_of_constant_and_two_valued_groups():
    # RMS of 128 copies of c is |c|; of 64 (+a) and 64 (-a) it is a.
    c = np.array([0.013, -0.0071, 3.0, 1e-6])
    W = np.repeat(c[:, None], 128, axis=1)
    np.testing.assert_array_equal(enc.base_scales(W)[:, 0], enc.to_f16(np.abs(c)))
    a = 0.02718
    W2 = np.tile(np.r_[np.full(64, a), np.full(64, -a)], (1, 1))
    assert enc.base_scales(W2)[0, 0] == enc.to_f16(a)


def test_scale_is_fp16_of_exact_rms():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((6, 384)) * 0.02
    s = enc.base_scales(W)
    fr, _ = _f16_table()
    for r in range(6):
        for g in range(3):
            ss = sum(Fraction(float(v)) ** 2 for v in W[r, 128 * g:128 * (g + 1)])
            rms2 = ss / 128
            h = Fraction(float(s[r, g]))
            i = fr.index(h)
            # rms lies within half an fp16 step of the scale: compare squares exactly
            lo, hi = (fr[i - 1] + h) / 2, (h + fr[i + 1]) / 2
            assert lo * lo <= rms2 <= hi * hi


def _nearest_exact(w, s, levels):
    """Brute force over the 4 points with exact rational distances; a tie
    goes to the smaller |level|, then the larger level."""
    W = Fraction(float(w))
    S = Fraction(float(s))
    best = None
    for c in range(4):
        L = Fraction(float(levels[c]))
        key = (abs(W - L * S), abs(L), -c)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_nearest_codes_brute_force_exact():
    rng = np.random.default_rng(4)
    Wt = rng.standard_normal((4, 256)) * 0.01
    s = enc.base_scales(Wt)
    codes = enc.nearest_codes(Wt, s, LEV)
    for r in range(4):
        for k in range(256):
            assert codes[r, k] == _nearest_exact(Wt[r, k], s[r, k // 128], LEV)


def test_values_on_midpoints_take_the_smaller_level():
    # scale 2^-6 (exact in fp16): points and midpoints are exact in fp64.
    s = np.float16(2.0 ** -6)
    L = LEV.astype(np.float64)
    mids = [(L[k] + L[k + 1]) / 2 * 2.0 ** -6 for k in range(3)]
    row = np.zeros(128)
    row[:3] = mids
    row[3:] = 1e-9
    codes = enc.nearest_codes(row[None, :], np.array([[s]]), LEV)[0]
    # boundaries (-L1,-L0) -> -L0 (code 1); (-L0,+L0) at 0 -> +L0 (code 2);
    # (+L0,+L1) -> +L0 (code 2)
    assert list(codes[:3]) == [1, 2, 2]
    for k in range(3):
        assert codes[k] == _nearest_exact(row[k], s, LEV)


def test_zero_group():
    W = np.zeros((2, 256))
    W[1, 128:] = 0.5
    out = enc.quantize_rotated(W, 7, LEV)
    assert out["base_scales"][0, 0] == 0 and out["resid_scales"][0, 0] == 0
    assert np.all(out["base_idx"][0, :128] == 2)      # |-L0| == |+L0|: the larger level
    assert np.all(out["resid"][0, :128] == 0)


def test_gaussian_base_distortion_is_lloyd_max():
    # For N(0,1) the 4-level Lloyd-Max quantiser has mean squared error
    # 0.1175 (Max 1960).  Rotated Gaussian weights with the group RMS as
    # scale land near it (the RMS of 128 samples varies by ~6%).
    rng = np.random.default_rng(6)
    W = rng.standard_normal((64, 4096))
    si = rng.choice([-1, 1], 4096).astype(np.int8)
    Wt = enc.rot_fwd(W, si)
    s = enc.base_scales(Wt)
    c = enc.nearest_codes(Wt, s, LEV)
    Q = LEV.astype(np.float64)[c] * np.repeat(s.astype(np.float64), 128, axis=1)
    d = np.mean((Wt - Q) ** 2) / np.mean(Wt ** 2)
    assert 0.112 < d < 0.124, d


# --- residual quantiser (POC section 3) ---------------------------------------

@pytest.mark.parametrize("bits", [6, 7, 8])
def test_residual_error_bounds(bits):
    rng = np.random.default_rng(bits)
    W = synth.make_dense_weights(32, 1024, cfg=7, idx=bits)
    si = synth.make_signs(1024, 7, bits, synth.STREAM_SIGN_IN)
    out = enc.encode(W, si, None, bits, LEV)
    Wt = enc.rot_fwd(W, si)
    sb = np.repeat(out["base_scales"].view(np.float16).astype(np.float64), 128, axis=1)
    sr = np.repeat(out["resid_scales"].view(np.float16).astype(np.float64), 128, axis=1)
    R = Wt - LEV.astype(np.float64)[out["base_idx"]] * sb
    E = R - out["resid"].astype(np.float64) * sr
    qm = (1 << (bits - 1)) - 1
    # a uniform step s quantises to within s/2, except where fp16 rounding
    # of max|R|/qm leaves the extreme value up to qm*s*2^-11 beyond the grid
    assert np.all(np.abs(E) <= sr / 2 + qm * sr * 2.0 ** -11 + 1e-18)
    assert np.abs(out["resid"]).max() == qm
    g = np.abs(R).reshape(32, 8, 128).argmax(axis=2)
    for r in range(32):
        for j in range(8):
            assert abs(int(out["resid"][r, 128 * j + g[r, j]])) == qm
    # the residual reduces the error, by about 2^-b of the group range
    assert np.linalg.norm(E) < np.linalg.norm(R) / (2 ** (bits - 2))
    del rng


def test_round_trip_through_the_pinned_decoder(orc):
    W = synth.make_dense_weights(24, 640, cfg=8, idx=0)
    si = synth.make_signs(640, 8, 0, synth.STREAM_SIGN_IN)
    bits = 7
    out = enc.encode(W, si, None, bits, LEV)
    lin = {"d_out": 24, "d_in": 640, "bits": bits, "levels": LEV,
           "base_codes": synth.pack_base(out["base_idx"]), "base_scales": out["base_scales"],
           "resid_codes": synth.pack_resid(out["resid"], bits), "resid_scales": out["resid_scales"],
           "sign_in": si, "sign_out": None}
    bi, rq = orc.decode(lin)
    np.testing.assert_array_equal(bi, out["base_idx"])
    np.testing.assert_array_equal(rq, out["resid"])
    sb = np.repeat(out["base_scales"].view(np.float16).astype(np.float64), 128, axis=1)
    sr = np.repeat(out["resid_scales"].view(np.float16).astype(np.float64), 128, axis=1)
    Q = LEV.astype(np.float64)[out["base_idx"]] * sb + out["resid"] * sr
    for r in (0, 11, 23):
        np.testing.assert_array_equal(orc.dequant_row(lin, r, True), Q[r])
    # and the dequantised weights rotate back close to W
    back = enc.rot_inv(Q, si)
    assert np.linalg.norm(back - W) / np.linalg.norm(W) < 0.02


# --- level fitter (POC section 2) ----------------------------------------------

def test_quantile_start_matches_numpy():
    rng = np.random.default_rng(9)
    for n in (1, 2, 7, 1000, 12345):
        v = rng.standard_normal(n)
        np.testing.assert_allclose(enc.quantile_start(v), np.quantile(v, enc.QUANTILES),
                                   rtol=0, atol=1e-15)


def test_fit_on_gaussian_quantiles_is_textbook_lloyd_max():
    # A deterministic N(0,1) sample (its quantiles at (i + 1/2)/n): the fit
    # lands on the Gaussian 4-level Lloyd-Max levels 0.4528 / 1.5104.
    from scipy.stats import norm
    n = 1 << 20
    v = norm.ppf((np.arange(n) + 0.5) / n)
    L = enc.lloyd_max_fit(v, 60)
    np.testing.assert_allclose(L, [-1.5104, -0.4528, 0.4528, 1.5104], atol=3e-4)


def test_fit_four_clusters_reaches_their_means():
    # Four well separated clusters: after the first Lloyd step every level is
    # its cluster's mean; symmetric clusters stay symmetric.
    rng = np.random.default_rng(10)
    off = rng.uniform(-0.1, 0.1, 4000)
    v = np.concatenate([-3 + off[:1000], -1 + off[1000:2000], 1 + off[2000:3000], 3 + off[3000:]])
    L = enc.lloyd_max_fit(v, 60, symmetrize=False)
    want = [np.mean(v[i * 1000:(i + 1) * 1000]) for i in range(4)]
    np.testing.assert_allclose(L, want, rtol=0, atol=1e-12)
    Ls = enc.lloyd_max_fit(v, 60)
    np.testing.assert_allclose(Ls, [-(want[3] - want[0]) / 2, -(want[2] - want[1]) / 2,
                                    (want[2] - want[1]) / 2, (want[3] - want[0]) / 2], atol=1e-12)


def test_fit_is_a_fixed_point_and_symmetric_data_stays_symmetric():
    rng = np.random.default_rng(11)
    h = rng.standard_t(5, 3000)
    v = np.concatenate([h, -h])
    L = enc.lloyd_max_fit(v, 200, symmetrize=False)
    # every level is the mean of the samples nearest to it (brute force by distance)
    d = np.abs(v[:, None] - L[None, :])
    cell = d.argmin(axis=1)
    for k in range(4):
        assert abs(v[cell == k].mean() - L[k]) < 1e-9
    np.testing.assert_allclose(L, -L[::-1], atol=1e-9)
    np.testing.assert_allclose(enc.lloyd_max_fit(v, 200), L, atol=1e-9)


def test_normalised_samples():
    W = np.zeros((1, 256))
    W[0, :128] = np.linspace(-1, 1, 128)
    v = enc.normalized(W)
    s = float(enc.base_scales(W)[0, 0])
    np.testing.assert_array_equal(v[0, :128], W[0, :128] / s)
    assert np.all(v[0, 128:] == 0)                     # zero scale gives zeros
