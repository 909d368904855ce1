"""Pins of the fp64 oracle to what the source pages and the mathematics fix.

Each test checks the oracle against something other than itself: the block
size examples the forum post prints, a dense Hadamard matrix grown by the
Sylvester recursion, the closed form of its entries, library conversions of
fp16/bf16, hand-derived storage bytes, a dense brute force of the two-sided
rotation algebra, the nesting property and the byte budgets.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sylvester(b: int) -> np.ndarray:
    """Dense normalised Hadamard matrix grown as the forum post's POC section 1
    describes: start from [1], double as [[H, H], [H, -H]], divide by sqrt(b)."""
    H = np.ones((1, 1))
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(b)


def block_diag_h(n: int, b: int) -> np.ndarray:
    H = np.zeros((n, n))
    Hb = sylvester(b)
    for s in range(0, n, b):
        H[s:s + b, s:s + b] = Hb
    return H


# --- rotation (POC section 1) -------------------------------------------------

@pytest.mark.parametrize("n,b", [(4096, 4096), (8192, 4096), (15360, 1024), (3840, 256), (5376, 256)])
def test_block_size_printed_examples(orc, n, b):
    # The five examples printed under "Block size" in POC section 1.
    assert orc.block_size(n) == b


@pytest.mark.parametrize("n,b", [(14336, 2048), (25600, 1024), (5120, 1024), (2048, 2048),
                                 (512, 512), (128256, 256), (1, 1), (7, 1), (12, 4)])
def test_block_size_rule(orc, n, b):
    # Largest power of two dividing n, capped at 4096.
    assert orc.block_size(n) == b
    assert n % b == 0 and (b == 4096 or (n // b) % 2 == 1)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 64, 256, 1024])
def test_fwht_equals_dense_sylvester(orc, b):
    rng = np.random.default_rng(b)
    v = rng.standard_normal((3, b))
    np.testing.assert_allclose(orc.fwht(v), v @ sylvester(b).T, rtol=0, atol=1e-12 * np.sqrt(b))


def test_dense_sylvester_closed_form():
    # Natural (Sylvester) order: H[i, j] = (-1)^popcount(i & j) / sqrt(b).
    b = 64
    i, j = np.meshgrid(np.arange(b), np.arange(b), indexing="ij")
    pc = np.vectorize(lambda a: bin(a).count("1"))(i & j)
    np.testing.assert_array_equal(sylvester(b) * np.sqrt(b), (-1.0) ** pc)


@pytest.mark.parametrize("n", [4096, 14336, 5120, 3840])
def test_fwht_is_its_own_inverse(orc, n):
    # Orthonormal and symmetric => H H = I; also Parseval.
    rng = np.random.default_rng(n)
    v = rng.standard_normal(n)
    w = orc.fwht(v)
    np.testing.assert_allclose(np.linalg.norm(w), np.linalg.norm(v), rtol=1e-13)
    np.testing.assert_allclose(orc.fwht(w), v, rtol=0, atol=1e-12)


def test_fwht_delta_gives_column(orc):
    b = 4096
    for j in (0, 1, 77, 4095):
        e = np.zeros(2 * b)
        e[b + j] = 1.0
        out = orc.fwht(e)
        i = np.arange(b)
        col = (-1.0) ** np.array([bin(a & j).count("1") for a in i]) / 64.0
        np.testing.assert_array_equal(out[:b], 0.0)
        np.testing.assert_array_equal(out[b:], col)


# --- number formats -----------------------------------------------------------

def test_half_conversion_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(p) for p in pats[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    np.testing.assert_array_equal(got[fin], r[fin])
    assert np.all(np.isnan(got[np.isnan(r)]))
    assert np.all(got[np.isinf(r)] == r[np.isinf(r)])


def test_formats_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "storage_format.json")))
    for e in g["fp16"]:
        assert orc.half_to_double(int(e["bits_hex"], 16)) == e["value"]
    for e in g["bf16"]:
        assert orc.bf16_to_double(int(e["bits_hex"], 16)) == e["value"]


# --- storage format (POC sections 2 and 3) ------------------------------------

def _lin_from_bytes(base_group: bytes | None, resid_group: bytes | None, bits: int):
    lin = {"d_out": 1, "d_in": 128, "bits": bits,
           "base_codes": np.frombuffer(base_group or bytes(32), np.uint8).reshape(1, 1, 32),
           "resid_codes": None}
    if bits:
        rg = bytearray(16 * bits)
        rg[:len(resid_group)] = resid_group
        lin["resid_codes"] = np.frombuffer(bytes(rg), np.uint8).reshape(1, 1, 16 * bits)
    return lin


def test_decode_golden_base(orc):
    g = json.load(open(os.path.join(GOLDEN, "storage_format.json")))["base_group"]
    bi, _ = orc.decode(_lin_from_bytes(bytes.fromhex(g["bytes_hex"]), None, 0))
    np.testing.assert_array_equal(bi[0], np.arange(128) % 4)


def test_decode_golden_resid(orc):
    g = json.load(open(os.path.join(GOLDEN, "storage_format.json")))["resid_fields"]
    for e in g:
        _, rq = orc.decode(_lin_from_bytes(None, bytes.fromhex(e["bytes_hex"]), e["bits"]))
        np.testing.assert_array_equal(rq[0, :4], e["values"])
        np.testing.assert_array_equal(rq[0, 4:], 0)


@pytest.mark.parametrize("bits", [6, 7, 8])
def test_decode_every_pattern_every_phase(orc, bits):
    # Every residual bit pattern (including the never-generated -2^(b-1)) at
    # every field position of a group, and every base code at every position.
    n = 1 << bits
    r = np.arange(n)[:, None]
    p = np.arange(128)[None, :]
    q = ((r + p) % n) - n // 2                       # row r, position p
    codes = ((r + p) % 4).astype(np.uint8)
    lin = {"d_out": n, "d_in": 128, "bits": bits,
           "base_codes": synth.pack_base(codes), "resid_codes": synth.pack_resid(q, bits)}
    bi, rq = orc.decode(lin)
    np.testing.assert_array_equal(bi, codes)
    np.testing.assert_array_equal(rq.astype(np.int64), q)


def test_ragged_group_is_zero_padded(orc):
    lin = synth.make_linear(3, 200, 7, cfg=90, idx=0, keep_codes=True)
    bi, rq = orc.decode(lin)
    np.testing.assert_array_equal(bi, lin["base_idx"])
    np.testing.assert_array_equal(rq, lin["resid_q"])


# --- the forward (POC section 4) against a dense brute force ------------------

def dense_weights(lin: dict, verify: bool) -> np.ndarray:
    """W~ from the generator's raw integers (not from the packed planes)."""
    g_of_k = np.arange(lin["d_in"]) // 128
    sb = lin["base_scales"].view(np.float16).astype(np.float64)[:, g_of_k]
    W = lin["levels"].astype(np.float64)[lin["base_idx"]] * sb
    if verify:
        sr = lin["resid_scales"].view(np.float16).astype(np.float64)[:, g_of_k]
        W = W + lin["resid_q"].astype(np.float64) * sr
    return W


def brute_force(lin: dict, x_bits: np.ndarray, verify: bool) -> np.ndarray:
    """y = W_v x with W_v = S_o H_o W~ H_i S_i built from dense matrices
    (POC section 1, "The math": W = S_o H_o W~ H_i S_i is the exact inverse
    of the rotation, and y = W x)."""
    d_out, d_in = lin["d_out"], lin["d_in"]
    Hi = block_diag_h(d_in, _bs(d_in))
    Si = np.diag(lin["sign_in"].astype(np.float64))
    Wt = dense_weights(lin, verify)
    if lin["sign_out"] is not None:
        Ho = block_diag_h(d_out, _bs(d_out))
        So = np.diag(lin["sign_out"].astype(np.float64))
        Wv = So @ Ho @ Wt @ Hi @ Si
    else:
        Wv = Wt @ Hi @ Si
    x = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    return x @ Wv.T


def _bs(n):
    b = 1
    while n % (2 * b) == 0 and 2 * b <= 4096:
        b *= 2
    return b


@pytest.mark.parametrize("d_out,d_in,bits,two", [(8, 8, 8, True), (16, 16, 6, True), (16, 16, 7, False),
                                                 (128, 256, 8, True), (256, 128, 6, True),
                                                 (24, 200, 7, True), (12, 384, 8, False)])
@pytest.mark.parametrize("verify", [False, True])
def test_forward_equals_dense_brute_force(orc, d_out, d_in, bits, two, verify):
    lin = synth.make_linear(d_out, d_in, bits, cfg=91, idx=d_out * 1000 + d_in, two_sided=two,
                            keep_codes=True)
    x = synth.make_x(5, d_in, cfg=91, idx=d_in)
    y = orc.forward(lin, x, verify)
    ref = brute_force(lin, x, verify)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_rot_inv_of_rot_fwd_is_identity(orc):
    # POC section 1 "rot_fwd"/"rot_inv": rotating a dense W into W~ with the
    # oracle's transform on both sides and back gives W.
    rng = np.random.default_rng(5)
    d_out, d_in = 96, 320           # blocks 32 and 64
    W = rng.standard_normal((d_out, d_in))
    si = rng.choice([-1.0, 1.0], d_in)
    so = rng.choice([-1.0, 1.0], d_out)
    Wr = orc.fwht(W * si)                       # W S_i H_i   (H symmetric)
    Wr = orc.fwht((Wr * so[:, None]).T).T       # H_o S_o (...)
    back = orc.fwht(Wr.T).T * so[:, None]       # S_o H_o W~
    back = orc.fwht(back) * si                  # ... H_i S_i
    np.testing.assert_allclose(back, W, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d_in", [256, 1024, 4096])
def test_unit_input_returns_dequantised_column(orc, d_in):
    # x = S_i H_i e_j makes x' = e_j, so the one-sided output is column j of
    # W~.  Entries of S_i H_i e_j are +-1/sqrt(b), exact in bf16 for these b.
    lin = synth.make_linear(64, d_in, 8, cfg=92, idx=d_in, two_sided=False, keep_codes=True)
    b = _bs(d_in)
    js = [0, 5, d_in - 1]
    X = np.zeros((len(js), d_in))
    for t, j in enumerate(js):
        blk = j // b
        X[t, blk * b:(blk + 1) * b] = sylvester(b)[:, j % b]
    X = X * lin["sign_in"]
    xb = synth.f32_to_bf16_bits(X.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), X)
    W = dense_weights(lin, True)
    y = orc.forward(lin, xb, True)
    for t, j in enumerate(js):
        np.testing.assert_allclose(y[t], W[:, j], rtol=1e-14, atol=1e-300)


# --- nesting (POC section 4: the draft forward is the verifier without y_r) ---

@pytest.mark.parametrize("bits", [6, 7, 8])
def test_verify_with_zero_residual_equals_draft(orc, bits):
    lin = synth.make_linear(128, 512, bits, cfg=93, idx=bits)
    x = synth.make_x(4, 512, cfg=93, idx=bits)
    zs = dict(lin, resid_scales=np.zeros_like(lin["resid_scales"]))
    zc = dict(lin, resid_codes=np.zeros_like(lin["resid_codes"]))
    d = orc.forward(lin, x, False)
    np.testing.assert_array_equal(orc.forward(zs, x, True), d)
    np.testing.assert_array_equal(orc.forward(zc, x, True), d)
    # and verify = draft + (residual-only) by linearity
    rb = dict(lin, base_scales=np.zeros_like(lin["base_scales"]))
    np.testing.assert_allclose(orc.forward(lin, x, True), d + orc.forward(rb, x, True),
                               rtol=0, atol=1e-12 * np.abs(d).max())


def test_row_subset_matches_full(orc):
    lin = synth.make_linear(6144, 256, 6, cfg=94, idx=0)            # block 2048, 3 blocks
    x = synth.make_x(3, 256, cfg=94, idx=0)
    full = orc.forward(lin, x, True)
    part = orc.forward(lin, x, True, rows=(2048, 4096))
    np.testing.assert_array_equal(part, full[:, 2048:4096])


# --- byte budgets (POC section 2 "2.125 bits/weight"; residual "b + 0.125") ---

@pytest.mark.parametrize("bits,bpw", [(6, 6.125), (7, 7.125), (8, 8.125)])
def test_bit_budgets_from_buffers(bits, bpw):
    lin = synth.make_linear(64, 1024, bits, cfg=95, idx=bits)
    n = 64 * 1024
    base = (lin["base_codes"].nbytes + lin["base_scales"].nbytes) * 8 / n
    res = (lin["resid_codes"].nbytes + lin["resid_scales"].nbytes) * 8 / n
    assert base == 2.125
    assert res == bpw
    assert synth.bytes_per_weight(bits) * 8 == 2.125 + bpw


def test_residual_vs_q8_0_savings():
    # "6-bit ... about 28% fewer bytes", "7-bit ... about 16% fewer" vs Q8_0's 8.5 b/w.
    assert round(100 * (1 - 6.125 / 8.5)) == 28
    assert round(100 * (1 - 7.125 / 8.5)) == 16


def test_31b_draft_bytes():
    # "the 31B 2-bit codes take 7.78 GB": 64 layers of 31B-class shapes at 2.125 b/w.
    h, i, kv = 5120, 25600, 1024
    per_layer = 2 * h * h + 2 * kv * h + 3 * i * h
    gb = 64 * per_layer * synth.bytes_per_weight(0) / 1e9
    assert abs(gb - 7.78) / 7.78 < 0.005


def test_levels_are_gaussian_lloyd_max():
    # POC section 2: the fitted levels are "essentially the Gaussian 4-level
    # Lloyd-Max".  Lloyd iteration on the N(0,1) density from the page's
    # quantile start.
    from scipy.stats import norm
    c = norm.ppf([0.125, 0.375, 0.625, 0.875])
    for _ in range(200):
        t = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
        num = norm.pdf(t[:-1]) - norm.pdf(t[1:])
        den = norm.cdf(t[1:]) - norm.cdf(t[:-1])
        c = num / den
    c = (c - c[::-1]) / 2
    np.testing.assert_allclose(synth.LEVELS, c, atol=1e-4)


def test_residual_codes_in_range():
    for bits in (6, 7, 8):
        q = synth.make_resid_codes(64, 512, bits, cfg=96, idx=bits)
        qm = (1 << (bits - 1)) - 1
        assert q.min() >= -qm and q.max() <= qm


# --- the grouped (mixture-of-experts) forward ("The verify's own cost") -------
#
# Pair p, routed to expert e by offsets[e] <= p < offsets[e+1], is expert e's
# Linear applied to token pair_token[p].  The pins below hold forward_grouped to
# that definition through the dense brute force and through unit inputs that
# pick known columns, so a wrong expert, a wrong token or a shifted offset fails.

def _unit_rows(lin, js):
    """Rows x_t = S_i H_i e_{j_t} (so x' = e_j), exact in bf16 for b a power of 4."""
    d_in = lin["d_in"]
    b = _bs(d_in)
    X = np.zeros((len(js), d_in))
    for t, j in enumerate(js):
        blk = j // b
        X[t, blk * b:(blk + 1) * b] = sylvester(b)[:, j % b]
    X = X * lin["sign_in"]
    xb = synth.f32_to_bf16_bits(X.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), X)
    return xb


@pytest.mark.parametrize("verify", [False, True])
def test_grouped_equals_per_pair_brute_force(orc, verify):
    d_out, d_in, bits = 48, 256, 7
    experts = [synth.make_linear(d_out, d_in, bits, cfg=95, idx=e, two_sided=e == 1, keep_codes=True)
               for e in range(4)]
    # expert 2 gets no pairs; token 3 is routed twice; tokens appear out of order
    offsets = np.array([0, 3, 5, 5, 8])
    pair_token = np.array([4, 0, 3, 3, 1, 2, 0, 4])
    x = synth.make_x(5, d_in, cfg=95, idx=0)
    y = orc.forward_grouped(experts, pair_token, offsets, x, verify)
    assert y.shape == (8, d_out)
    for e in range(4):
        for p in range(offsets[e], offsets[e + 1]):
            ref = brute_force(experts[e], x[pair_token[p]:pair_token[p] + 1], verify)[0]
            np.testing.assert_allclose(y[p], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_grouped_unit_inputs_return_each_experts_column(orc):
    # Every token is a unit input e_j; pair p of expert e must return column
    # j(pair_token[p]) of expert e's W~, which differs between experts.
    d_in = 1024
    experts = [synth.make_linear(32, d_in, 8, cfg=96, idx=e, two_sided=False, keep_codes=True) for e in range(3)]
    for lin in experts[1:]:                       # one sign vector for all (x is shared)
        lin["sign_in"] = experts[0]["sign_in"]
    js = [7, 1000, 0, 513]
    x = _unit_rows(experts[0], js)
    offsets = np.array([0, 2, 2, 6])               # the middle expert is empty
    pair_token = np.array([3, 1, 0, 1, 2, 3])
    y = orc.forward_grouped(experts, pair_token, offsets, x, True)
    for e in range(3):
        W = dense_weights(experts[e], True)
        for p in range(offsets[e], offsets[e + 1]):
            np.testing.assert_allclose(y[p], W[:, js[pair_token[p]]], rtol=1e-14, atol=1e-300)


def test_grouped_single_expert_holding_every_pair(orc):
    lin = synth.make_linear(40, 512, 6, cfg=97, idx=0, keep_codes=True)
    x = synth.make_x(6, 512, cfg=97, idx=0)
    pair_token = np.array([5, 5, 2, 0, 1, 3, 4])
    y = orc.forward_grouped([lin], pair_token, np.array([0, 7]), x, True)
    np.testing.assert_allclose(y, brute_force(lin, x[pair_token], True), rtol=0,
                               atol=1e-12 * np.abs(y).max())
    # no pairs at all: an empty result of the right width
    assert orc.forward_grouped([lin], np.zeros(0, np.int64), np.array([0, 0]), x, False).shape == (0, 40)
