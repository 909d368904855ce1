"""Pins of the W4/W8 dual-plane oracle (oracle/w4w8.py) to the BitNest paper
(page 2): hand-decoded nibble bytes, the eq. 10 identity over every code
pair, the int8 range that the eq. 9 boundary rule guarantees (and that
breaks without it), the refinement's error bound, the draft as an exact
subset of the target, unit-vector columns and a loop brute force of y = W x.
"""
import numpy as np
import pytest

import synth
from oracle import w4w8 as w48


def test_nibble_bytes_by_hand():
    # byte i holds weight 2i in its low nibble; two's complement
    plane = np.array([[0x8F, 0x70, 0x01, 0xF8]], np.uint8)
    assert w48.unpack_nibbles(plane, 8).tolist() == [[-1, -8, 0, 7, 1, 0, -8, -1]]
    assert synth.pack_nibbles(np.array([[-1, -8, 0, 7, 1, 0, -8, -1]])).tolist() == plane.tolist()


def test_eq10_identity_every_code_pair():
    rng = np.random.default_rng(1)
    q4, qr = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    for s4 in rng.uniform(1e-4, 3.0, 20).astype(np.float16).astype(np.float64):
        lhs = q4 * s4 + qr * (s4 / 16)            # eq. 10, first form
        rhs = (16 * q4 + qr) * (s4 / 16)          # second form
        np.testing.assert_array_equal(lhs, rhs)   # exact: small integers times an fp16 value


def test_boundary_rule_keeps_composite_in_int8():
    allowed = [(a, b) for a in range(-8, 8) for b in (range(0, 8) if a == -8 else range(-8, 8))]
    comp = [16 * a + b for a, b in allowed]
    assert min(comp) == -128 and max(comp) == 119   # inside the int8 range [-128, 127]
    assert len(set(comp)) == len(comp)             # one composite per pair
    assert 16 * -8 + -1 < -128                     # what the rule prevents


def test_dequant_of_packed_codes():
    lin = synth.make_w4w8_linear(8, 384, cfg=40, keep_codes=True)
    s = np.repeat(lin["scales"].view(np.float16).astype(np.float64), 128, axis=1)
    np.testing.assert_array_equal(w48.dequant(lin, False), lin["q4"] * s)
    np.testing.assert_array_equal(w48.dequant(lin, True), (16.0 * lin["q4"] + lin["qr"]) * s / 16)
    # the draft is the target with a zero refinement plane
    z = dict(lin, ref_plane=np.zeros_like(lin["ref_plane"]))
    np.testing.assert_array_equal(w48.dequant(z, True), w48.dequant(lin, False))


def test_refinement_bound_and_boundary():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((32, 512)) * 0.02
    q4, s4 = w48.rtn_base(W)
    assert q4.min() >= -7                          # max|W| / 7 never reaches -8
    # a base that uses -8 (as GPTQ's can): scale max|W| / 7.5
    g = np.abs(W).reshape(32, 4, 128).max(axis=2)
    s4 = (g / 7.5).astype(np.float16)
    sd = np.repeat(s4.astype(np.float64), 128, axis=1)
    q4 = np.clip(np.rint(W / sd), -8, 7).astype(np.int8)
    qr = w48.refine(W, q4, s4)
    s = np.repeat(s4.astype(np.float64), 128, axis=1)
    target = (16.0 * q4 + qr) * s / 16
    dW = W - q4 * s
    inside = (dW / (s / 16) > -8.5) & (dW / (s / 16) < 7.5) & ~((q4 == -8) & (dW < 0))
    assert np.all(np.abs(W - target)[inside] <= s[inside] / 32 * (1 + 1e-12))
    assert np.all(qr[q4 == -8] >= 0)
    assert (q4 == -8).any()
    c = 16 * q4.astype(int) + qr
    assert c.min() >= -128 and c.max() <= 127
    # the W8 target is about 16x closer than the W4 draft
    e4 = np.linalg.norm(W - q4 * s)
    e8 = np.linalg.norm(W - target)
    assert 8 < e4 / e8 < 32


def test_unit_vectors_return_columns():
    lin = synth.make_w4w8_linear(16, 256, cfg=41)
    x = np.zeros((3, 256), np.float32)
    for t, k in enumerate((0, 129, 255)):
        x[t, k] = 1.0
    xb = synth.f32_to_bf16_bits(x)
    for verify in (False, True):
        y = w48.forward(lin, xb, verify)
        W = w48.dequant(lin, verify)
        for t, k in enumerate((0, 129, 255)):
            np.testing.assert_array_equal(y[t], W[:, k])


@pytest.mark.parametrize("verify", [False, True])
def test_forward_loop_brute_force(verify):
    lin = synth.make_w4w8_linear(4, 256, cfg=42, keep_codes=True)
    x = synth.make_x(2, 256, cfg=42)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    s4 = lin["scales"].view(np.float16).astype(np.float64)
    y = w48.forward(lin, x, verify)
    for t in range(2):
        for r in range(4):
            acc = 0.0
            for k in range(256):
                q = 16 * int(lin["q4"][r, k]) + int(lin["qr"][r, k]) if verify else int(lin["q4"][r, k])
                acc += q * (s4[r, k // 128] / (16 if verify else 1)) * xf[t, k]
            assert abs(y[t, r] - acc) <= 1e-12 * max(1.0, abs(acc))
