"""Pins of the nested-KV oracle (oracle/kv.py) to the BitNest paper's
appendix A.2 (eq. 11-14) and to plain attention: the quantiser's closed-form
error bounds and extremes, KV4 as a subset of KV8, the packed planes, and
attention that reduces to causal attention on a chain, to an average for
equal keys, and to a brute force over the tree mask."""
import numpy as np

import synth
from oracle import kv


def test_quantiser_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    x[0] = 0.0
    xb = synth.f32_to_bf16_bits(x)
    q4, qr, s = kv.quantize(xb)
    xf = kv.bf16_to_f32(xb).reshape(-1, 128).astype(np.float64)
    assert s[0] == 0 and not q4[0].any() and not qr[0].any()
    # the largest magnitude maps to +-7 (eq. 11), codes stay in range
    for i in range(1, 200):
        k = np.argmax(np.abs(xf[i]))
        assert abs(int(q4[i, k])) == 7
    assert q4.min() >= -8 and q4.max() <= 7 and qr.min() >= -8 and qr.max() <= 7
    sd = s.astype(np.float64)[:, None]
    # KV4 error within half a step s; KV8 within half a refinement step s/16,
    # except where q_r clips at +7 (the residual reaches +s/2 but the grid
    # stops at 7 s/16): there within s/16
    assert np.all(np.abs(xf - kv.dequant(q4, qr, s, False)) <= sd / 2 * (1 + 1e-6))
    e8 = np.abs(xf - kv.dequant(q4, qr, s, True))
    assert np.all(e8[qr < 7] <= np.broadcast_to(sd, e8.shape)[qr < 7] / 32 * (1 + 1e-5))
    assert np.all(e8 <= sd / 16 * (1 + 1e-5))
    # KV4 is KV8 with a zero refinement (eq. 12 vs 14)
    np.testing.assert_array_equal(kv.dequant(q4, np.zeros_like(qr), s, True), kv.dequant(q4, qr, s, False))


def test_nibble_planes_round_trip():
    rng = np.random.default_rng(2)
    q = rng.integers(-8, 8, (5, 128)).astype(np.int8)
    plane = synth.pack_nibbles(q)
    assert plane.shape == (5, 64)
    lo = (plane & 0x0F).astype(np.int16)
    hi = (plane >> 4).astype(np.int16)
    back = np.empty((5, 128), np.int16)
    back[:, 0::2], back[:, 1::2] = lo, hi
    back[back >= 8] -= 16
    np.testing.assert_array_equal(back, q)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_chain_tree_is_causal_attention():
    rng = np.random.default_rng(3)
    L, T, H_q, H_kv = 5, 4, 4, 2
    q = synth.f32_to_bf16_bits(_rand(rng, T, H_q, 128).astype(np.float32))
    k, v = _rand(rng, L + T, H_kv, 128), _rand(rng, L + T, H_kv, 128)
    anc = [(1 << (t + 1)) - 1 for t in range(T)]           # token t sees tree nodes 0..t
    out = kv.attention(q, k, v, L, anc, H_kv)
    qf = kv.bf16_to_f32(q).astype(np.float64)
    for t in range(T):
        for j in range(H_q):
            h = j // 2
            n = L + t + 1                                   # causal: context and tokens 0..t
            sc = k[:n, h] @ qf[t, j] / np.sqrt(128)
            w = np.exp(sc - sc.max())
            np.testing.assert_allclose(out[t, j], (w / w.sum()) @ v[:n, h], rtol=1e-12, atol=1e-12)


def test_equal_keys_average_the_visible_values():
    rng = np.random.default_rng(4)
    L, T = 3, 3
    q = synth.f32_to_bf16_bits(_rand(rng, T, 2, 128).astype(np.float32))
    k = np.ones((L + T, 1, 128))
    v = _rand(rng, L + T, 1, 128)
    anc = [0b001, 0b011, 0b101]                            # node 2 hangs off node 0
    out = kv.attention(q, k, v, L, anc, 1)
    for t, vis in enumerate([[0, 1, 2, 3], [0, 1, 2, 3, 4], [0, 1, 2, 3, 5]]):
        np.testing.assert_allclose(out[t, 0], v[vis, 0].mean(axis=0), atol=1e-12)
        np.testing.assert_allclose(out[t, 1], v[vis, 0].mean(axis=0), atol=1e-12)


def test_mask_brute_force():
    rng = np.random.default_rng(5)
    L, T, H_q, H_kv = 4, 5, 2, 1
    q = synth.f32_to_bf16_bits(_rand(rng, T, H_q, 128).astype(np.float32))
    k, v = _rand(rng, L + T, H_kv, 128), _rand(rng, L + T, H_kv, 128)
    anc = [0b00001, 0b00011, 0b00101, 0b01011, 0b10101]
    out = kv.attention(q, k, v, L, anc, H_kv)
    qf = kv.bf16_to_f32(q).astype(np.float64)
    for t in range(T):
        for j in range(H_q):
            num, den = np.zeros(128), 0.0
            for pos in range(L + T):
                if pos >= L and not (anc[t] >> (pos - L)) & 1:
                    continue
                w = np.exp(float(k[pos, 0] @ qf[t, j]) / np.sqrt(128))
                num += w * v[pos, 0]
                den += w
            np.testing.assert_allclose(out[t, j], num / den, rtol=1e-10, atol=1e-12)
