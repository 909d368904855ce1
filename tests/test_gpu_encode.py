"""Parity of the HIP encoder and level fitter (include/nested_encode.h) with
the fp64 oracle (oracle/encode.py).

The rotation runs in fp64 with the oracle's butterfly order, so the rotated
matrix is compared bit for bit; codes and scales are integer decisions taken
from it exactly (midpoints, fp16 rounding straight from fp64), so the packed
planes are compared byte for byte.  The fitter's cell sums are added in a
different order than numpy's, so its levels are compared to within 1e-9
relative: an fp64 sum of n <= 2^21 terms of one sign is off by at most
n * 2^-53 ~ 2.3e-10 relative, and the Lloyd map does not amplify it.  Its
quantile start (iters = 0) is exact: order statistics from the radix select
and the same interpolation formula.
"""
import numpy as np
import pytest

import synth
from oracle import encode as enc

pytestmark = pytest.mark.gpu
LEV = synth.LEVELS


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


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def oracle_planes(out, bits):
    planes = {"base_codes": synth.pack_base(out["base_idx"]), "base_scales": out["base_scales"]}
    if bits:
        planes["resid_codes"] = synth.pack_resid(out["resid"], bits)
        planes["resid_scales"] = out["resid_scales"]
    return planes


def assert_planes_equal(got, want, bits, rows=None):
    keys = ["base_codes", "base_scales"] + (["resid_codes", "resid_scales"] if bits else [])
    for k in keys:
        g = got[k] if rows is None else got[k][rows[0]:rows[1]]
        w = want[k].reshape(g.shape)
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            raise AssertionError(f"{k}: {len(bad)} mismatches, first at {bad[0].tolist()}")


ONE_SIDED = [(3, 384, 6), (37, 5120, 7), (64, 4096, 8), (20, 14336, 7), (5, 640, 0), (1, 128, 8),
             (130, 1152, 6)]


@pytest.mark.parametrize("d_out,d_in,bits", ONE_SIDED, ids=[f"{a}x{b}-{c}bit" for a, b, c in ONE_SIDED])
def test_fused_one_sided_encode(nl, torch_cuda, d_out, d_in, bits):
    W = synth.make_dense_weights(d_out, d_in, cfg=20, idx=d_in + bits)
    si = synth.make_signs(d_in, 20, d_in, synth.STREAM_SIGN_IN)
    c = nl.encode(dev(torch_cuda, W), dev(torch_cuda, si), None, bits, LEV)
    torch_cuda.cuda.synchronize()
    want = oracle_planes(enc.encode(W, si, None, bits, LEV), bits)
    assert_planes_equal(c.host(), want, bits)


TWO_SIDED = [(96, 640, 7), (1024, 256, 8), (4096, 128, 6), (3, 256, 0), (200, 384, 8)]


@pytest.mark.parametrize("d_out,d_in,bits", TWO_SIDED, ids=[f"{a}x{b}-{c}bit" for a, b, c in TWO_SIDED])
def test_two_sided_encode(nl, torch_cuda, d_out, d_in, bits):
    W = synth.make_dense_weights(d_out, d_in, cfg=21, idx=d_out)
    si = synth.make_signs(d_in, 21, d_out, synth.STREAM_SIGN_IN)
    so = synth.make_signs(d_out, 21, d_out, synth.STREAM_SIGN_OUT)
    c = nl.encode(dev(torch_cuda, W), dev(torch_cuda, si), dev(torch_cuda, so), bits, LEV)
    torch_cuda.cuda.synchronize()
    want = oracle_planes(enc.encode(W, si, so, bits, LEV), bits)
    assert_planes_equal(c.host(), want, bits)


@pytest.mark.parametrize("two", [False, True])
def test_rotation_is_bit_exact(nl, torch_cuda, two):
    d_out, d_in = 512, 5376                  # blocks 512 and 256
    W = synth.make_dense_weights(d_out, d_in, cfg=22, idx=int(two))
    si = synth.make_signs(d_in, 22, 0, synth.STREAM_SIGN_IN)
    so = synth.make_signs(d_out, 22, 0, synth.STREAM_SIGN_OUT) if two else None
    wt = torch_cuda.empty((d_out, d_in), dtype=torch_cuda.float64, device="cuda")
    nl.nested_encode_rotate(d_out, d_in, dev(torch_cuda, W), dev(torch_cuda, si),
                            None if so is None else dev(torch_cuda, so), wt)
    got = wt.cpu().numpy()
    np.testing.assert_array_equal(got, enc.rot_fwd(W, si, so))


def planted_rotated(d_out=6, d_in=512, seed=23):
    """fp64 rotated weights with hand-made groups: values exactly on the
    midpoints between reconstruction points, an all-zero group, a group
    that saturates fp16, tiny values (subnormal fp16 scales)."""
    rng = np.random.default_rng(seed)
    Wt = rng.standard_normal((d_out, d_in)) * 0.02
    L = LEV.astype(np.float64)
    # group (0, 0): 120 entries of +-1 and 8 entries on the three midpoints
    g = rng.choice([-1.0, 1.0], 128)
    s = 1.0
    for _ in range(5):
        mids = [(L[k] * s + L[k + 1] * s) * 0.5 for k in range(3)]
        g[:8] = [mids[i % 3] for i in range(8)]
        s = float(enc.base_scales(g[None, :])[0, 0])
    assert all(v in [(L[k] * s + L[k + 1] * s) * 0.5 for k in range(3)] for v in g[:8])
    Wt[0, :128] = g
    Wt[1, 128:256] = 0.0
    Wt[2, 256:384] = rng.standard_normal(128) * 1e6
    Wt[3, :128] = rng.standard_normal(128) * 1e-6
    Wt[4, 384:512] = rng.standard_normal(128) * 3e-8
    return Wt


@pytest.mark.parametrize("bits", [0, 6, 7, 8])
def test_quantize_planted_groups(nl, torch_cuda, bits):
    Wt = planted_rotated()
    c = nl.Codes(Wt.shape[0], Wt.shape[1], bits, LEV)
    nl.nested_encode_quantize(dev(torch_cuda, Wt), c.desc)
    torch_cuda.cuda.synchronize()
    want = oracle_planes(enc.quantize_rotated(Wt, bits, LEV), bits)
    assert_planes_equal(c.host(), want, bits)
    got = c.host()
    assert got["base_scales"][2, 2] == 0x7BFF                       # saturated
    assert got["base_scales"][1, 1] == 0                            # zero group


def test_normalized_samples_bit_exact(nl, torch_cuda):
    Wt = planted_rotated(8, 1024, seed=24)
    v = torch_cuda.empty(Wt.shape, dtype=torch_cuda.float64, device="cuda")
    nl.nested_encode_normalize(Wt.shape[0], Wt.shape[1], dev(torch_cuda, Wt), v)
    np.testing.assert_array_equal(v.cpu().numpy(), enc.normalized(Wt))


def fit(nl, torch, v, iters):
    ws = torch.empty(nl.nested_encode_fit_workspace_bytes(v.size), dtype=torch.uint8, device="cuda")
    return np.array(nl.nested_encode_fit_levels(dev(torch, v), v.size, iters, ws))


@pytest.mark.parametrize("n", [1, 2, 7, 1000, 4097, 300001])
def test_quantile_start_is_exact(nl, torch_cuda, n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal(n)
    if n > 100:
        v[: n // 3] = np.rint(v[: n // 3] * 4) / 4            # many equal values
        v[n // 3: n // 3 + 50] = -0.0
    np.testing.assert_array_equal(fit(nl, torch_cuda, v, 0), enc.lloyd_max_fit(v, 0))


def test_fit_on_rotated_weights(nl, torch_cuda):
    # the post's recipe: ~2M rotated weights normalised by their group RMS
    d_out, d_in = 512, 4096
    W = synth.make_dense_weights(d_out, d_in, cfg=25, idx=0)
    si = synth.make_signs(d_in, 25, 0, synth.STREAM_SIGN_IN)
    wt = torch_cuda.empty((d_out, d_in), dtype=torch_cuda.float64, device="cuda")
    nl.nested_encode_rotate(d_out, d_in, dev(torch_cuda, W), dev(torch_cuda, si), None, wt)
    v = torch_cuda.empty_like(wt)
    nl.nested_encode_normalize(d_out, d_in, wt, v)
    ws = torch_cuda.empty(nl.nested_encode_fit_workspace_bytes(v.numel()), dtype=torch_cuda.uint8,
                          device="cuda")
    got = np.array(nl.nested_encode_fit_levels(v, v.numel(), 60, ws))
    vo = enc.normalized(enc.rot_fwd(W, si))
    want = enc.lloyd_max_fit(vo, 60)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=0)
    # and it is the Gaussian 4-level Lloyd-Max quantiser, as the post found
    np.testing.assert_allclose(got, [-1.5104, -0.4528, 0.4528, 1.5104], atol=0.01)
    # repeated calls agree exactly (fixed summation order)
    np.testing.assert_array_equal(np.array(nl.nested_encode_fit_levels(v, v.numel(), 60, ws)), got)


@pytest.mark.parametrize("n,iters", [(5, 60), (1 << 16, 7), (123457, 60)])
def test_fit_small_and_ragged(nl, torch_cuda, n, iters):
    v = np.random.default_rng(n).standard_t(4, n)
    np.testing.assert_allclose(fit(nl, torch_cuda, v, iters), enc.lloyd_max_fit(v, iters), rtol=1e-9, atol=1e-15)


# --- full sizes, sampled rows -------------------------------------------------

FULL = [("llama8b gate/up", 14336, 4096, 7), ("llama8b down", 4096, 14336, 7), ("31b down", 5120, 25600, 8)]


@pytest.mark.parametrize("name,d_out,d_in,bits", FULL, ids=[f[0] for f in FULL])
def test_full_size_one_sided_sampled_rows(nl, torch_cuda, name, d_out, d_in, bits):
    W = synth.make_dense_weights(d_out, d_in, cfg=26, idx=d_out + d_in)
    si = synth.make_signs(d_in, 26, 0, synth.STREAM_SIGN_IN)
    c = nl.encode(dev(torch_cuda, W), dev(torch_cuda, si), None, bits, LEV)
    torch_cuda.cuda.synchronize()
    got = c.host()
    mid = d_out // 2 - 37
    for r0, r1 in [(0, 64), (mid, mid + 64), (d_out - 64, d_out)]:
        want = oracle_planes(enc.encode(W[r0:r1], si, None, bits, LEV), bits)
        assert_planes_equal(got, want, bits, rows=(r0, r1))


# --- the encoder's output drives the forward ------------------------------------

def test_encoded_linear_forward(nl, torch_cuda):
    import oracle
    d_out, d_in, bits = 384, 2048, 8
    W = synth.make_dense_weights(d_out, d_in, cfg=27, idx=0)
    si = synth.make_signs(d_in, 27, 0, synth.STREAM_SIGN_IN)
    so = synth.make_signs(d_out, 27, 0, synth.STREAM_SIGN_OUT)
    c = nl.encode(dev(torch_cuda, W), dev(torch_cuda, si), dev(torch_cuda, so), bits, LEV)
    lin = dict(c.host(), sign_in=si, sign_out=so)
    x = synth.make_x(8, d_in, cfg=27, idx=1)
    L = nl.Linear(lin)
    try:
        xd = torch_cuda.from_numpy(x.view(np.int16)).cuda()
        for verify in (False, True):
            y = L.forward(xd, verify).cpu().numpy().astype(np.float64)
            ref = oracle.forward(lin, x, verify)
            assert np.abs(y - ref).max() <= 2e-3 * np.abs(ref).max()
        # the verify output approximates the dense product W x
        dense = synth.bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
        assert np.linalg.norm(y - dense) / np.linalg.norm(dense) < 0.02
    finally:
        L.close()


def test_encoder_argument_errors(nl, torch_cuda):
    W = torch_cuda.zeros((4, 256), dtype=torch_cuda.float32, device="cuda")
    si = torch_cuda.ones(256, dtype=torch_cuda.int8, device="cuda")
    with pytest.raises(nl.NLError) as e:
        nl.encode(W, si, None, 7, [-1.0, 0.5, 0.4, 1.0])
    assert e.value.status == nl.NL_EINVAL
    c = nl.Codes(4, 256, 7, LEV)
    so = torch_cuda.ones(4, dtype=torch_cuda.int8, device="cuda")
    with pytest.raises(nl.NLError) as e:
        nl.nested_encode(W, si, so, c.desc, None)          # two-sided needs a workspace
    assert e.value.status == nl.NL_EINVAL
