"""Parity of the HIP W4/W8 dual-plane linear (include/nested_w4w8.h) with the
fp64 oracle (oracle/w4w8.py), through the C-ABI.

Bar: max|dy| <= 2e-3 * max|y_oracle| per call, as for the nested linear.
The kernel's error budget: x' is bf16 widened exactly to fp16 (a power of two
per token and group puts the group's largest magnitude in [2^14, 2^15)),
the codes enter the MFMA exactly as 1024 + u, products are exact in fp32 and
the fp32 sums of 128 terms then lose ~2^-24 relative to the biased sum,
about 20x the signed one: ~1e-5 relative, far inside the bar.
"""
import numpy as np
import pytest

import synth
from oracle import w4w8 as w48

pytestmark = pytest.mark.gpu
TOL = 2e-3


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


def xdev(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def check(y, ref):
    y = y.cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all()
    err = np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= TOL, err
    return err


SHAPES = [(64, 128), (100, 384), (1024, 1024), (1024, 4096), (4096, 4096), (200, 14336)]


@pytest.mark.parametrize("d_out,d_in", SHAPES, ids=[f"{a}x{b}" for a, b in SHAPES])
@pytest.mark.parametrize("T", [1, 3, 16, 17, 33, 64])
def test_forward_matches_oracle(nl, torch_cuda, d_out, d_in, T):
    lin = synth.make_w4w8_linear(d_out, d_in, cfg=50, idx=d_in)
    x = synth.make_x(T, d_in, cfg=50, idx=T)
    L = nl.W4W8Linear(lin)
    try:
        ws = L.workspace(T)
        for verify in (False, True):
            y = L.forward(xdev(torch_cuda, x), verify, ws=ws)
            check(y, w48.forward(lin, x, verify))
        # the split-K tickets are back at zero
        assert int(ws[:256].view(torch_cuda.int32).abs().sum().item()) == 0
    finally:
        L.close()


def test_repeated_calls_are_bitwise_equal(nl, torch_cuda):
    lin = synth.make_w4w8_linear(4096, 4096, cfg=51)
    x = synth.make_x(16, 4096, cfg=51)
    L = nl.W4W8Linear(lin)
    try:
        ws = L.workspace(16)
        xd = xdev(torch_cuda, x)
        a = L.forward(xd, True, ws=ws).clone()
        b = L.forward(xd, True, ws=ws)
        assert torch_cuda.equal(a, b)
    finally:
        L.close()


def test_wide_dynamic_range_inputs(nl, torch_cuda):
    # per-group power-of-two scaling: groups of tiny, huge, zero and mixed values
    d_out, d_in, T = 128, 1024, 5
    lin = synth.make_w4w8_linear(d_out, d_in, cfg=52)
    rng = np.random.default_rng(52)
    xf = rng.standard_normal((T, d_in)).astype(np.float32)
    xf[0, :128] *= 1e-30
    xf[1, 128:256] *= 1e30
    xf[2, 256:384] = 0.0
    xf[3, 384:512] *= np.where(rng.random(128) < 0.5, 1e-3, 1e3).astype(np.float32)
    x = synth.f32_to_bf16_bits(xf)
    L = nl.W4W8Linear(lin)
    try:
        for verify in (False, True):
            y = L.forward(xdev(torch_cuda, x), verify).cpu().numpy().astype(np.float64)
            ref = w48.forward(lin, x, verify)
            for t in range(T):   # per token: the rows differ by 60 orders of magnitude
                assert np.abs(y[t] - ref[t]).max() <= TOL * np.abs(ref[t]).max(), t
    finally:
        L.close()


def test_draft_only_linear(nl, torch_cuda):
    lin = synth.make_w4w8_linear(256, 512, cfg=53)
    lin = dict(lin, ref_plane=None)
    x = synth.make_x(4, 512, cfg=53)
    L = nl.W4W8Linear(lin)
    try:
        check(L.forward(xdev(torch_cuda, x), False), w48.forward(lin, x, False))
        with pytest.raises(nl.NLError) as e:
            L.forward(xdev(torch_cuda, x), True)
        assert e.value.status == nl.NL_EINVAL
    finally:
        L.close()


def test_draft_equals_verify_with_zero_refinement(nl, torch_cuda):
    lin = synth.make_w4w8_linear(512, 2048, cfg=54)
    z = dict(lin, ref_plane=np.zeros_like(lin["ref_plane"]))
    x = synth.make_x(16, 2048, cfg=54)
    La, Lb = nl.W4W8Linear(lin), nl.W4W8Linear(z)
    try:
        yd = La.forward(xdev(torch_cuda, x), False).cpu().numpy()
        yv = Lb.forward(xdev(torch_cuda, x), True).cpu().numpy()
        # same math up to the fp32 bias cancellation (1032 vs 1160)
        assert np.abs(yd - yv).max() <= 1e-4 * np.abs(yd).max()
    finally:
        La.close()
        Lb.close()


FULL = [("q/o", 4096, 4096), ("k/v", 1024, 4096), ("gate/up", 14336, 4096), ("down", 4096, 14336)]


@pytest.mark.parametrize("name,d_out,d_in", FULL, ids=[f[0] for f in FULL])
@pytest.mark.parametrize("T", [4, 16, 64])
def test_full_size_sampled_rows(nl, torch_cuda, name, d_out, d_in, T):
    lin = synth.make_w4w8_linear(d_out, d_in, cfg=55, idx=d_out + d_in)
    x = synth.make_x(T, d_in, cfg=55, idx=1)
    L = nl.W4W8Linear(lin)
    try:
        ws = L.workspace(T)
        for verify in (False, True):
            y = L.forward(xdev(torch_cuda, x), verify, ws=ws).cpu().numpy().astype(np.float64)
            mid = d_out // 2 - 37
            for r0, r1 in [(0, 64), (mid, mid + 64), (d_out - 64, d_out)]:
                ref = w48.forward(lin, x, verify, rows=(r0, r1))
                assert np.abs(y[:, r0:r1] - ref).max() <= TOL * np.abs(ref).max(), (verify, r0)
    finally:
        L.close()


RT_SHAPES = [(6000, 1024), (14336, 512)]


@pytest.mark.parametrize("d_out,d_in", RT_SHAPES, ids=[f"{a}x{b}" for a, b in RT_SHAPES])
@pytest.mark.parametrize("T", [1, 2, 4])
def test_row_tiles_with_k_shares(nl, torch_cuda, d_out, d_in, T):
    """For small T * d_in a workgroup holds the whole K-range and splits it
    among the waves of each of its 16-row tiles: 376 tiles take two tiles
    per workgroup, 896 take four (the smaller shapes above take one)."""
    lin = synth.make_w4w8_linear(d_out, d_in, cfg=57, idx=d_out)
    x = synth.make_x(T, d_in, cfg=57, idx=T)
    L = nl.W4W8Linear(lin)
    try:
        ws = L.workspace(T)
        for verify in (False, True):
            y = L.forward(xdev(torch_cuda, x), verify, ws=ws)
            check(y, w48.forward(lin, x, verify))
    finally:
        L.close()


@pytest.mark.parametrize("T", [17, 40, 64])
def test_x_staged_in_pieces(nl, torch_cuda, T):
    """16384 x 4224 (33 groups): two splits of 17 and 16 groups, more than the
    LDS holds at these T, so each split stages x in pieces of whole ring
    rounds (12 + 5 groups at T = 17, 6 + 6 + 5 at T = 40 and 64), the last
    one ragged; checked on sampled rows."""
    d_out, d_in = 16384, 4224
    lin = synth.make_w4w8_linear(d_out, d_in, cfg=56, idx=T)
    x = synth.make_x(T, d_in, cfg=56, idx=T)
    L = nl.W4W8Linear(lin)
    try:
        ws = L.workspace(T)
        for verify in (False, True):
            y = L.forward(xdev(torch_cuda, x), verify, ws=ws).cpu().numpy().astype(np.float64)
            for r0, r1 in [(0, 64), (8191, 8319), (d_out - 64, d_out)]:
                ref = w48.forward(lin, x, verify, rows=(r0, r1))
                assert np.abs(y[:, r0:r1] - ref).max() <= TOL * np.abs(ref).max(), (verify, r0)
    finally:
        L.close()


def test_errors(nl, torch_cuda):
    lin = synth.make_w4w8_linear(64, 256, cfg=56)
    L = nl.W4W8Linear(lin)
    try:
        x = xdev(torch_cuda, synth.make_x(65, 256, cfg=56))
        ws = L.workspace(64)
        y = torch_cuda.empty((65, 64), dtype=torch_cuda.float32, device="cuda")
        with pytest.raises(nl.NLError) as e:
            nl.nested_w4w8_verify(L.h, x, 65, y, ws)
        assert e.value.status == nl.NL_EUNSUPPORTED
        with pytest.raises(nl.NLError) as e:
            nl.nested_w4w8_verify(L.h, x, 0, y, ws)
        assert e.value.status == nl.NL_EINVAL
        with pytest.raises(nl.NLError) as e:
            nl.nested_w4w8_verify(L.h, x.view(-1)[1:], 4, y, ws)    # misaligned x
        assert e.value.status == nl.NL_EINVAL
    finally:
        L.close()
