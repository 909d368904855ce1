"""Edge cases of the nested linear's forward, checked token by token.

The bar of a call, max|dy| <= 2e-3 * max|y_oracle|, would hide a small token
behind a large one; here every token t must meet max|dy_t| <= 2e-3 *
max|y_oracle,t| on its own, and a token whose oracle output is zero must come
out exactly zero.  Inputs follow the method's sensitive spots (forum post,
POC sections 1-4):
  * activations that the rotation maps to a constant per block
    (x = c S_i H_i 1: one spike per block), a single spike channel, and a few
    large outlier channels over N(0,1);
  * token magnitudes from 1e-20 to 1e20 in one call, and a zero token;
  * residual codes all zero (or all at one end of the range) with nonzero
    residual scales;
  * asymmetric and wide-ratio base levels;
  * fp16-subnormal and 65504 group scales;
  * a lost hand-over between workgroups, forced from the host with the wait
    hooks, which must show in the workspace error word and as NaN outputs.
Each call's workspace error word is asserted to be zero afterwards.
"""
import numpy as np
import pytest

import oracle
import synth

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


def to_dev(torch, a, dt=np.int16):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to("cuda")


def block(n):
    b = 1
    while n % (2 * b) == 0 and 2 * b <= 4096:
        b *= 2
    return b


def call(nl, torch, L, x, verify):
    """One call on a fresh workspace; the error word must stay zero."""
    T = x.shape[0]
    ws = L.workspace(T)
    y = L.forward(to_dev(torch, x), verify, ws=ws)
    assert nl.nested_linear_workspace_status(ws) == 0
    return y.cpu().numpy().astype(np.float64)


def check_tokens(y, ref, what=""):
    assert y.shape == ref.shape
    for t in range(ref.shape[0]):
        m = np.abs(ref[t]).max()
        if m == 0.0:
            assert np.all(y[t] == 0.0), f"{what} token {t}: oracle zero, got max {np.abs(y[t]).max()}"
        else:
            e = np.abs(y[t] - ref[t]).max() / m
            assert e <= TOL, f"{what} token {t}: rel err {e:.3e} (max|y| {m:.3e})"


def both_modes(nl, torch, lin, x, what, modes=(False, True)):
    L = nl.Linear(lin)
    try:
        for verify in modes:
            if verify and not lin["bits"]:
                continue
            check_tokens(call(nl, torch, L, x, verify), oracle.forward(lin, x, verify),
                         f"{what} {'verify' if verify else 'draft'}")
    finally:
        L.close()


def bf16(a):
    b = synth.f32_to_bf16_bits(np.asarray(a, np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(b), np.asarray(a, np.float32)), "not exact in bf16"
    return b


# --- activations -------------------------------------------------------------

def spike_tokens(lin, cfg):
    """Seven tokens: one spike per block (x' constant over each block) at two
    magnitudes, one spike channel at either end of x, four outlier channels
    over N(0,1), plain N(0,1), and zero."""
    d_in = lin["d_in"]
    b = block(d_in)
    si = lin["sign_in"].astype(np.float32)
    X = np.zeros((7, d_in), np.float32)
    X[0, ::b] = 3.0 * si[::b]                        # x' = 3 / sqrt(b) everywhere
    X[1, ::b] = 1.0e4 * si[::b]
    X[2, 0] = -5.0
    X[3, d_in - 1] = 0.75
    r = np.random.default_rng(cfg)
    X[4] = r.standard_normal(d_in)
    ch = r.choice(d_in, 4, replace=False)
    X[4, ch] = np.array([300.0, -512.0, 1024.0, -96.0])
    X[5] = r.standard_normal(d_in)
    return bf16(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(X)))


@pytest.mark.parametrize("d_out,d_in,bits,two", [(1024, 4096, 6, False), (1024, 4096, 8, True),
                                                 (1000, 2560, 7, False), (512, 14336, 6, False)])
def test_spikes_and_outliers_per_token(nl, torch_cuda, d_out, d_in, bits, two):
    lin = synth.make_linear(d_out, d_in, bits, cfg=140, idx=d_in + bits, two_sided=two)
    x = spike_tokens(lin, d_in)
    # T = 7 (rotation workgroups), T = 2 (each workgroup rotates x itself)
    # and T = 35 (three token tiles, eight-wave form)
    both_modes(nl, torch_cuda, lin, x, "spikes T=7")
    both_modes(nl, torch_cuda, lin, x[:2], "spikes T=2")
    both_modes(nl, torch_cuda, lin, np.concatenate([x] * 5), "spikes T=35")


@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("d_in", [4096, 2560])
def test_token_magnitudes_from_1e_minus20_to_1e20(nl, torch_cuda, two, d_in):
    lin = synth.make_linear(1024, d_in, 7, cfg=141, idx=d_in, two_sided=two)
    base = synth.bf16_bits_to_f32(synth.make_x(41, d_in, cfg=141, idx=d_in)).astype(np.float64)
    X = base * (10.0 ** np.arange(-20, 21, dtype=np.float64))[:, None]
    x = synth.f32_to_bf16_bits(X.astype(np.float32))
    x[20] = 0                                         # a zero token among them
    both_modes(nl, torch_cuda, lin, x, "magnitudes T=41")
    both_modes(nl, torch_cuda, lin, x[[0, 40]], "magnitudes T=2")
    both_modes(nl, torch_cuda, lin, x[[20]], "zero T=1")
    both_modes(nl, torch_cuda, lin, x[14:30], "magnitudes T=16")


# --- residual codes ----------------------------------------------------------

@pytest.mark.parametrize("bits", [6, 7, 8])
@pytest.mark.parametrize("fill", ["zero", "min", "max"])
def test_constant_residual_codes_with_nonzero_scales(nl, torch_cuda, bits, fill):
    d_out, d_in = 512, 4096
    lin = synth.make_linear(d_out, d_in, bits, cfg=142, idx=bits, two_sided=False, keep_codes=True)
    v = {"zero": 0, "min": -(1 << (bits - 1)), "max": (1 << (bits - 1)) - 1}[fill]
    q = np.full((d_out, d_in), v, np.int8)
    lin["resid_codes"] = synth.pack_resid(q, bits)
    x = np.concatenate([spike_tokens(lin, 7)[:2], synth.make_x(14, d_in, cfg=142, idx=bits)])
    for T in (16, 1):
        both_modes(nl, torch_cuda, lin, x[:T], f"resid {fill} T={T}")
    if fill == "zero":
        # verify then equals draft within the bar, token by token
        L = nl.Linear(lin)
        try:
            yv = call(nl, torch_cuda, L, x, True)
            yd = call(nl, torch_cuda, L, x, False)
            check_tokens(yv, yd, "zero-residual verify vs draft")
        finally:
            L.close()


# --- levels ------------------------------------------------------------------

@pytest.mark.parametrize("levels", [(-3.1, -0.02, 0.7, 2.4), (-1.0, -1e-6, 1e-5, 1.0), (-1.0, -3e-8, 5e-8, 1.0),
                                    (0.0, 0.25, 0.5, 64.0), (-2.0, 0.0, 0.0, 0.0)])
def test_asymmetric_and_wide_ratio_levels(nl, torch_cuda, levels):
    lin = synth.make_linear(768, 2048, 7, cfg=143, idx=0, two_sided=False)
    lin["levels"] = np.array(levels, np.float32)
    L = nl.Linear(lin)
    try:
        err = nl.nested_linear_info(L.h)["level_rel_err"]
        assert 0.0 <= err <= 2e-3, err
    finally:
        L.close()
    x = np.concatenate([synth.make_x(5, 2048, cfg=143, idx=1), spike_tokens(lin, 3)[:3]])
    both_modes(nl, torch_cuda, lin, x, f"levels {levels}")
    both_modes(nl, torch_cuda, lin, x[:1], f"levels {levels} T=1")


def test_levels_beyond_fp16_are_rejected(nl, torch_cuda):
    lin = synth.make_linear(64, 512, 0, cfg=144, idx=0, two_sided=False)
    lin["levels"] = np.array([-1.0, 1e-12, 0.5, 1.0], np.float32)
    with pytest.raises(nl.NLError):
        nl.Linear(lin)


# --- scales ------------------------------------------------------------------

def f16_bits(v):
    return np.asarray(v, np.float16).view(np.uint16)


def scale_case(kind, shape, r):
    n = int(np.prod(shape))
    if kind == "subnormal":       # every fp16 subnormal magnitude 2^-24 .. 2^-14 - 2^-24
        return r.integers(1, 0x400, n, dtype=np.uint16).reshape(shape)
    if kind == "max":
        return np.full(shape, 0x7BFF, np.uint16)     # 65504
    if kind == "mixed":           # per group: subnormal, ordinary or 65504
        pick = r.integers(0, 3, n)
        out = np.where(pick == 0, r.integers(1, 0x400, n), np.where(pick == 1, 0x2000 + r.integers(0, 0x400, n),
                                                                     0x7BFF))
        return out.astype(np.uint16).reshape(shape)
    raise ValueError(kind)


@pytest.mark.parametrize("base_kind,resid_kind", [("subnormal", None), (None, "subnormal"), ("max", "max"),
                                                  ("subnormal", "max"), ("mixed", "mixed")])
@pytest.mark.parametrize("two", [False, True])
def test_subnormal_and_65504_scales(nl, torch_cuda, base_kind, resid_kind, two):
    d_out, d_in, bits = 1024, 4096, 8
    lin = synth.make_linear(d_out, d_in, bits, cfg=145, idx=int(two), two_sided=two)
    r = np.random.default_rng(145)
    if base_kind:
        lin["base_scales"] = scale_case(base_kind, lin["base_scales"].shape, r)
    if resid_kind:
        lin["resid_scales"] = scale_case(resid_kind, lin["resid_scales"].shape, r)
    x = np.concatenate([synth.make_x(9, d_in, cfg=145, idx=2), spike_tokens(lin, 5)[:4]])
    both_modes(nl, torch_cuda, lin, x, f"scales {base_kind}/{resid_kind}")
    both_modes(nl, torch_cuda, lin, x[:2], f"scales {base_kind}/{resid_kind} T=2")


# --- a lost hand-over ----------------------------------------------------------

# (T, verify): the single launch with rotation workgroups (verify, T = 4) and
# the staged-x' launch (verify at T = 16, the draft at any T)
@pytest.mark.parametrize("T,verify", [(4, True), (16, True), (4, False)])
@pytest.mark.parametrize("two", [False, True])
def test_lost_handover_is_reported_and_recoverable(nl, torch_cuda, two, T, verify):
    # The host raises every wait's target (wait_extra) and shortens the spin
    # limit, so each bounded wait gives up after a few thousand polls: the
    # error word counts them, the outputs those waits fed are NaN, and every
    # workgroup still exits.  Clearing the workspace then restores normal
    # calls on it.
    torch = torch_cuda
    lin = synth.make_linear(1024, 4096, 6, cfg=146, idx=int(two), two_sided=two)
    x = synth.make_x(T, 4096, cfg=146, idx=0)
    L = nl.Linear(lin)
    ws = L.workspace(T)
    xd = to_dev(torch, x)
    plan = nl.nested_linear_describe_call([1024], 4096, 6 if verify else 0, two, T)
    assert not plan["local"], plan  # a form with waits between workgroups
    try:
        nl.nested_linear_set_tuning("spin_limit", 2000)
        nl.nested_linear_set_tuning("wait_extra", 1)
        y = L.forward(xd, verify, ws=ws)
        torch.cuda.synchronize()
        err = nl.nested_linear_workspace_status(ws)
        yn = y.cpu().numpy()
    finally:
        nl.nested_linear_set_tuning("wait_extra", 0)
        nl.nested_linear_set_tuning("spin_limit", 0)
    assert err > 0
    assert np.isnan(yn).all()
    assert nl.nested_linear_workspace_status(ws, clear=True) == err
    assert nl.nested_linear_workspace_status(ws) == 0
    y = L.forward(xd, verify, ws=ws).cpu().numpy().astype(np.float64)
    assert nl.nested_linear_workspace_status(ws) == 0
    check_tokens(y, oracle.forward(lin, x, verify), "after clear")
    L.close()
