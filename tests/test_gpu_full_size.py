"""Parity at full model sizes, on sampled outputs.

Every linear of a Llama-8B-shaped verify pass (hidden 4096, intermediate
14336, GQA kv 1024, lm_head 128256x4096; 7-bit residual, T = 16) and of the
31B-class dense shapes (hidden 5120, intermediate 25600, kv 1024; 8-bit
residual, draft at T = 1 and verify at T = 64) runs at its full size through
the single launch that bench.py times.  The linears are one-sided, so output
rows are independent: three windows of rows (the first, an unaligned one in
the middle and the last) are compared with the fp64 oracle computed for those
rows only, to the bar max|dy| <= 2e-3 * max|y_oracle| over each window.

The lm_head's codes repeat a generated 4096-row block (generating all 128256
rows costs half a minute of host time); its scales are generated for every
row, so a row read from the wrong place still changes the output.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3

LLAMA8B = [("q/o", 4096, 4096), ("k/v", 1024, 4096), ("gate/up", 14336, 4096), ("down", 4096, 14336),
           ("lm_head", 128256, 4096)]
DENSE31B = [("q/o", 5120, 5120), ("k/v", 1024, 5120), ("gate/up", 25600, 5120), ("down", 5120, 25600)]


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


def windows(d_out, n=64):
    mid = d_out // 2 - 37
    return [(0, n), (mid, mid + n), (d_out - n, d_out)]


def make_linear(d_out, d_in, bits, cfg, idx, tile=4096):
    if d_out <= 2 * tile:
        return synth.make_linear(d_out, d_in, bits, cfg=cfg, idx=idx, two_sided=False)
    lin = dict(synth.make_linear(tile, d_in, bits, cfg=cfg, idx=idx, two_sided=False))
    reps = -(-d_out // tile)
    lin["d_out"] = d_out
    for k in ("base_codes", "resid_codes"):
        lin[k] = np.ascontiguousarray(np.tile(lin[k], (reps, 1, 1))[:d_out])
    lin["base_scales"] = synth.make_scales(d_out, d_in, cfg, idx, synth.STREAM_BASE_SCALE)
    lin["resid_scales"] = synth.make_scales(d_out, d_in, cfg, idx, synth.STREAM_RESID_SCALE)
    return lin


def check_sampled(nl, torch, lin, x, runs):
    """runs: [(T, verify)]; x holds max(T) rows."""
    L = nl.Linear(lin)
    try:
        ws = L.workspace(max(T for T, _ in runs))
        for T, verify in runs:
            xd = torch.from_numpy(np.ascontiguousarray(x[:T]).view(np.int16)).cuda()
            y = L.forward(xd, verify, ws=ws)
            torch.cuda.synchronize()
            y = y.cpu().numpy()
            assert np.isfinite(y).all()
            for r0, r1 in windows(lin["d_out"]):
                ref = oracle.forward(lin, x[:T], verify, rows=(r0, r1))
                err = float(np.abs(y[:, r0:r1].astype(np.float64) - ref).max() / np.abs(ref).max())
                assert err <= TOL, (lin["d_out"], lin["d_in"], T, verify, r0, err)
    finally:
        L.close()


@pytest.mark.parametrize("name,d_out,d_in", LLAMA8B, ids=[s[0] for s in LLAMA8B])
def test_llama8b_shaped_verify_7bit_T16(nl, torch_cuda, name, d_out, d_in):
    idx = [s[0] for s in LLAMA8B].index(name)
    lin = make_linear(d_out, d_in, 7, cfg=2, idx=idx, tile=4096 if name == "lm_head" else d_out)
    x = synth.make_x(16, d_in, cfg=2, idx=100 + idx)
    check_sampled(nl, torch_cuda, lin, x, [(16, True)])


@pytest.mark.parametrize("name,d_out,d_in", DENSE31B, ids=[s[0] for s in DENSE31B])
def test_31b_class_draft_T1_verify_T64_8bit(nl, torch_cuda, name, d_out, d_in):
    idx = [s[0] for s in DENSE31B].index(name)
    lin = make_linear(d_out, d_in, 8, cfg=3, idx=idx, tile=d_out)
    x = synth.make_x(64, d_in, cfg=3, idx=100 + idx)
    check_sampled(nl, torch_cuda, lin, x, [(1, False), (64, True)])
