"""The forward on the library's static scratch (no allocation) against the
workspace form of the same call, through the C ABI.

Two calls in a row on the same GPU (the array keeps the last call's
contents), the second with a smaller input, each in both modes; outputs must
equal the workspace form's bit for bit (same plan, same kernels), and so also
meet the oracle bar.  A plan beyond the array's size is refused.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


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


def to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


@pytest.mark.parametrize("two", [False, True])
def test_static_scratch_forward_matches_workspace_form(nl, torch_cuda, two):
    torch = torch_cuda
    # a large call (rotation workgroups, split K), then a smaller one
    cases = [(14336, 4096, 6, 16), (1024, 2048, 8, 3)]
    for d_out, d_in, bits, T in cases:
        lin = synth.make_linear(d_out, d_in, bits, cfg=150, idx=d_out + int(two), two_sided=two)
        x = synth.make_x(T, d_in, cfg=150, idx=T)
        L = nl.Linear(lin)
        xd = to_dev(torch, x)
        ws = L.workspace(T)
        for verify in (True, False):
            want = L.forward(xd, verify, ws=ws)
            torch.cuda.synchronize()
            assert nl.nested_linear_workspace_status(ws) == 0
            y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device="cuda")
            nl.nested_linear_forward_static(L.h, verify, xd, T, y)
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            np.testing.assert_array_equal(got, want.cpu().numpy())
            ref = oracle.forward(lin, x, verify, rows=(0, min(d_out, 4096)))
            e = np.abs(got[:, :ref.shape[1]].astype(np.float64) - ref).max() / np.abs(ref).max()
            assert e <= 2e-3, e
        L.close()


def test_static_scratch_refuses_a_plan_beyond_its_size(nl, torch_cuda):
    torch = torch_cuda
    # two-sided, 131072 outputs at T = 64: the sums before the output rotation
    # alone take 64 x 131072 x 4 bytes = 32 MiB, beyond the array
    lin = synth.make_linear(131072, 128, 0, cfg=151, idx=0, two_sided=True)
    L = nl.Linear(lin)
    x = to_dev(torch, synth.make_x(64, 128, cfg=151, idx=0))
    y = torch.empty((64, 131072), dtype=torch.float32, device="cuda")
    with pytest.raises(nl.NLError) as ei:
        nl.nested_linear_forward_static(L.h, False, x, 64, y)
    assert ei.value.status == nl.NL_EUNSUPPORTED
    # a small T of the same linear fits
    nl.nested_linear_forward_static(L.h, False, x, 1, y)
    torch.cuda.synchronize()
    ref = oracle.forward(lin, synth.make_x(64, 128, cfg=151, idx=0)[:1], False, rows=(0, 4096))
    got = y[:1, :4096].cpu().numpy().astype(np.float64)
    assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max()
    L.close()
