"""The kernel-timing hook: dispatch-attached events around each single launch."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def test_timing_records_eager_launches_only():
    import torch
    import bit_nested_quantized_amd as nl
    lin = synth.make_linear(1024, 1024, 8, cfg=0, idx=0, two_sided=False)
    L = nl.Linear(lin)
    x = torch.from_numpy(synth.make_x(4, 1024, cfg=0, idx=0).view(np.int16)).cuda()
    ws = L.workspace(4)
    y = torch.empty((4, 1024), dtype=torch.float32, device="cuda")
    ref = L.forward(x, True, ws=ws).clone()
    # a captured launch is not recorded and does not use up a slot
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    nl.nested_linear_timing_begin(3)
    with torch.cuda.graph(g, stream=s):
        nl.nested_linear_verify(L.h, x, 4, y, ws, torch.cuda.current_stream())
    for _ in range(5):
        nl.nested_linear_verify(L.h, x, 4, y, ws)
    us = nl.nested_linear_timing_end(8)
    assert len(us) == 3, us                      # capacity 3: the first three eager launches
    assert all(0.5 < u < 1e5 for u in us), us    # microseconds of kernel time
    torch.cuda.synchronize()
    assert torch.equal(y, ref)                   # timing changes no result
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
