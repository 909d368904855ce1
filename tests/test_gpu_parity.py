"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: code unpacking bit-exact; outputs max|dy| <= 2e-3 * max|y_oracle|
over all T x d_out outputs of a call (fp32 accumulation, bf16 activations).
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


def rel_err(y, ref):
    return float(np.abs(y.astype(np.float64) - ref).max() / max(np.abs(ref).max(), 1e-300))


# White box: every workspace starts with a 1 MiB region of counters, zero
# between calls; x' follows it.
COUNTER_BYTES = 1 << 20


def block(n):
    b = 1
    while n % (2 * b) == 0 and 2 * b <= 4096:
        b *= 2
    return b


def run(nl, torch, lin, x, verify, L=None):
    L = L or nl.Linear(lin)
    ws = L.workspace(x.shape[0])
    y = L.forward(to_dev(torch, x), verify, ws=ws)
    torch.cuda.synchronize()
    assert nl.nested_linear_workspace_status(ws) == 0   # no wait gave up
    return y.cpu().numpy()


# --- unpacking: bit-exact --------------------------------------------------------

@pytest.mark.parametrize("bits", [0, 6, 7, 8])
def test_decode_every_pattern_every_position(nl, torch_cuda, bits):
    torch = torch_cuda
    nb = bits if bits else 2
    n = 1 << nb
    rows = max(n, 16) + 5                               # ragged last tile
    r = np.arange(rows)[:, None]
    p = np.arange(640)[None, :]                         # 5 groups: a ragged chunk
    codes = ((r + p) % 4).astype(np.uint8)
    lin = synth.make_linear(rows, 640, bits, cfg=50, idx=bits)
    lin["base_codes"] = synth.pack_base(codes)
    if bits:
        q = ((r + p) % n) - n // 2
        lin["resid_codes"] = synth.pack_resid(q, bits)
    L = nl.Linear(lin)
    for row0, nrows in [(0, rows), (3, 17), (rows - 1, 1)]:
        bi = torch.zeros((nrows, 640), dtype=torch.uint8, device="cuda")
        rq = torch.zeros((nrows, 640), dtype=torch.int8, device="cuda")
        nl.nested_linear_decode(L.h, row0, nrows, bi, rq)
        torch.cuda.synchronize()
        ob, orq = oracle.decode(lin, row0, nrows)
        np.testing.assert_array_equal(bi.cpu().numpy(), ob)
        if bits:
            np.testing.assert_array_equal(rq.cpu().numpy(), orq)


def test_decode_random_linear(nl, torch_cuda):
    lin = synth.make_linear(200, 1536, 7, cfg=51, idx=0)
    L = nl.Linear(lin)
    torch = torch_cuda
    bi = torch.zeros((200, 1536), dtype=torch.uint8, device="cuda")
    rq = torch.zeros((200, 1536), dtype=torch.int8, device="cuda")
    nl.nested_linear_decode(L.h, 0, 200, bi, rq)
    torch.cuda.synchronize()
    ob, orq = oracle.decode(lin)
    np.testing.assert_array_equal(bi.cpu().numpy(), ob)
    np.testing.assert_array_equal(rq.cpu().numpy(), orq)


def test_level_table_is_near_exact(nl, torch_cuda):
    L = nl.Linear(synth.make_linear(16, 128, 0, cfg=52, idx=0))
    info = nl.nested_linear_info(L.h)
    assert info["level_rel_err"] < 2e-5
    assert info["block_in"] == 128 and info["block_out"] == 16


# --- the input rotation (white box: the workspace holds x' as fp16 * 2^s) ----------

def test_prepare_input_matches_oracle_rotation(nl, torch_cuda):
    torch = torch_cuda
    d_in, T = 14336, 5                                  # block 2048, 7 blocks, 28 chunks
    lin = synth.make_linear(64, d_in, 6, cfg=53, idx=0)
    x = synth.make_x(T, d_in, cfg=53, idx=0, scale=3.0)
    L = nl.Linear(lin)
    ws = L.workspace(T)
    nl.nested_linear_prepare_input(L.h, to_dev(torch, x), T, ws)
    torch.cuda.synchronize()
    nch = d_in // 512
    o_xh = COUNTER_BYTES
    # x' is row-major fp16 [T][Kp], Kp = chunks * 512 (= d_in here)
    xh = ws[o_xh: o_xh + T * d_in * 2].view(torch.float16).float().cpu().numpy().reshape(T, d_in)
    o_meta = o_xh + (T * d_in * 2 + 255) // 256 * 256
    meta = ws[o_meta: o_meta + T * nch * 20].view(torch.float32).reshape(nch, 5, T).cpu().numpy()
    xs, tsc = meta[:, :4, :], meta[:, 4, :]
    got = xh * np.repeat(tsc.T, 512, axis=1)
    ref = oracle.rotate_input(lin, x)
    for t in range(T):
        for c in range(nch):
            seg = slice(512 * c, 512 * (c + 1))
            m = np.abs(ref[t, seg]).max()
            assert np.abs(got[t, seg] - ref[t, seg]).max() <= m * 2.0 ** -11
            # the chunk's scaled maximum lands in [2^14, 2^15]
            assert 2 ** 14 <= np.abs(xh[t, seg]).max() <= 2 ** 15
    gsum = xh.reshape(T, nch, 4, 128)
    want = gsum.sum(-1).transpose(1, 2, 0)
    assert np.all(np.abs(xs - want) <= 1e-6 * np.abs(gsum).sum(-1).transpose(1, 2, 0) + 1e-6)


# --- end-to-end parity ---------------------------------------------------------

@pytest.mark.parametrize("T", [1, 16])
@pytest.mark.parametrize("verify", [False, True])
def test_single_1024_int8(nl, torch_cuda, T, verify):
    # 1024 x 1024, int8 residual, T = 1 and 16: the small single-linear workload
    lin = synth.make_linear(1024, 1024, 8, cfg=0, idx=0)
    x = synth.make_x(T, 1024, cfg=0, idx=T)
    y = run(nl, torch_cuda, lin, x, verify)
    assert rel_err(y, oracle.forward(lin, x, verify)) <= TOL


SHAPES = [
    # d_out, d_in, bits, T, two-sided
    (64, 512, 6, 1, True),
    (48, 384, 7, 5, False),     # block 128, one partial chunk
    (100, 640, 8, 17, True),    # ragged rows (block_out 4), two token tiles
    (1000, 1152, 6, 33, True),  # block_in 128, ragged tile, three token tiles
    (256, 2048, 7, 64, True),   # four token tiles
    (512, 2048, 8, 48, False),
    (4096, 4096, 6, 16, True),
    (2048, 5120, 8, 64, True),  # block_in 1024
]


@pytest.mark.parametrize("d_out,d_in,bits,T,two", SHAPES)
@pytest.mark.parametrize("verify", [False, True])
def test_shapes(nl, torch_cuda, d_out, d_in, bits, T, two, verify):
    lin = synth.make_linear(d_out, d_in, bits, cfg=60, idx=d_out + d_in, two_sided=two)
    x = synth.make_x(T, d_in, cfg=60, idx=T)
    y = run(nl, torch_cuda, lin, x, verify)
    assert rel_err(y, oracle.forward(lin, x, verify)) <= TOL


CFG1 = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]


@pytest.mark.parametrize("d_out,d_in", CFG1)
def test_llama8b_projections_6bit(nl, torch_cuda, d_out, d_in):
    # 7B/8B-class projections, 6-bit residual, draft and verify at T = 1..32
    torch = torch_cuda
    lin = synth.make_linear(d_out, d_in, 6, cfg=1, idx=d_out * 7 + d_in)
    x = synth.make_x(32, d_in, cfg=1, idx=d_in)
    L = nl.Linear(lin)
    ws = L.workspace(32)
    xd = to_dev(torch, x)
    for verify in (False, True):
        ref = oracle.forward(lin, x, verify)
        for T in (1, 4, 8, 16, 32):
            y = L.forward(xd[:T].contiguous(), verify, ws=ws).cpu().numpy()
            e = rel_err(y, ref[:T])
            assert e <= TOL, (verify, T, e)


# --- properties ----------------------------------------------------------------

@pytest.mark.parametrize("bits", [6, 7, 8])
def test_nesting_zero_residual_equals_draft_bitwise(nl, torch_cuda, bits):
    lin = synth.make_linear(512, 2048, bits, cfg=61, idx=bits)
    zs = dict(lin, resid_scales=np.zeros_like(lin["resid_scales"]))
    x = synth.make_x(12, 2048, cfg=61, idx=bits)
    d = run(nl, torch_cuda, lin, x, False)
    v0 = run(nl, torch_cuda, zs, x, True)
    np.testing.assert_array_equal(v0, d)


def test_repeat_runs_are_bitwise_identical(nl, torch_cuda):
    torch = torch_cuda
    lin = synth.make_linear(4096, 4096, 7, cfg=62, idx=0)
    x = to_dev(torch, synth.make_x(16, 4096, cfg=62, idx=0))
    L = nl.Linear(lin)
    ws = L.workspace(16)
    a = L.forward(x, True, ws=ws).cpu().numpy()
    for _ in range(3):
        np.testing.assert_array_equal(L.forward(x, True, ws=ws).cpu().numpy(), a)


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("two", [False, True])
def test_staged_calls_and_fused_call_match_oracle(nl, torch_cuda, T, two):
    # The staged kernels rotate x in their own launch and split K their own
    # way; both paths are held to the oracle.
    torch = torch_cuda
    lin = synth.make_linear(2048, 4096, 8, cfg=63, idx=T, two_sided=two)
    xh = synth.make_x(T, 4096, cfg=63, idx=T)
    x = to_dev(torch, xh)
    L = nl.Linear(lin)
    ws = L.workspace(T)
    a = L.forward(x, True, ws=ws)
    y = torch.empty_like(a)
    nl.nested_linear_prepare_input(L.h, x, T, ws)
    nl.nested_linear_contract(L.h, True, T, y, ws)
    nl.nested_linear_finish(L.h, T, y, ws)
    torch.cuda.synchronize()
    ref = oracle.forward(lin, xh, True)
    assert rel_err(a.cpu().numpy(), ref) <= TOL
    assert rel_err(y.cpu().numpy(), ref) <= TOL


def test_unit_column_closed_form(nl, torch_cuda):
    # x = S_i H_i e_j makes the one-sided output column j of W~.
    torch = torch_cuda
    d_in = 1024
    lin = synth.make_linear(256, d_in, 8, cfg=64, idx=0, two_sided=False, keep_codes=True)
    H = np.ones((1, 1))
    while H.shape[0] < d_in:
        H = np.block([[H, H], [H, -H]])
    js = [0, 3, 1023]
    X = (H[:, js].T / 32.0) * lin["sign_in"]
    xb = synth.f32_to_bf16_bits(X.astype(np.float32))
    y = run(nl, torch, lin, xb, True)
    g_of_k = np.arange(d_in) // 128
    W = lin["levels"].astype(np.float64)[lin["base_idx"]] * lin["base_scales"].view(np.float16).astype(np.float64)[:, g_of_k]
    W += lin["resid_q"] * lin["resid_scales"].view(np.float16).astype(np.float64)[:, g_of_k]
    for t, j in enumerate(js):
        assert np.abs(y[t] - W[:, j]).max() <= TOL * np.abs(W[:, j]).max()


# --- error paths on the device ---------------------------------------------------

def test_call_errors(nl, torch_cuda):
    torch = torch_cuda
    lin = synth.make_linear(64, 512, 6, cfg=65, idx=0)
    L = nl.Linear(lin)
    x = to_dev(torch, synth.make_x(4, 512, cfg=65, idx=0))
    y = torch.empty((4, 64), dtype=torch.float32, device="cuda")
    ws = L.workspace(4)
    with pytest.raises(nl.NLError) as e:
        nl.nested_linear_verify(L.h, x, 0, y, ws)
    assert e.value.status == nl.NL_EINVAL
    with pytest.raises(nl.NLError) as e:
        nl.nested_linear_verify(L.h, x, 65, y, ws)
    assert e.value.status == nl.NL_EUNSUPPORTED
    with pytest.raises(nl.NLError) as e:
        nl.nested_linear_verify(L.h, x, 4, y, ws[:128])
    assert e.value.status == nl.NL_EINVAL
    D = nl.Linear(synth.make_linear(64, 512, 0, cfg=65, idx=1))
    with pytest.raises(nl.NLError):
        nl.nested_linear_verify(D.h, x, 4, y, D.workspace(4))
    bad = synth.make_linear(64, 512, 6, cfg=65, idx=2)
    bad["sign_in"] = bad["sign_in"].copy()
    bad["sign_in"][7] = 0
    with pytest.raises(nl.NLError) as e:
        nl.Linear(bad)
    assert e.value.status == nl.NL_EINVAL
    with pytest.raises(nl.NLError):
        nl.nested_linear_decode(L.h, 60, 10, torch.zeros((10, 512), dtype=torch.uint8, device="cuda"), None)


# --- single-launch hand-over: one workspace across shapes and modes -------------

# (d_out, d_in, bits, two-sided): direct store, split-K reduction, two-sided
# with one and with several output superblocks
MIXED = [(1024, 4096, 6, False), (4096, 4096, 6, True), (14336, 4096, 7, True),
         (3000, 1536, 8, False), (256, 512, 8, True)]


def test_one_workspace_many_calls_counters_return_to_zero(nl, torch_cuda):
    torch = torch_cuda
    Ls, xs, lins = [], [], []
    for i, (o, d, b, two) in enumerate(MIXED):
        lin = synth.make_linear(o, d, b, cfg=66, idx=i, two_sided=two)
        lins.append(lin)
        Ls.append(nl.Linear(lin))
        xs.append(synth.make_x(64, d, cfg=66, idx=i))
    n = max(nl.nested_linear_workspace_bytes(L.h, 64) for L in Ls)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for i, (o, d, b, two) in enumerate(MIXED):
            for T in (1, 16, 64) if rnd == 0 else (7,):
                for verify in (False, True):
                    x = xs[i][:T]
                    y = Ls[i].forward(to_dev(torch, x), verify, ws=ws).cpu().numpy()
                    e = rel_err(y, oracle.forward(lins[i], x, verify))
                    assert e <= TOL, (o, d, b, two, T, verify, e)
                    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0, (o, d, T, verify)


def test_split_k_shape_matches_oracle(nl, torch_cuda):
    # every split count gives the same result within the bar
    torch = torch_cuda
    lin = synth.make_linear(512, 4096, 6, cfg=67, idx=0)
    x = synth.make_x(16, 4096, cfg=67, idx=0)
    ref = oracle.forward(lin, x, True)
    y = run(nl, torch, lin, x, True)
    assert rel_err(y, ref) <= TOL


@pytest.mark.parametrize("T", [12, 24])
@pytest.mark.parametrize("two", [False, True])
def test_staged_eight_tile_waves_knob(nl, torch_cuda, T, two):
    # the staged launch with eight tile waves at one and two token tiles (a
    # tuning knob; by default only short grouped linears take it): split
    # counts double, the output superblocks of the two-sided form hold more
    # row blocks
    torch = torch_cuda
    lin = synth.make_linear(2048, 4096, 6, cfg=71, idx=0, two_sided=two)
    x = synth.make_x(T, 4096, cfg=71, idx=0)
    nl.nested_linear_set_tuning("staged_waves", 8)
    try:
        for verify in (True, False):
            y = run(nl, torch, lin, x, verify)
            assert rel_err(y, oracle.forward(lin, x, verify)) <= TOL
    finally:
        nl.nested_linear_set_tuning("staged_waves", 0)


# --- linears that share x in one call (*_multi) ------------------------------------

def run_multi(nl, torch, lins, x, verify):
    Ls = [nl.Linear(lin) for lin in lins]
    hs = [L.h for L in Ls]
    T = x.shape[0]
    ws = torch.zeros(nl.nested_linear_multi_workspace_bytes(hs, T), dtype=torch.uint8, device="cuda")
    ys = [torch.full((T, lin["d_out"]), float("nan"), dtype=torch.float32, device="cuda") for lin in lins]
    fn = nl.nested_linear_verify_multi if verify else nl.nested_linear_draft_multi
    xd = to_dev(torch, x)
    fn(hs, xd, T, ys, ws)
    fn(hs, xd, T, ys, ws)   # the same workspace again
    torch.cuda.synchronize()
    assert nl.nested_linear_workspace_status(ws) == 0
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    out = [y.cpu().numpy() for y in ys]
    del Ls
    return out


@pytest.mark.parametrize("T", [1, 3, 16, 40])
@pytest.mark.parametrize("two", [False, True])
def test_multi_linears_of_several_shapes(nl, torch_cuda, T, two):
    # q/k/v-like: three linears of different d_out on one x, each with its own signs and levels
    lins = [synth.make_linear(o, 1024, 6, cfg=72, idx=i, two_sided=two) for i, o in enumerate((768, 256, 256))]
    x = synth.make_x(T, 1024, cfg=72, idx=T)
    for verify in (True, False):
        ys = run_multi(nl, torch_cuda, lins, x, verify)
        for lin, y in zip(lins, ys):
            assert rel_err(y, oracle.forward(lin, x, verify)) <= TOL


@pytest.mark.parametrize("d_out,d_in", [(768, 1024), (2048, 512)])
@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("T", [1, 17, 40, 64])
def test_multi_linears_of_one_shape_staged(nl, torch_cuda, d_out, d_in, n, T):
    # gate/up-like: linears of one shape through the staged launch's grouped
    # form (forced from T = 1 by the thresholds), each writing its own y: with
    # K split (768x1024) and without (2048x512, one chunk)
    lins = [synth.make_linear(d_out, d_in, 7, cfg=73, idx=i) for i in range(n)]
    x = synth.make_x(T, d_in, cfg=73, idx=T)
    nl.nested_linear_set_tuning("multi_staged_t_verify", 1)
    nl.nested_linear_set_tuning("multi_staged_t_draft", 1)
    try:
        for verify in (True, False):
            ys = run_multi(nl, torch_cuda, lins, x, verify)
            for lin, y in zip(lins, ys):
                assert rel_err(y, oracle.forward(lin, x, verify)) <= TOL
    finally:
        nl.nested_linear_set_tuning("multi_staged_t_verify", 0)
        nl.nested_linear_set_tuning("multi_staged_t_draft", 0)


# --- grouped mixture-of-experts projections ---------------------------------------

def make_moe(n_exp, d_out, d_in, bits, T, k, rho, two, cfg, shared=True):
    experts = [synth.make_linear(d_out, d_in, bits, cfg=cfg, idx=e, two_sided=two)
               for e in range(n_exp + int(shared))]
    _, pt, off = synth.router_topk(T, n_exp, k, rho, cfg=cfg, idx=0)
    if shared:  # the shared expert takes every token, after the routed ones
        pt = np.concatenate([pt, np.arange(T, dtype=np.int32)])
        off = np.concatenate([off, [off[-1] + T]]).astype(np.int32)
    return experts, pt.astype(np.int32), off


def run_grouped(nl, torch, experts, pt, off, x, verify, T=None):
    """One grouped call twice on one workspace.  x holds x_rows rows (tokens,
    or one per pair); T bounds the pairs of any one expert (default x_rows)."""
    Ls = [nl.Linear(e) for e in experts]
    g = nl.nested_linear_group_create([L.h for L in Ls])
    try:
        P, x_rows = len(pt), x.shape[0]
        T = x_rows if T is None else T
        ws = torch.zeros(nl.nested_linear_group_workspace_bytes(g, P), dtype=torch.uint8, device="cuda")
        y = torch.full((P, experts[0]["d_out"]), float("nan"), dtype=torch.float32, device="cuda")
        fn = nl.nested_linear_verify_grouped if verify else nl.nested_linear_draft_grouped
        pt_d = torch.from_numpy(pt).to("cuda")
        off_d = torch.from_numpy(off).to("cuda")
        xd = to_dev(torch, x)
        fn(g, pt_d, off_d, P, xd, x_rows, T, y, ws)
        a = y.cpu().numpy()
        fn(g, pt_d, off_d, P, xd, x_rows, T, y, ws)   # same workspace again
        b = y.cpu().numpy()
        torch.cuda.synchronize()
        assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
        return a, b, ws
    finally:
        nl.nested_linear_group_destroy(g)


@pytest.mark.parametrize("d_out,d_in", [(512, 2048), (1024, 2048), (2048, 512)])
@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("verify", [False, True])
def test_grouped_moe_block(nl, torch_cuda, d_out, d_in, two, verify):
    # 64 routed experts + 1 shared, top-8 routing of a 16-token block with
    # correlated logits (rho = 0.62), 8-bit residual
    experts, pt, off = make_moe(64, d_out, d_in, 8, 16, 8, 0.62, two, cfg=70 + d_out % 7)
    x = synth.make_x(16, d_in, cfg=70, idx=d_in)
    a, b, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
    ref = oracle.forward_grouped(experts, pt, off, x, verify)
    assert rel_err(a, ref) <= TOL
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("rho", [0.0, 0.9])
def test_grouped_routing_mixes(nl, torch_cuda, rho):
    experts, pt, off = make_moe(32, 256, 1024, 7, 16, 4, rho, True, cfg=71)
    x = synth.make_x(16, 1024, cfg=71, idx=int(rho * 10))
    a, _, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, True)
    assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, True)) <= TOL


def test_grouped_many_tokens_per_expert(nl, torch_cuda):
    # 40 tokens, top-2 of 6 experts: experts get up to 40 rows (3 token tiles)
    experts, pt, off = make_moe(6, 384, 1536, 6, 40, 2, 0.3, False, cfg=72)
    x = synth.make_x(40, 1536, cfg=72, idx=0)
    for verify in (False, True):
        a, _, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
        assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, verify)) <= TOL


def test_grouped_single_expert_equals_single_linear(nl, torch_cuda):
    # one expert holding every token: the grouped and the single-linear call
    # both match the oracle
    torch = torch_cuda
    lin = synth.make_linear(1024, 2048, 8, cfg=73, idx=0)
    x = synth.make_x(16, 2048, cfg=73, idx=0)
    pt = np.arange(16, dtype=np.int32)
    off = np.array([0, 16], dtype=np.int32)
    a, _, _ = run_grouped(nl, torch, [lin], pt, off, x, True)
    y = run(nl, torch, lin, x, True)
    ref = oracle.forward(lin, x, True)
    assert rel_err(a, ref) <= TOL and rel_err(y, ref) <= TOL


def test_grouped_partial_workgroups(nl, torch_cuda):
    # 14 pairs over 1024-wide blocks: the rotation and finish workgroups (4
    # tasks each) end half full, so lanes without a task run in every role
    experts, pt, off = make_moe(5, 1024, 1024, 6, 7, 1, 0.5, True, cfg=74)
    x = synth.make_x(7, 1024, cfg=74, idx=0)
    assert len(pt) % 4 != 0
    for verify in (False, True):
        a, _, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
        assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, verify)) <= TOL


@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("T", [16, 2])
def test_grouped_down_projection_per_pair_rows(nl, torch_cuda, two, T):
    # The MoE down projection: each pair's own 512-wide activation, so x has
    # one row per pair (pair_token = 0..P-1) while no expert gets more than T
    # pairs.  64 routed experts, top-8 of a T-token block plus the shared
    # expert: P = 9 T rows of x.
    experts, pt, off = make_moe(64, 2048, 512, 8, T, 8, 0.62, two, cfg=77 + T)
    P = len(pt)
    assert P == 9 * T
    xp = synth.make_x(P, 512, cfg=77, idx=T)
    ident = np.arange(P, dtype=np.int32)
    for verify in (False, True):
        a, b, _ = run_grouped(nl, torch_cuda, experts, ident, off, xp, verify, T=T)
        assert rel_err(a, oracle.forward_grouped(experts, ident, off, xp, verify)) <= TOL
        np.testing.assert_array_equal(a, b)
        # pair p of expert e is expert e applied to x row p
        e = int(np.searchsorted(off, P - 1, side="right") - 1)
        ref = oracle.forward(experts[e], xp[P - 1:P], verify)
        assert rel_err(a[P - 1:P], ref) <= TOL


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("two", [False, True])
def test_grouped_few_tokens(nl, torch_cuda, T, two):
    # with at most 2 tokens each contraction workgroup rotates its expert's
    # rows itself (T = 2 is that form's limit); T = 4 takes the rotation
    # workgroups
    experts, pt, off = make_moe(16, 512, 2048, 8, T, 4, 0.62, two, cfg=75 + T)
    x = synth.make_x(T, 2048, cfg=75, idx=T)
    for verify in (False, True):
        a, b, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
        assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, verify)) <= TOL
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("d_out", [384, 100])
@pytest.mark.parametrize("two", [False, True])
def test_grouped_two_token_tiles_short_experts(nl, torch_cuda, two, d_out):
    # 24 tokens, top-4 of 16 experts + shared, K of two chunks: experts hold
    # up to 24 rows (two token tiles) and the workgroups run eight tile waves
    # (100 rows: a ragged last tile and idle tile waves)
    experts, pt, off = make_moe(16, d_out, 1024, 7, 24, 4, 0.5, two, cfg=77)
    x = synth.make_x(24, 1024, cfg=77, idx=0)
    assert max(np.diff(off)) > 16
    for verify in (False, True):
        a, b, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
        assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, verify)) <= TOL
        np.testing.assert_array_equal(a, b)


def test_grouped_many_experts_few_active(nl, torch_cuda):
    # 600 experts (8 distinct weight sets, expert e holds set e % 8), rows
    # only at experts 3, 511, 512 and 598: the grid has one slot per pair at
    # most and each slot finds its expert past the first 512 as well
    base = [synth.make_linear(256, 256, 6, cfg=76, idx=i) for i in range(8)]
    experts = [base[e % 8] for e in range(600)]
    rows = {3: [0, 1], 511: [2], 512: [0, 3], 598: [1, 2, 3]}
    pt = np.array([t for e in sorted(rows) for t in rows[e]], dtype=np.int32)
    counts = np.zeros(600, np.int32)
    for e, ts in rows.items():
        counts[e] = len(ts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.make_x(4, 256, cfg=76, idx=0)
    for verify in (False, True):
        a, b, _ = run_grouped(nl, torch_cuda, experts, pt, off, x, verify)
        assert rel_err(a, oracle.forward_grouped(experts, pt, off, x, verify)) <= TOL
        np.testing.assert_array_equal(a, b)


def test_misaligned_x_is_rejected(nl, torch_cuda):
    torch = torch_cuda
    lin = synth.make_linear(256, 256, 6, cfg=0, idx=5)
    L = nl.Linear(lin)
    x = torch.zeros(4 * 256 + 8, dtype=torch.int16, device="cuda")
    ws = L.workspace(4)
    y = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    lib = nl.lib()
    import ctypes
    base = x.data_ptr()
    st = lib.nested_linear_verify(L.h, ctypes.c_void_p(base + 2), 4, ctypes.c_void_p(y.data_ptr()),
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == nl.NL_EINVAL and b"16-byte" in lib.nested_linear_last_error()
    assert lib.nested_linear_verify(L.h, ctypes.c_void_p(base + 16), 4, ctypes.c_void_p(y.data_ptr()),
                                    ctypes.c_void_p(ws.data_ptr()), ws.numel(), None) == nl.NL_OK
    torch.cuda.synchronize()
