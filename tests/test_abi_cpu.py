"""The C-ABI library loads, exports every symbol include/*.h declares, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import glob
import os
import re

import pytest

import bit_nested_quantized_amd as nl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"\b(nested_(?:linear|encode|w4w8|tree|kv)\w*)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    L = nl.lib()
    names = declared_symbols()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert names == set(nl.EXPORTS)


def test_last_error_is_empty_string_initially():
    assert isinstance(nl.lib().nested_linear_last_error(), bytes)


def _status(fn, *args):
    return getattr(nl.lib(), fn)(*args)


def test_create_rejects_null_and_bad_shapes():
    L = nl.lib()
    h = ctypes.c_void_p()
    assert L.nested_linear_create(None, ctypes.byref(h)) == nl.NL_EINVAL
    for d_out, d_in, bits in [(0, 1024, 8), (16, 100, 8), (16, 0, 8), (16, 1024, 5), (16, 1024, 9)]:
        d = nl.nl_desc(d_out, d_in, bits, 1, 1, 1, 1, 1, None, (ctypes.c_float * 4)(-1.5, -.5, .5, 1.5))
        assert L.nested_linear_create(ctypes.byref(d), ctypes.byref(h)) == nl.NL_EINVAL
        assert L.nested_linear_last_error()
    # residual arrays missing / present with bits == 0
    d = nl.nl_desc(16, 1024, 8, 1, 1, None, None, 1, None, (ctypes.c_float * 4)(-1.5, -.5, .5, 1.5))
    assert L.nested_linear_create(ctypes.byref(d), ctypes.byref(h)) == nl.NL_EINVAL
    d = nl.nl_desc(16, 1024, 0, 1, 1, 1, 1, 1, None, (ctypes.c_float * 4)(-1.5, -.5, .5, 1.5))
    assert L.nested_linear_create(ctypes.byref(d), ctypes.byref(h)) == nl.NL_EINVAL
    # non-finite level
    d = nl.nl_desc(16, 1024, 0, 1, 1, None, None, 1, None, (ctypes.c_float * 4)(-1.5, float("nan"), .5, 1.5))
    assert L.nested_linear_create(ctypes.byref(d), ctypes.byref(h)) == nl.NL_EINVAL
    assert b"level" in L.nested_linear_last_error()


def test_create_rejects_levels_fp16_cannot_hold():
    # one common rescale puts the largest level in [1024, 2048); a level 1e12
    # times smaller is below fp16's smallest subnormal whatever the rescale
    # (relative error 1).  The check runs before any device pointer is read.
    L = nl.lib()
    h = ctypes.c_void_p()
    for lv in [(-1.0, 1e-12, 0.5, 1.0), (-3e4, -2.0, 1e-9, 5e-4)]:
        d = nl.nl_desc(16, 1024, 0, 1, 1, None, None, 1, None, (ctypes.c_float * 4)(*lv))
        assert L.nested_linear_create(ctypes.byref(d), ctypes.byref(h)) == nl.NL_EUNSUPPORTED
        assert b"ratio" in L.nested_linear_last_error()


def test_calls_reject_invalid_handles():
    L = nl.lib()
    n = ctypes.c_size_t()
    bogus = ctypes.c_void_p(0)
    assert L.nested_linear_destroy(bogus) == nl.NL_EINVAL
    assert L.nested_linear_workspace_bytes(bogus, 16, ctypes.byref(n)) == nl.NL_EINVAL
    assert L.nested_linear_verify(bogus, 1, 16, 1, 1, 1 << 20, None) == nl.NL_EINVAL
    assert L.nested_linear_draft(bogus, 1, 16, 1, 1, 1 << 20, None) == nl.NL_EINVAL
    assert L.nested_linear_decode(bogus, 0, 1, 1, 1, None) == nl.NL_EINVAL
    assert L.nested_linear_group_destroy(bogus) == nl.NL_EINVAL
    g = ctypes.c_void_p()
    assert L.nested_linear_group_create(None, 0, ctypes.byref(g)) == nl.NL_EINVAL
    arr = (ctypes.c_void_p * 1)(None)
    assert L.nested_linear_group_create(arr, 1, ctypes.byref(g)) == nl.NL_EINVAL
    assert L.nested_linear_info(bogus, None, None, None, None, None, None) == nl.NL_EINVAL


def test_binding_raises_nlerror():
    with pytest.raises(nl.NLError) as ei:
        nl.nested_linear_destroy(ctypes.c_void_p(0))
    assert ei.value.status == nl.NL_EINVAL


def test_timing_rejects_bad_use():
    # no HIP call is made on these paths
    L = nl.lib()
    n = ctypes.c_int32(7)
    buf = (ctypes.c_float * 4)()
    assert L.nested_linear_timing_end(buf, 4, ctypes.byref(n)) == nl.NL_EINVAL  # end without begin
    assert b"not begun" in L.nested_linear_last_error()
    assert L.nested_linear_timing_begin(0) == nl.NL_EINVAL
    assert L.nested_linear_timing_begin(-3) == nl.NL_EINVAL


def test_encoder_rejects_bad_arguments_without_touching_the_gpu():
    L = nl.lib()
    lev = (ctypes.c_float * 4)(-1.5, -0.45, 0.45, 1.5)
    sz = ctypes.c_size_t()
    # shapes
    for d_out, d_in in [(0, 128), (4, 100), (4, 0), (-1, 256)]:
        assert L.nested_encode_workspace_bytes(d_out, d_in, 1, ctypes.byref(sz)) == nl.NL_EINVAL
        assert L.nested_encode_rotate(d_out, d_in, 16, 16, None, 4096, None) == nl.NL_EINVAL
        assert L.nested_linear_last_error()
    assert L.nested_encode_workspace_bytes(4, 256, 0, ctypes.byref(sz)) == nl.NL_OK and sz.value == 0
    assert L.nested_encode_workspace_bytes(4, 256, 1, ctypes.byref(sz)) == nl.NL_OK and sz.value == 8 * 4 * 256
    # codes descriptor: bits, levels, missing or extra residual arrays, alignment
    bad = [nl.nl_codes(4, 256, 5, lev, 16, 16, 16, 16),
           nl.nl_codes(4, 256, 7, (ctypes.c_float * 4)(-1.5, 0.45, -0.45, 1.5), 16, 16, 16, 16),
           nl.nl_codes(4, 256, 7, (ctypes.c_float * 4)(-1.5, float("inf"), 0.45, 1.5), 16, 16, 16, 16),
           nl.nl_codes(4, 256, 7, lev, 16, 16, None, None),
           nl.nl_codes(4, 256, 0, lev, 16, 16, 16, 16),
           nl.nl_codes(4, 256, 7, lev, 18, 16, 16, 16)]
    for c in bad:
        assert L.nested_encode(16, 16, None, ctypes.byref(c), None, 0, None) == nl.NL_EINVAL
        assert L.nested_encode_quantize(16, ctypes.byref(c), None) == nl.NL_EINVAL
    assert L.nested_encode_quantize(16, ctypes.byref(bad[1]), None) == nl.NL_EINVAL
    assert b"ascending" in L.nested_linear_last_error()
    good = nl.nl_codes(4, 256, 7, lev, 16, 16, 16, 16)
    # two-sided without a workspace; misaligned w; NULL inputs
    assert L.nested_encode(16, 16, 16, ctypes.byref(good), None, 0, None) == nl.NL_EINVAL
    assert L.nested_encode(20, 16, None, ctypes.byref(good), None, 0, None) == nl.NL_EINVAL
    assert L.nested_encode(None, 16, None, ctypes.byref(good), None, 0, None) == nl.NL_EINVAL
    # overlapping rotate / normalise buffers
    assert L.nested_encode_rotate(4, 256, 4096, 16, None, 4096 + 256, None) == nl.NL_EINVAL
    assert L.nested_encode_normalize(4, 256, 4096, 4096 + 256, None) == nl.NL_EINVAL
    # level fit: n, iters, workspace
    assert L.nested_encode_fit_workspace_bytes(0, ctypes.byref(sz)) == nl.NL_EINVAL
    assert L.nested_encode_fit_workspace_bytes(1000, ctypes.byref(sz)) == nl.NL_OK and sz.value > 0
    out = (ctypes.c_double * 4)()
    assert L.nested_encode_fit_levels(16, 0, 60, out, 256, sz.value, None) == nl.NL_EINVAL
    assert L.nested_encode_fit_levels(16, 100, -1, out, 256, sz.value, None) == nl.NL_EINVAL
    assert L.nested_encode_fit_levels(16, 100, 60, out, 256, sz.value - 8, None) == nl.NL_EINVAL
    assert L.nested_encode_fit_levels(16, 100, 60, out, 300, sz.value, None) == nl.NL_EINVAL


def test_tree_calls_reject_bad_arguments():
    L = nl.lib()
    for D, R, N in [(0, 4, 8), (3, 0, 8), (3, 17, 8), (3, 4, 0), (3, 4, 65)]:
        assert L.nested_tree_build(16, D, R, N, 16, 16, 16, 16, 16, 16, None) == nl.NL_EINVAL
    assert L.nested_tree_build(None, 3, 4, 8, 16, 16, 16, 16, 16, 16, None) == nl.NL_EINVAL
    for N, B in [(0, 4), (65, 4), (8, 0)]:
        assert L.nested_tree_accept(16, N, B, 16, 16, 16, 16, 16, None) == nl.NL_EINVAL
    assert L.nested_tree_accept(16, 8, 4, None, 16, 16, 16, 16, None) == nl.NL_EINVAL
    assert b"N must be" in L.nested_linear_last_error() or L.nested_linear_last_error()


def test_kv_calls_reject_bad_arguments():
    L = nl.lib()
    sz = ctypes.c_size_t()
    for T, H_q, H_kv, Lc in [(0, 8, 2, 10), (65, 8, 2, 10), (4, 6, 4, 10), (4, 8, 0, 10), (64, 32, 4, 10), (4, 8, 2, -1)]:
        assert L.nested_kv_attention_workspace_bytes(T, H_q, H_kv, Lc, ctypes.byref(sz)) == nl.NL_EINVAL
    assert L.nested_kv_attention_workspace_bytes(16, 32, 8, 4096, ctypes.byref(sz)) == nl.NL_OK and sz.value > 0
    assert L.nested_kv_write(16, 0, 16, 16, 16, 16, None) == nl.NL_EINVAL
    assert L.nested_kv_write(None, 4, 16, 16, 16, 16, None) == nl.NL_EINVAL
    # verify without the refinement planes; small workspace
    assert L.nested_kv_attention(256, 4, 8, 2, 10, 256, None, 256, 256, None, 256, 256, 1, 256, 256, 1 << 20,
                                 None) == nl.NL_EINVAL
    assert L.nested_kv_attention(256, 4, 8, 2, 10, 256, 256, 256, 256, 256, 256, 256, 1, 256, 256, 16,
                                 None) == nl.NL_EINVAL
