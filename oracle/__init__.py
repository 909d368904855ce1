"""fp64 CPU oracle of the bit-nested quantized linear (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product package never does.
The arithmetic lives in ``nl_oracle.c`` (plain C, fp64, OpenMP over rows),
which shares no code with the HIP library.  ``build()`` compiles it with gcc.

Every function below states the passage of the source pages it follows; the
pins that tie it to the pages rather than to itself are in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nl_oracle.c")
_LIB = os.path.join(_HERE, "libnl_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libnl_oracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.nlo_block_size.argtypes = [i]
        L.nlo_block_size.restype = i
        L.nlo_fwht.argtypes = [P, i]
        L.nlo_fwht_b.argtypes = [P, i, i]
        L.nlo_half_to_double.argtypes = [ctypes.c_uint16]
        L.nlo_half_to_double.restype = ctypes.c_double
        L.nlo_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.nlo_bf16_to_double.restype = ctypes.c_double
        L.nlo_base_code.argtypes = [P, i, i, i]
        L.nlo_base_code.restype = i
        L.nlo_resid_code.argtypes = [P, i, i, i, i]
        L.nlo_resid_code.restype = i
        L.nlo_dequant_row.argtypes = [i, i, i, P, P, P, P, P, i, P]
        L.nlo_rotate_input.argtypes = [i, P, P, i, P]
        L.nlo_forward_rows.argtypes = [i, i, i, i, P, P, P, P, P, P, P, P, i, i, i, P]
        L.nlo_forward_rows.restype = i
        L.nlo_decode.argtypes = [i, i, P, P, i, i, P, P]
        L.nlo_num_threads.argtypes = []
        L.nlo_num_threads.restype = i
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def block_size(n: int) -> int:
    """POC section 1 block-size rule."""
    return lib().nlo_block_size(int(n))


def fwht(v: np.ndarray, b: int | None = None) -> np.ndarray:
    """Block-diagonal normalised Sylvester-Hadamard transform along the last
    axis (POC section 1).  Returns a new fp64 array."""
    a = np.array(v, dtype=np.float64, order="C", copy=True)
    n = a.shape[-1]
    flat = a.reshape(-1, n)
    assert flat.flags["C_CONTIGUOUS"] and np.shares_memory(flat, a)
    for row in flat:
        if b is None:
            lib().nlo_fwht(_p(row), n)
        else:
            lib().nlo_fwht_b(_p(row), n, int(b))
    return flat.reshape(a.shape)


def num_threads() -> int:
    """OpenMP threads the oracle's row loops use."""
    return lib().nlo_num_threads()


def half_to_double(h: int) -> float:
    return lib().nlo_half_to_double(int(h))


def bf16_to_double(b: int) -> float:
    return lib().nlo_bf16_to_double(int(b))


def decode(lin: dict, row0: int = 0, nrows: int | None = None):
    """Decode base indices (0..3) and residual integers of rows
    [row0, row0 + nrows) from the canonical planes (POC sections 2-3)."""
    d_in = lin["d_in"]
    nrows = lin["d_out"] - row0 if nrows is None else nrows
    bi = np.zeros((nrows, d_in), np.uint8)
    rq = np.zeros((nrows, d_in), np.int8) if lin["bits"] else None
    bc = _c(lin["base_codes"], np.uint8)
    rc = _c(lin["resid_codes"], np.uint8)
    lib().nlo_decode(d_in, lin["bits"], _p(bc), _p(rc), row0, nrows, _p(bi), _p(rq))
    return bi, rq


def dequant_row(lin: dict, r: int, verify: bool) -> np.ndarray:
    """Row r of the rotated-basis weights W~ in fp64 (POC sections 2-3)."""
    w = np.zeros(lin["d_in"], np.float64)
    lib().nlo_dequant_row(lin["d_in"], lin["bits"], int(verify),
                          _p(_c(lin["base_codes"], np.uint8)), _p(_c(lin["base_scales"], np.uint16)),
                          _p(_c(lin["resid_codes"], np.uint8)), _p(_c(lin["resid_scales"], np.uint16)),
                          _p(_c(lin["levels"], np.float32)), int(r), _p(w))
    return w


def rotate_input(lin: dict, x_bf16: np.ndarray) -> np.ndarray:
    """x' = H_i S_i x in fp64, [T][d_in] (POC sections 1 and 4)."""
    x = _c(x_bf16, np.uint16)
    T = x.shape[0]
    out = np.zeros((T, lin["d_in"]), np.float64)
    lib().nlo_rotate_input(lin["d_in"], _p(_c(lin["sign_in"], np.int8)), _p(x), T, _p(out))
    return out


def forward(lin: dict, x_bf16: np.ndarray, verify: bool, rows: tuple | None = None) -> np.ndarray:
    """The nested Linear's forward (POC section 4) in fp64: verify includes
    the residual, draft does not; y = S_o H_o (W~ H_i S_i x) when the linear
    has sign_out, else the rotated-basis y~ = W~ H_i S_i x.  ``rows`` =
    (row0, row1) restricts the output to those rows (whole output blocks when
    sign_out is set).  Returns fp64 [T][row1 - row0]."""
    x = _c(x_bf16, np.uint16)
    T = x.shape[0]
    r0, r1 = (0, lin["d_out"]) if rows is None else rows
    y = np.zeros((T, r1 - r0), np.float64)
    if verify and not lin["bits"]:
        raise ValueError("verify needs a residual")
    rc = lib().nlo_forward_rows(
        lin["d_out"], lin["d_in"], lin["bits"], int(verify),
        _p(_c(lin["base_codes"], np.uint8)), _p(_c(lin["base_scales"], np.uint16)),
        _p(_c(lin["resid_codes"], np.uint8)), _p(_c(lin["resid_scales"], np.uint16)),
        _p(_c(lin["levels"], np.float32)), _p(_c(lin["sign_in"], np.int8)),
        _p(_c(lin["sign_out"], np.int8)), _p(x), T, r0, r1, _p(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def forward_grouped(experts: list, pair_token: np.ndarray, offsets: np.ndarray,
                    x_bf16: np.ndarray, verify: bool) -> np.ndarray:
    """Grouped (mixture-of-experts) forward: pair p, routed to expert e
    (offsets[e] <= p < offsets[e+1]), gets expert e's Linear applied to token
    pair_token[p].  This is the per-expert loop that a grouped GEMM replaces
    (DFlash write-up, "The verify's own cost").  Returns fp64 [P][d_out]."""
    P = len(pair_token)
    d_out = experts[0]["d_out"]
    y = np.zeros((P, d_out), np.float64)
    x = np.asarray(x_bf16, np.uint16)
    for e, lin in enumerate(experts):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = forward(lin, x[pair_token[a:b]], verify)
    return y
