"""Python binding of libnested_linear.so, the bit-nested quantized linear for
AMD MI355X (gfx950).

Argument marshalling only: every step of the draft/verify forward runs in the
library's HIP kernels.  The functions carry the C ABI's names
(include/nested_linear.h); tensors are torch device tensors, the stream is
the current torch stream unless given.  A failing call raises NLError with
the library's message.  The library is built in-tree by
``bit_nested_quantized_amd.build.build()``; importing this package never
falls back to anything else: if the library is missing, the first call
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnested_linear.so")

NL_OK, NL_EINVAL, NL_ENOMEM, NL_EHIP, NL_EUNSUPPORTED = 0, 1, 2, 3, 4
NL_MAX_T = 64

# Every symbol the C header declares (checked by the CPU tests).
EXPORTS = (
    "nested_linear_create", "nested_linear_destroy", "nested_linear_workspace_bytes",
    "nested_linear_verify", "nested_linear_draft", "nested_linear_prepare_input",
    "nested_linear_contract", "nested_linear_finish", "nested_linear_group_create",
    "nested_linear_group_destroy", "nested_linear_group_workspace_bytes",
    "nested_linear_verify_grouped", "nested_linear_draft_grouped", "nested_linear_decode",
    "nested_linear_info", "nested_linear_timing_begin", "nested_linear_timing_end",
    "nested_linear_last_error", "nested_linear_verify_multi", "nested_linear_draft_multi",
    "nested_linear_multi_workspace_bytes", "nested_linear_workspace_status", "nested_linear_set_tuning",
    "nested_linear_describe_call", "nested_linear_stream_read", "nested_linear_forward_static",
    "nested_encode_rotate", "nested_encode_quantize", "nested_encode_workspace_bytes", "nested_encode",
    "nested_encode_normalize", "nested_encode_fit_workspace_bytes", "nested_encode_fit_levels",
    "nested_w4w8_create", "nested_w4w8_destroy", "nested_w4w8_workspace_bytes", "nested_w4w8_verify",
    "nested_w4w8_draft", "nested_tree_build", "nested_tree_accept",
    "nested_kv_write", "nested_kv_attention_workspace_bytes", "nested_kv_attention",
)


class NLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class nl_desc(ctypes.Structure):
    _fields_ = [
        ("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32), ("residual_bits", ctypes.c_int32),
        ("base_codes", ctypes.c_void_p), ("base_scales", ctypes.c_void_p),
        ("resid_codes", ctypes.c_void_p), ("resid_scales", ctypes.c_void_p),
        ("sign_in", ctypes.c_void_p), ("sign_out", ctypes.c_void_p),
        ("levels", ctypes.c_float * 4),
    ]


class nl_codes(ctypes.Structure):
    _fields_ = [
        ("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32), ("residual_bits", ctypes.c_int32),
        ("levels", ctypes.c_float * 4),
        ("base_codes", ctypes.c_void_p), ("base_scales", ctypes.c_void_p),
        ("resid_codes", ctypes.c_void_p), ("resid_scales", ctypes.c_void_p),
    ]


class nl_w4w8_desc(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32), ("base_plane", ctypes.c_void_p),
                ("ref_plane", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run bit_nested_quantized_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "nested_linear_create": [ctypes.POINTER(nl_desc), ctypes.POINTER(P)],
            "nested_linear_destroy": [P],
            "nested_linear_workspace_bytes": [P, i32, ctypes.POINTER(sz)],
            "nested_linear_verify": [P, P, i32, P, P, sz, P],
            "nested_linear_draft": [P, P, i32, P, P, sz, P],
            "nested_linear_prepare_input": [P, P, i32, P, sz, P],
            "nested_linear_contract": [P, i32, i32, P, P, sz, P],
            "nested_linear_finish": [P, i32, P, P, sz, P],
            "nested_linear_group_create": [P, i32, ctypes.POINTER(P)],
            "nested_linear_group_destroy": [P],
            "nested_linear_group_workspace_bytes": [P, i32, ctypes.POINTER(sz)],
            "nested_linear_verify_grouped": [P, P, P, i32, P, i32, i32, P, P, sz, P],
            "nested_linear_draft_grouped": [P, P, P, i32, P, i32, i32, P, P, sz, P],
            "nested_linear_decode": [P, i32, i32, P, P, P],
            "nested_linear_info": [P] + [ctypes.POINTER(i32)] * 5 + [ctypes.POINTER(ctypes.c_float)],
            "nested_linear_timing_begin": [i32],
            "nested_linear_timing_end": [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)],
            "nested_linear_verify_multi": [P, i32, P, i32, P, P, sz, P],
            "nested_linear_draft_multi": [P, i32, P, i32, P, P, sz, P],
            "nested_linear_multi_workspace_bytes": [P, i32, i32, ctypes.POINTER(sz)],
            "nested_linear_workspace_status": [P, ctypes.POINTER(ctypes.c_uint32), i32, P],
            "nested_linear_set_tuning": [i32, ctypes.c_double],
            "nested_linear_describe_call": [P, i32, i32, i32, i32, i32, ctypes.POINTER(i32), i32],
            "nested_linear_stream_read": [P, sz, P, i32, P],
            "nested_linear_forward_static": [P, i32, P, i32, P, P],
            "nested_encode_rotate": [i32, i32, P, P, P, P, P],
            "nested_encode_quantize": [P, ctypes.POINTER(nl_codes), P],
            "nested_encode_workspace_bytes": [i32, i32, i32, ctypes.POINTER(sz)],
            "nested_encode": [P, P, P, ctypes.POINTER(nl_codes), P, sz, P],
            "nested_encode_normalize": [i32, i32, P, P, P],
            "nested_encode_fit_workspace_bytes": [ctypes.c_int64, ctypes.POINTER(sz)],
            "nested_encode_fit_levels": [P, ctypes.c_int64, i32, ctypes.POINTER(ctypes.c_double), P, sz, P],
            "nested_w4w8_create": [ctypes.POINTER(nl_w4w8_desc), ctypes.POINTER(P)],
            "nested_w4w8_destroy": [P],
            "nested_w4w8_workspace_bytes": [P, i32, ctypes.POINTER(sz)],
            "nested_w4w8_verify": [P, P, i32, P, P, sz, P],
            "nested_w4w8_draft": [P, P, i32, P, P, sz, P],
            "nested_tree_build": [P, i32, i32, i32, P, P, P, P, P, P, P],
            "nested_tree_accept": [P, i32, i32, P, P, P, P, P, P],
            "nested_kv_write": [P, i32, P, P, P, P, P],
            "nested_kv_attention_workspace_bytes": [i32, i32, i32, i32, ctypes.POINTER(sz)],
            "nested_kv_attention": [P, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P, P, sz, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.nested_linear_last_error.argtypes = []
        L.nested_linear_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st: int):
    if st != NL_OK:
        raise NLError(st, lib().nested_linear_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def nested_linear_create(d_out: int, d_in: int, residual_bits: int, base_codes, base_scales,
                         resid_codes, resid_scales, sign_in, sign_out, levels) -> ctypes.c_void_p:
    """Device tensors of the canonical format (uint8 codes, fp16-bit scales as
    int16/uint16, int8 signs); levels is a host sequence of 4 floats."""
    d = nl_desc(int(d_out), int(d_in), int(residual_bits), _ptr(base_codes), _ptr(base_scales),
                _ptr(resid_codes), _ptr(resid_scales), _ptr(sign_in), _ptr(sign_out),
                (ctypes.c_float * 4)(*[float(v) for v in levels]))
    h = ctypes.c_void_p()
    _check(lib().nested_linear_create(ctypes.byref(d), ctypes.byref(h)))
    return h


def nested_linear_destroy(h):
    _check(lib().nested_linear_destroy(h))


def nested_linear_workspace_bytes(h, T_max: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_linear_workspace_bytes(h, int(T_max), ctypes.byref(n)))
    return n.value


def nested_linear_verify(h, x, T: int, y, ws, stream=None):
    _check(lib().nested_linear_verify(h, _ptr(x), int(T), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)))


def nested_linear_draft(h, x, T: int, y, ws, stream=None):
    _check(lib().nested_linear_draft(h, _ptr(x), int(T), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def _handles(hs):
    return (ctypes.c_void_p * len(hs))(*[h.value for h in hs])


def nested_linear_verify_multi(hs, x, T: int, ys, ws, stream=None):
    yp = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    _check(lib().nested_linear_verify_multi(_handles(hs), len(hs), _ptr(x), int(T), yp, _ptr(ws), _nbytes(ws),
                                            _stream(stream)))


def nested_linear_draft_multi(hs, x, T: int, ys, ws, stream=None):
    yp = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    _check(lib().nested_linear_draft_multi(_handles(hs), len(hs), _ptr(x), int(T), yp, _ptr(ws), _nbytes(ws),
                                           _stream(stream)))


def nested_linear_multi_workspace_bytes(hs, T_max: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_linear_multi_workspace_bytes(_handles(hs), len(hs), int(T_max), ctypes.byref(n)))
    return n.value


def nested_linear_workspace_status(ws, clear: bool = False, stream=None) -> int:
    """Error word of a workspace (waits that gave up); synchronises."""
    e = ctypes.c_uint32(0)
    _check(lib().nested_linear_workspace_status(_ptr(ws), ctypes.byref(e), int(bool(clear)), _stream(stream)))
    return int(e.value)


def nested_linear_forward_static(h, verify: bool, x, T: int, y, stream=None):
    """Verify or draft forward on the library's static scratch (no allocation)."""
    _check(lib().nested_linear_forward_static(h, int(bool(verify)), _ptr(x), int(T), _ptr(y), _stream(stream)))


def nested_linear_stream_read(src, sink, grid: int = 0, stream=None):
    """Streaming-read reference: one launch reading all of ``src`` once."""
    _check(lib().nested_linear_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), int(grid),
                                           _stream(stream)))


def nested_linear_describe_call(d_outs, d_in: int, bits: int, two_sided: bool, T: int) -> dict:
    """The launch plan of a call (host query; bits = 0 for the draft)."""
    n = len(d_outs)
    arr = (ctypes.c_int32 * n)(*[int(d) for d in d_outs])
    buf = (ctypes.c_int32 * (8 + 6 * n))()
    _check(lib().nested_linear_describe_call(arr, n, int(d_in), int(bits), int(bool(two_sided)), int(T), buf,
                                             8 + 6 * n))
    v = list(buf)
    keys = ("local", "mt", "waves", "n_rot", "n_con", "n_fin", "lds", "blob")
    d = dict(zip(keys, v[:8]))
    d["jobs"] = [dict(zip(("S", "cps", "rt", "kw", "n_rb", "n_sb"), v[8 + 6 * i: 14 + 6 * i])) for i in range(n)]
    return d


NL_TUNE = {"splits": 1, "row_tiles": 2, "waves_per_tile": 3, "local_t": 4, "cus": 5, "lat_us": 6, "hbm_gbs": 7,
           "split_us": 8, "xdma_gbs": 9, "spin_limit": 10, "wait_extra": 11, "waves": 12,
           "staged_t_verify": 13, "staged_t_draft": 14, "staged_waves": 15,
           "multi_staged_t_verify": 16, "multi_staged_t_draft": 17}


def nested_linear_set_tuning(knob: str, value: float):
    _check(lib().nested_linear_set_tuning(NL_TUNE[knob], float(value)))


def nested_linear_prepare_input(h, x, T: int, ws, stream=None):
    _check(lib().nested_linear_prepare_input(h, _ptr(x), int(T), _ptr(ws), ws.numel() * ws.element_size(),
                                             _stream(stream)))


def nested_linear_contract(h, verify: bool, T: int, y, ws, stream=None):
    _check(lib().nested_linear_contract(h, int(bool(verify)), int(T), _ptr(y), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def nested_linear_finish(h, T: int, y, ws, stream=None):
    _check(lib().nested_linear_finish(h, int(T), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)))


def nested_linear_group_create(handles) -> ctypes.c_void_p:
    arr = (ctypes.c_void_p * len(handles))(*[h.value for h in handles])
    g = ctypes.c_void_p()
    _check(lib().nested_linear_group_create(arr, len(handles), ctypes.byref(g)))
    return g


def nested_linear_group_destroy(g):
    _check(lib().nested_linear_group_destroy(g))


def nested_linear_group_workspace_bytes(g, P_max: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_linear_group_workspace_bytes(g, int(P_max), ctypes.byref(n)))
    return n.value


def nested_linear_verify_grouped(g, pair_token, offsets, P: int, x, x_rows: int, T: int, y, ws, stream=None):
    _check(lib().nested_linear_verify_grouped(g, _ptr(pair_token), _ptr(offsets), int(P), _ptr(x), int(x_rows), int(T),
                                              _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                              _stream(stream)))


def nested_linear_draft_grouped(g, pair_token, offsets, P: int, x, x_rows: int, T: int, y, ws, stream=None):
    _check(lib().nested_linear_draft_grouped(g, _ptr(pair_token), _ptr(offsets), int(P), _ptr(x), int(x_rows), int(T),
                                             _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                             _stream(stream)))


def nested_linear_decode(h, row0: int, nrows: int, base_idx, resid, stream=None):
    _check(lib().nested_linear_decode(h, int(row0), int(nrows), _ptr(base_idx), _ptr(resid), _stream(stream)))


def nested_linear_timing_begin(capacity: int):
    _check(lib().nested_linear_timing_begin(capacity))


def nested_linear_timing_end(capacity: int) -> list:
    """Kernel durations (microseconds) of the launches recorded since begin."""
    buf = (ctypes.c_float * max(capacity, 1))()
    n = ctypes.c_int32(0)
    _check(lib().nested_linear_timing_end(buf, capacity, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


def nested_linear_info(h) -> dict:
    v = [ctypes.c_int32() for _ in range(5)]
    e = ctypes.c_float()
    _check(lib().nested_linear_info(h, *[ctypes.byref(x) for x in v], ctypes.byref(e)))
    return {"d_out": v[0].value, "d_in": v[1].value, "bits": v[2].value, "block_in": v[3].value,
            "block_out": v[4].value, "level_rel_err": e.value}


# --- encoder (include/nested_encode.h) ----------------------------------------

def nested_encode_rotate(d_out: int, d_in: int, w, sign_in, sign_out, wt, stream=None):
    _check(lib().nested_encode_rotate(int(d_out), int(d_in), _ptr(w), _ptr(sign_in), _ptr(sign_out),
                                      _ptr(wt), _stream(stream)))


def nested_encode_quantize(wt, codes: nl_codes, stream=None):
    _check(lib().nested_encode_quantize(_ptr(wt), ctypes.byref(codes), _stream(stream)))


def nested_encode_workspace_bytes(d_out: int, d_in: int, two_sided: bool) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_encode_workspace_bytes(int(d_out), int(d_in), int(bool(two_sided)), ctypes.byref(n)))
    return n.value


def nested_encode(w, sign_in, sign_out, codes: nl_codes, ws=None, stream=None):
    _check(lib().nested_encode(_ptr(w), _ptr(sign_in), _ptr(sign_out), ctypes.byref(codes), _ptr(ws),
                               _nbytes(ws), _stream(stream)))


def nested_encode_normalize(d_out: int, d_in: int, wt, v, stream=None):
    _check(lib().nested_encode_normalize(int(d_out), int(d_in), _ptr(wt), _ptr(v), _stream(stream)))


def nested_encode_fit_workspace_bytes(n: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().nested_encode_fit_workspace_bytes(int(n), ctypes.byref(b)))
    return b.value


def nested_encode_fit_levels(v, n: int, iters: int, ws, stream=None) -> list:
    """Returns the four fitted levels (host floats, fp64); synchronises."""
    out = (ctypes.c_double * 4)()
    _check(lib().nested_encode_fit_levels(_ptr(v), int(n), int(iters), out, _ptr(ws), _nbytes(ws),
                                          _stream(stream)))
    return [float(x) for x in out]


class Codes:
    """Device arrays of one linear's canonical planes, written by the encoder
    (torch uint8 / int16 tensors), and the nl_codes descriptor that points at
    them."""

    def __init__(self, d_out: int, d_in: int, bits: int, levels, device="cuda"):
        import torch
        G = d_in // 128
        self.d_out, self.d_in, self.bits = d_out, d_in, bits
        self.levels = [float(x) for x in levels]
        self.base_codes = torch.empty((d_out, G, 32), dtype=torch.uint8, device=device)
        self.base_scales = torch.empty((d_out, G), dtype=torch.int16, device=device)
        self.resid_codes = torch.empty((d_out, G, 16 * bits), dtype=torch.uint8, device=device) if bits else None
        self.resid_scales = torch.empty((d_out, G), dtype=torch.int16, device=device) if bits else None
        self.desc = nl_codes(int(d_out), int(d_in), int(bits), (ctypes.c_float * 4)(*self.levels),
                             _ptr(self.base_codes), _ptr(self.base_scales), _ptr(self.resid_codes),
                             _ptr(self.resid_scales))

    def host(self) -> dict:
        """The canonical dict (numpy) that synth.make_linear produces."""
        import numpy as np

        def h(t, dt):
            return None if t is None else t.cpu().numpy().view(dt)

        return {"d_out": self.d_out, "d_in": self.d_in, "bits": self.bits,
                "levels": np.array(self.levels, np.float32),
                "base_codes": h(self.base_codes, np.uint8), "base_scales": h(self.base_scales, np.uint16),
                "resid_codes": h(self.resid_codes, np.uint8), "resid_scales": h(self.resid_scales, np.uint16)}


def encode(w, sign_in, sign_out, bits: int, levels, stream=None) -> Codes:
    """Encode a dense fp32 device matrix w [d_out][d_in] (nested_encode);
    the two-sided form gets its workspace from torch."""
    import torch
    d_out, d_in = w.shape
    c = Codes(d_out, d_in, bits, levels, device=w.device)
    nws = nested_encode_workspace_bytes(d_out, d_in, sign_out is not None)
    ws = torch.empty(nws, dtype=torch.uint8, device=w.device) if nws else None
    nested_encode(w, sign_in, sign_out, c.desc, ws, stream)
    return c


# --- W4/W8 dual-plane linear (include/nested_w4w8.h) -------------------------

def nested_w4w8_create(d_out: int, d_in: int, base_plane, ref_plane, scales) -> ctypes.c_void_p:
    d = nl_w4w8_desc(int(d_out), int(d_in), _ptr(base_plane), _ptr(ref_plane), _ptr(scales))
    h = ctypes.c_void_p()
    _check(lib().nested_w4w8_create(ctypes.byref(d), ctypes.byref(h)))
    return h


def nested_w4w8_destroy(h):
    _check(lib().nested_w4w8_destroy(h))


def nested_w4w8_workspace_bytes(h, T_max: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_w4w8_workspace_bytes(h, int(T_max), ctypes.byref(n)))
    return n.value


def nested_w4w8_verify(h, x, T: int, y, ws, stream=None):
    _check(lib().nested_w4w8_verify(h, _ptr(x), int(T), _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)))


def nested_w4w8_draft(h, x, T: int, y, ws, stream=None):
    _check(lib().nested_w4w8_draft(h, _ptr(x), int(T), _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)))


class W4W8Linear:
    """Owns one W4/W8 dual-plane linear built from a canonical dict (numpy
    arrays as produced by ``synth.make_w4w8_linear``)."""

    def __init__(self, lin: dict, device="cuda"):
        import numpy as np
        import torch

        def dev(a, dt):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        self.d_out, self.d_in = lin["d_out"], lin["d_in"]
        self.h = nested_w4w8_create(self.d_out, self.d_in, dev(lin["base_plane"], np.uint8),
                                    dev(lin.get("ref_plane"), np.uint8), dev(lin["scales"], np.int16))

    def close(self):
        if self.h is not None:
            nested_w4w8_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, T_max: int, device="cuda"):
        import torch
        n = nested_w4w8_workspace_bytes(self.h, T_max)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)

    def forward(self, x, verify: bool, ws=None, y=None, stream=None):
        import torch
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        y = torch.empty((T, self.d_out), dtype=torch.float32, device=x.device) if y is None else y
        (nested_w4w8_verify if verify else nested_w4w8_draft)(self.h, x, T, y, ws, stream)
        return y


# --- draft tree (include/nested_tree.h) ----------------------------------------

def nested_tree_build(p, D: int, R: int, N: int, parent, depth, rank, prio, anc, count, stream=None):
    _check(lib().nested_tree_build(_ptr(p), int(D), int(R), int(N), _ptr(parent), _ptr(depth), _ptr(rank),
                                   _ptr(prio), _ptr(anc), _ptr(count), _stream(stream)))


def nested_tree_accept(parent, N: int, B: int, draft_token, argmax, n_accepted, path, bonus, stream=None):
    _check(lib().nested_tree_accept(_ptr(parent), int(N), int(B), _ptr(draft_token), _ptr(argmax),
                                    _ptr(n_accepted), _ptr(path), _ptr(bonus), _stream(stream)))


def tree_build(p, N: int, stream=None) -> dict:
    """Best-first tree from a device fp64 tensor p [D][R]; device outputs."""
    import torch
    D, R = p.shape
    dev = p.device
    out = {"parent": torch.empty(N, dtype=torch.int32, device=dev), "depth": torch.empty(N, dtype=torch.int32, device=dev),
           "rank": torch.empty(N, dtype=torch.int32, device=dev), "prio": torch.empty(N, dtype=torch.float64, device=dev),
           "anc": torch.empty(N, dtype=torch.int64, device=dev), "count": torch.empty(1, dtype=torch.int32, device=dev)}
    nested_tree_build(p, D, R, N, out["parent"], out["depth"], out["rank"], out["prio"], out["anc"], out["count"],
                      stream)
    return out


def tree_accept(parent, draft_token, argmax, stream=None):
    """Greedy acceptance for B sequences (device int32 tensors)."""
    import torch
    B, N = draft_token.shape
    dev = draft_token.device
    n = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.full((B, N), -1, dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    nested_tree_accept(parent, N, B, draft_token, argmax, n, path, bonus, stream)
    return n, path, bonus


# --- nested KV cache (include/nested_kv.h) -------------------------------------

def nested_kv_write(x, n: int, row, base, ref, scale, stream=None):
    _check(lib().nested_kv_write(_ptr(x), int(n), _ptr(row), _ptr(base), _ptr(ref), _ptr(scale), _stream(stream)))


def nested_kv_attention_workspace_bytes(T: int, H_q: int, H_kv: int, L: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().nested_kv_attention_workspace_bytes(int(T), int(H_q), int(H_kv), int(L), ctypes.byref(n)))
    return n.value


def nested_kv_attention(q, T: int, H_q: int, H_kv: int, L: int, k_base, k_ref, k_scale, v_base, v_ref, v_scale, anc,
                        verify: bool, out, ws, stream=None):
    _check(lib().nested_kv_attention(_ptr(q), int(T), int(H_q), int(H_kv), int(L), _ptr(k_base), _ptr(k_ref),
                                     _ptr(k_scale), _ptr(v_base), _ptr(v_ref), _ptr(v_scale), _ptr(anc),
                                     int(bool(verify)), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


class Linear:
    """Owns one nested linear built from a canonical dict (numpy arrays as
    produced by ``synth.make_linear``), copied to ``device`` first."""

    def __init__(self, lin: dict, device="cuda"):
        import numpy as np
        import torch

        def dev(a, dt):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        bufs = dict(
            base_codes=dev(lin["base_codes"], np.uint8), base_scales=dev(lin["base_scales"], np.int16),
            resid_codes=dev(lin["resid_codes"], np.uint8), resid_scales=dev(lin["resid_scales"], np.int16),
            sign_in=dev(lin["sign_in"], np.int8), sign_out=dev(lin["sign_out"], np.int8))
        self.d_out, self.d_in, self.bits = lin["d_out"], lin["d_in"], lin["bits"]
        self.h = nested_linear_create(self.d_out, self.d_in, self.bits, levels=lin["levels"], **bufs)

    def close(self):
        if self.h is not None:
            nested_linear_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, T_max: int, device="cuda"):
        import torch
        n = nested_linear_workspace_bytes(self.h, T_max)
        # zero-filled once: the calls hand work over through counters at its
        # start and leave them at zero
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)

    def forward(self, x, verify: bool, ws=None, y=None, stream=None):
        """x: int16/uint16 bf16-bit tensor [T][d_in] (or torch.bfloat16)."""
        import torch
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        y = torch.empty((T, self.d_out), dtype=torch.float32, device=x.device) if y is None else y
        (nested_linear_verify if verify else nested_linear_draft)(self.h, x, T, y, ws, stream)
        return y
