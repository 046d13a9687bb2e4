"""ctypes binding of libbconv.so.

Functions carry the names of the C ABI in ``include/bconv.h`` and only
marshal arguments: device pointers are plain integers (or torch tensors, whose
``data_ptr()`` is taken), host arrays are numpy arrays.  Nothing here
computes any step of the forward pass; if the shared library is missing every
entry point raises ``BconvLibraryMissing``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbconv.so")

# bconv_status_t
BCONV_OK = 0
BCONV_ERR_INVALID_ARGUMENT = 1
BCONV_ERR_UNSUPPORTED = 2
BCONV_ERR_WORKSPACE = 3
BCONV_ERR_ALLOC = 4
BCONV_ERR_HIP = 5
# bconv_type_t
BCONV_BINARY_WEIGHTS = 0
BCONV_XNOR = 1
BCONV_AND = 2
# flags
BCONV_FLAG_NONE = 0
BCONV_FLAG_USE_BETA_SCALING = 1
BCONV_FLAG_INT8_MFMA = 2
BCONV_FLAG_BETA_VALID_TAPS = 4
BCONV_FLAG_FP4_MFMA = 8
# bconv_neuron_t
BCONV_NEURON_NONE = 0
BCONV_NEURON_RELU = 1
NEURON_NAMES = ("none", "relu", "leaky_relu", "linear", "sigmoid", "hard_sigmoid", "tanh", "absolute", "softplus",
                "softsign", "elu", "clamp")

TYPE_CODES = {"binary_weights": BCONV_BINARY_WEIGHTS, "xnor": BCONV_XNOR, "and": BCONV_AND}
NEURON_CODES = {name: code for code, name in enumerate(NEURON_NAMES)}
SIZE_MAX = ctypes.c_size_t(-1).value
BCONV_SCRATCH_MAX_BYTES = 16 << 20


class BconvLibraryMissing(RuntimeError):
    pass


class BconvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


class bconv_desc_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "in_h", "in_w", "in_c", "out_c", "kernel_h", "kernel_w", "stride_h", "stride_w",
        "pad_h", "pad_w", "groups", "neuron")] + [("scale_value", ctypes.c_float)] + \
        [("pad_h_end", ctypes.c_int32), ("pad_w_end", ctypes.c_int32),
         ("neuron_a", ctypes.c_float), ("neuron_b", ctypes.c_float)]


class bconv_workspace_layout_t(ctypes.Structure):
    _fields_ = [("bits_offset", ctypes.c_size_t), ("bits_rows", ctypes.c_int32),
                ("bits_cols", ctypes.c_int32), ("bits_words", ctypes.c_int32),
                ("bits_pad_h", ctypes.c_int32), ("bits_pad_w", ctypes.c_int32),
                ("a_map_offset", ctypes.c_size_t), ("beta_offset", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t)]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libbconv.so and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise BconvLibraryMissing(
            f"{p} is not built: run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(p)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    st = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    up = ctypes.POINTER(ctypes.c_uint32)
    sigs = {
        "bconv_validate_desc": (st, [ctypes.POINTER(bconv_desc_t), i32, u32]),
        "bconv_create": (st, [ctypes.POINTER(bconv_desc_t), up, fp, fp, fp, fp, i32, u32,
                              ctypes.POINTER(vp)]),
        "bconv_create_fc": (st, [i32, i32, i32, i32, i32, ctypes.c_float, up, fp, fp, fp, fp,
                                 i32, u32, ctypes.POINTER(vp)]),
        "bconv_get_info": (st, [vp] + [ctypes.POINTER(i32)] * 4),
        "bconv_workspace_size": (st, [vp, i32, ctypes.POINTER(sz)]),
        "bconv_workspace_layout": (st, [vp, i32, ctypes.POINTER(bconv_workspace_layout_t)]),
        "bconv_forward": (st, [vp, vp, i32, vp, vp, vp, sz]),
        "bconv_forward_noalloc": (st, [vp, vp, i32, vp, vp]),
        "bconv_forward_accum": (st, [vp, vp, i32, vp, vp, vp, sz]),
        "bconv_forward_profiled": (st, [vp, vp, i32, vp, vp, vp, sz, vp, vp, vp, vp]),
        "bconv_forward_bits": (st, [vp, vp, i32, vp, vp, vp, sz]),
        "bconv_forward_bits_profiled": (st, [vp, vp, i32, vp, vp, vp, sz, vp, vp, vp, vp]),
        "bconv_main_kernel": (ctypes.c_char_p, [vp, i32]),
        "bconv_forward_packed": (st, [vp, vp, i32, vp, vp, vp, sz]),
        "bconv_forward_packed_bits": (st, [vp, vp, i32, vp, vp, vp, sz]),
        "bconv_calibrate_popcount": (st, [vp, i32, i32, u32, vp]),
        "bconv_destroy": (st, [vp]),
        "bconv_status_string": (ctypes.c_char_p, [st]),
        "bconv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_name(s: int) -> str:
    try:
        return load_library().bconv_status_string(s).decode()
    except BconvLibraryMissing:
        return f"status {s}"


def _check(status: int) -> None:
    if status != BCONV_OK:
        raise BconvError(status, bconv_last_error())


def _host_f32(a) -> Optional[ctypes.POINTER(ctypes.c_float)]:
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.float32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor or a plain integer address."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def make_desc(in_h, in_w, in_c, out_c, kernel_h, kernel_w, stride_h=1, stride_w=1, pad_h=0,
              pad_w=0, groups=1, neuron=BCONV_NEURON_NONE, scale_value=1.0, pad_h_end=None,
              pad_w_end=None, neuron_a=0.0, neuron_b=0.0) -> bconv_desc_t:
    """Trailing padding defaults to the leading one (symmetric padding)."""
    return bconv_desc_t(in_h, in_w, in_c, out_c, kernel_h, kernel_w, stride_h, stride_w, pad_h,
                        pad_w, groups, neuron, scale_value, pad_h if pad_h_end is None else pad_h_end,
                        pad_w if pad_w_end is None else pad_w_end, neuron_a, neuron_b)


def bconv_validate_desc(desc: bconv_desc_t, type: int, flags: int) -> int:
    return load_library().bconv_validate_desc(ctypes.byref(desc), type, flags)


def bconv_create(desc: bconv_desc_t, weight_bits: np.ndarray, output_scale=None, output_bias=None,
                 input_scale=None, input_bias=None, type: int = BCONV_XNOR,
                 flags: int = BCONV_FLAG_NONE) -> int:
    lib = load_library()
    wb = np.ascontiguousarray(weight_bits, dtype=np.uint32)
    keep = [_host_f32(a) for a in (output_scale, output_bias, input_scale, input_bias)]
    ptrs = [k[1] if k else None for k in keep]
    h = ctypes.c_void_p()
    _check(lib.bconv_create(ctypes.byref(desc), wb.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                            *ptrs, type, flags, ctypes.byref(h)))
    return h.value


def bconv_create_fc(in_h, in_w, in_c, out_c, neuron, scale_value, weight_bits, output_scale=None,
                    output_bias=None, input_scale=None, input_bias=None, type=BCONV_XNOR,
                    flags=BCONV_FLAG_NONE) -> int:
    lib = load_library()
    wb = np.ascontiguousarray(weight_bits, dtype=np.uint32)
    keep = [_host_f32(a) for a in (output_scale, output_bias, input_scale, input_bias)]
    ptrs = [k[1] if k else None for k in keep]
    h = ctypes.c_void_p()
    _check(lib.bconv_create_fc(in_h, in_w, in_c, out_c, neuron, scale_value,
                               wb.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), *ptrs, type,
                               flags, ctypes.byref(h)))
    return h.value


def bconv_get_info(h: int):
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(load_library().bconv_get_info(h, *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)


def bconv_workspace_size(h: int, n: int) -> int:
    b = ctypes.c_size_t()
    _check(load_library().bconv_workspace_size(h, n, ctypes.byref(b)))
    return b.value


def bconv_workspace_layout(h: int, n: int) -> dict:
    L = bconv_workspace_layout_t()
    _check(load_library().bconv_workspace_layout(h, n, ctypes.byref(L)))
    d = {name: getattr(L, name) for name, _ in L._fields_}
    for k in ("bits_offset", "a_map_offset", "beta_offset"):
        if d[k] == SIZE_MAX:
            d[k] = None
    return d


def bconv_forward(h: int, stream, n: int, inp, out, workspace, workspace_bytes: int) -> None:
    _check(load_library().bconv_forward(h, _ptr(stream), n, _ptr(inp), _ptr(out), _ptr(workspace),
                                        workspace_bytes))


def bconv_forward_noalloc(h: int, stream, n: int, inp, out) -> None:
    _check(load_library().bconv_forward_noalloc(h, _ptr(stream), n, _ptr(inp), _ptr(out)))


def bconv_forward_accum(h: int, stream, n: int, inp, acc, workspace, workspace_bytes: int) -> None:
    _check(load_library().bconv_forward_accum(h, _ptr(stream), n, _ptr(inp), _ptr(acc),
                                              _ptr(workspace), workspace_bytes))


def bconv_forward_profiled(h: int, stream, n: int, inp, out, workspace, workspace_bytes: int,
                           main_begin=None, main_end=None, input_begin=None, input_end=None) -> None:
    _check(load_library().bconv_forward_profiled(h, _ptr(stream), n, _ptr(inp), _ptr(out),
                                                 _ptr(workspace), workspace_bytes,
                                                 _ptr(main_begin), _ptr(main_end),
                                                 _ptr(input_begin), _ptr(input_end)))


def bconv_forward_bits(h: int, stream, n: int, inp, out_bits, workspace, workspace_bytes: int) -> None:
    _check(load_library().bconv_forward_bits(h, _ptr(stream), n, _ptr(inp), _ptr(out_bits), _ptr(workspace),
                                             workspace_bytes))


def bconv_forward_bits_profiled(h: int, stream, n: int, inp, out_bits, workspace, workspace_bytes: int,
                                main_begin=None, main_end=None, input_begin=None, input_end=None) -> None:
    _check(load_library().bconv_forward_bits_profiled(h, _ptr(stream), n, _ptr(inp), _ptr(out_bits),
                                                      _ptr(workspace), workspace_bytes,
                                                      _ptr(main_begin), _ptr(main_end),
                                                      _ptr(input_begin), _ptr(input_end)))


def bconv_forward_packed(h: int, stream, n: int, in_bits, out, workspace, workspace_bytes: int) -> None:
    _check(load_library().bconv_forward_packed(h, _ptr(stream), n, _ptr(in_bits), _ptr(out), _ptr(workspace),
                                               workspace_bytes))


def bconv_forward_packed_bits(h: int, stream, n: int, in_bits, out_bits, workspace, workspace_bytes: int) -> None:
    _check(load_library().bconv_forward_packed_bits(h, _ptr(stream), n, _ptr(in_bits), _ptr(out_bits),
                                                    _ptr(workspace), workspace_bytes))


def bconv_main_kernel(h: int, n: int) -> str:
    return load_library().bconv_main_kernel(h, n).decode()


def bconv_calibrate_popcount(stream, blocks: int, iters: int, seed: int, sink) -> None:
    _check(load_library().bconv_calibrate_popcount(_ptr(stream), blocks, iters, seed, _ptr(sink)))


def bconv_destroy(h: int) -> None:
    _check(load_library().bconv_destroy(h))


def bconv_status_string(s: int) -> str:
    return load_library().bconv_status_string(s).decode()


def bconv_last_error() -> str:
    return load_library().bconv_last_error().decode()
