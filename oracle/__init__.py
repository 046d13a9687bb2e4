"""CPU oracle of binary convolution -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library: ``oracle.c`` is a direct, unpacked
evaluation of the output equation of Apple's "MPSCNNBinaryConvolution" page
(Overview), which the "MPSCNNFullyConnected" page reduces the fully connected
layer to (kernel = source size, stride 1, output 1x1).

``bconv(...)`` builds ``liboracle.so`` with gcc on first use if it is missing.

``packed_bconv(...)`` is a second CPU reference point for throughput, not a
checker: the packed-bit popcount form of XNOR / AND on the CPU
(``packed_cpu.c``), itself checked against ``bconv`` by the tests.  The same
import rule applies to it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

TYPE_CODES = {"binary_weights": 0, "xnor": 1, "and": 2}
NEURON_CODES = {"none": 0, "relu": 1,
                "leaky_relu": 2, "linear": 3, "sigmoid": 4,
                "hard_sigmoid": 5, "tanh": 6, "absolute": 7, "softplus": 8,
                "softsign": 9, "elu": 10, "clamp": 11}

_PACKED_SRC = os.path.join(_HERE, "packed_cpu.c")
_PACKED_LIB = os.path.join(_HERE, "libpacked_cpu.so")

_lib = None
_packed = None


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fp contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: Optional[str] = None):
    """Load (building if needed) the oracle library and declare its functions."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if path is None and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(p)
    i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.oracle_bconv.restype = i
    lib.oracle_bconv.argtypes = [i] * 16 + [f, f, f] + [vp] * 12 + [i]
    lib.oracle_out_dim.restype = i
    lib.oracle_out_dim.argtypes = [i, i, i, i]
    lib.oracle_out_dim2.restype = i
    lib.oracle_out_dim2.argtypes = [i, i, i, i, i]
    if path is None:
        _lib = lib
    return lib


def build_packed(out: str = _PACKED_LIB) -> str:
    """Compile the packed CPU baseline with gcc (-O3, OpenMP, hardware popcount)."""
    cmd = ["gcc", "-std=c11", "-O3", "-mpopcnt", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           _PACKED_SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load_packed():
    global _packed
    if _packed is not None:
        return _packed
    if not os.path.exists(_PACKED_LIB) or os.path.getmtime(_PACKED_LIB) < os.path.getmtime(_PACKED_SRC):
        build_packed()
    lib = ctypes.CDLL(_PACKED_LIB)
    i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.packed_bconv.restype = i
    lib.packed_bconv.argtypes = [i] * 16 + [f] + [vp] * 8 + [i]
    _packed = lib
    return lib


def packed_bconv(layer, inputs: dict, threads: int = 0, images=None) -> dict:
    """The packed-bit CPU baseline on a ``workloads.Layer`` (XNOR / AND,
    neuron none or ReLU): fp32 ``out`` and int32 ``acc``."""
    lib = load_packed()
    x = inputs["x"] if images is None else inputs["x"][images]
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    out = np.empty((n, layer.out_h, layer.out_w, layer.out_c), np.float32)
    acc = np.empty(out.shape, np.int32)

    def f32(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.float32)

    keep = [f32(inputs.get(k)) for k in ("output_scale", "output_bias", "input_scale", "input_bias")]
    wb = np.ascontiguousarray(inputs["weight_bits"], dtype=np.uint32)
    rc = lib.packed_bconv(n, layer.in_h, layer.in_w, layer.in_c, layer.out_c, layer.kernel_h, layer.kernel_w,
                          layer.stride_h, layer.stride_w, layer.pad_h, layer.pad_w, layer.pad_h_end, layer.pad_w_end,
                          TYPE_CODES[layer.type], 0 if not layer.use_beta else (2 if layer.beta_valid_taps else 1),
                          NEURON_CODES[layer.neuron],
                          float(layer.scale_value), _ptr(x), _ptr(wb), *[_ptr(k) for k in keep], _ptr(out),
                          _ptr(acc), int(threads))
    if rc != 0:
        raise ValueError("packed CPU baseline: arguments outside its scope")
    return {"out": out, "acc": acc}


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def out_dim(size: int, kernel: int, stride: int, pad: int, pad_end: Optional[int] = None) -> int:
    """Output extent for leading padding `pad` and trailing `pad_end` (= pad when omitted)."""
    return load().oracle_out_dim2(size, kernel, stride, pad, pad if pad_end is None else pad_end)


def bconv(x: np.ndarray, weight_bits: np.ndarray, *, type: str, out_c: int,
          kernel=(1, 1), stride=(1, 1), pad=(0, 0), pad_end=None, output_scale=None, output_bias=None,
          input_scale=None, input_bias=None, use_beta: bool = False, neuron: str = "none",
          scale_value: float = 1.0, neuron_a: float = 0.0, neuron_b: float = 0.0, threads: int = 0,
          want=("out", "acc", "beta", "a_map", "signs"), beta_divisor: str = "window",
          lib=None) -> dict:
    """Evaluate binary convolution on the CPU.

    ``x`` is float32 NHWC, ``weight_bits`` uint32 ``[out_c][kh][kw][ceil(Cin/32)]``.
    ``pad`` is the leading (top, left) zero padding and ``pad_end`` the
    trailing (bottom, right) one, equal to ``pad`` when omitted.
    Returns a dict of float64 ``out``, the pre-epilogue sum ``acc`` (int32 for
    XNOR/AND, float64 for binary_weights), ``beta`` [n,oh,ow], ``a_map``
    [n,h,w] (with ``use_beta``) and the binarised input ``signs`` (int8).
    ``beta_divisor`` is "window" (beta = window sum of A / (kh*kw)) or
    "valid" (/ the window's in-image taps).
    """
    if beta_divisor not in ("window", "valid"):
        raise ValueError(f"beta_divisor {beta_divisor!r}")
    beta_mode = 0 if not use_beta else (2 if beta_divisor == "valid" else 1)
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    weight_bits = np.ascontiguousarray(weight_bits, dtype=np.uint32)
    n, h, w, c = x.shape
    kh, kw = kernel
    sh, sw = stride
    ph, pw = pad
    phe, pwe = pad if pad_end is None else pad_end
    words = (c + 31) // 32
    if weight_bits.shape != (out_c, kh, kw, words):
        raise ValueError(f"weight_bits shape {weight_bits.shape} != {(out_c, kh, kw, words)}")
    oh = lib.oracle_out_dim2(h, kh, sh, ph, phe)
    ow = lib.oracle_out_dim2(w, kw, sw, pw, pwe)
    if oh <= 0 or ow <= 0:
        raise ValueError("kernel larger than the padded input")

    def f32(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.float32)

    output_scale, output_bias = f32(output_scale), f32(output_bias)
    input_scale, input_bias = f32(input_scale), f32(input_bias)
    out = np.empty((n, oh, ow, out_c), np.float64)
    t = TYPE_CODES[type]
    acc_i = np.empty((n, oh, ow, out_c), np.int32) if ("acc" in want and t != 0) else None
    acc_r = np.empty((n, oh, ow, out_c), np.float64) if ("acc" in want and t == 0) else None
    signs = np.empty((n, h, w, c), np.int8) if ("signs" in want and t != 0) else None
    a_map = np.empty((n, h, w), np.float64) if ("a_map" in want and use_beta) else None
    beta = np.empty((n, oh, ow), np.float64) if "beta" in want else None
    rc = lib.oracle_bconv(n, h, w, c, out_c, kh, kw, sh, sw, ph, pw, phe, pwe, t, beta_mode,
                          NEURON_CODES[neuron], float(scale_value), float(neuron_a), float(neuron_b),
                          _ptr(x), _ptr(weight_bits),
                          _ptr(output_scale), _ptr(output_bias), _ptr(input_scale),
                          _ptr(input_bias), _ptr(out), _ptr(acc_i), _ptr(acc_r), _ptr(signs),
                          _ptr(a_map), _ptr(beta), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return {"out": out, "acc": acc_i if t != 0 else acc_r, "beta": beta, "a_map": a_map,
            "signs": signs}


def bconv_layer(layer, inputs: dict, threads: int = 0, lib=None, **kw) -> dict:
    """``bconv`` on a ``workloads.Layer`` and the arrays ``make_inputs`` drew."""
    return bconv(inputs["x"], inputs["weight_bits"], type=layer.type, out_c=layer.out_c,
                 kernel=(layer.kernel_h, layer.kernel_w), stride=(layer.stride_h, layer.stride_w),
                 pad=(layer.pad_h, layer.pad_w), pad_end=(layer.pad_h_end, layer.pad_w_end),
                 output_scale=inputs.get("output_scale"),
                 output_bias=inputs.get("output_bias"), input_scale=inputs.get("input_scale"),
                 input_bias=inputs.get("input_bias"), use_beta=layer.use_beta,
                 neuron=layer.neuron, scale_value=layer.scale_value, neuron_a=layer.neuron_a,
                 neuron_b=layer.neuron_b, threads=threads, lib=lib,
                 beta_divisor="valid" if layer.beta_valid_taps else "window", **kw)
