"""Host-side checks that need no GPU: the shared library loads and exports
every function include/bconv.h declares, descriptor validation returns the
documented codes, the binding fails loudly without the library, and the
seeded workloads are deterministic."""

import ctypes
import os
import re

import numpy as np
import pytest

import popcount_convolution_amd as pca
from popcount_convolution_amd import _binding, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bconv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIB_PATH):
        from popcount_convolution_amd import _build
        _build.build()
    return pca.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bconv_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) == 19, names
    raw = ctypes.CDLL(_binding.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing


def _desc(**kw):
    d = dict(in_h=8, in_w=8, in_c=64, out_c=32, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
             pad_h=1, pad_w=1, groups=1, neuron=0, scale_value=1.0)
    d.update(kw)
    return pca.make_desc(**d)


@pytest.mark.parametrize("kw,type,flags,code", [
    ({}, pca.BCONV_XNOR, 0, pca.BCONV_OK),
    ({}, pca.BCONV_AND, 1, pca.BCONV_OK),
    ({}, pca.BCONV_BINARY_WEIGHTS, 1, pca.BCONV_OK),
    (dict(kernel_h=8, kernel_w=8, pad_h=0, pad_w=0), pca.BCONV_XNOR, 0, pca.BCONV_OK),  # FC shape
    (dict(groups=2), pca.BCONV_XNOR, 0, pca.BCONV_ERR_UNSUPPORTED),
    (dict(groups=0), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, 3, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_XNOR, pca.BCONV_FLAG_INT8_MFMA, pca.BCONV_OK),
    ({}, pca.BCONV_AND, pca.BCONV_FLAG_INT8_MFMA | 1, pca.BCONV_OK),
    ({}, pca.BCONV_BINARY_WEIGHTS, pca.BCONV_FLAG_INT8_MFMA, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_XNOR, pca.BCONV_FLAG_BETA_VALID_TAPS, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_XNOR, pca.BCONV_FLAG_BETA_VALID_TAPS | pca.BCONV_FLAG_USE_BETA_SCALING, pca.BCONV_OK),
    ({}, pca.BCONV_BINARY_WEIGHTS, pca.BCONV_FLAG_BETA_VALID_TAPS | pca.BCONV_FLAG_USE_BETA_SCALING, pca.BCONV_OK),
    ({}, pca.BCONV_AND, 16, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_XNOR, pca.BCONV_FLAG_FP4_MFMA, pca.BCONV_OK),  # the shape is checked by bconv_create
    ({}, pca.BCONV_BINARY_WEIGHTS, pca.BCONV_FLAG_FP4_MFMA, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_AND, pca.BCONV_FLAG_FP4_MFMA | pca.BCONV_FLAG_INT8_MFMA, pca.BCONV_ERR_INVALID_ARGUMENT),
    ({}, pca.BCONV_XNOR, 4, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(neuron=11, neuron_a=-1.0, neuron_b=1.0), pca.BCONV_XNOR, 0, pca.BCONV_OK),  # clamp
    (dict(neuron=12), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(neuron=-1), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(in_h=0), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(in_c=-1), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(out_c=0), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(stride_w=0), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(pad_h=3), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(kernel_h=2, kernel_w=4, pad_h=1, pad_w=2, pad_h_end=0, pad_w_end=1), pca.BCONV_XNOR, 0,
     pca.BCONV_OK),  # centred even kernels
    (dict(pad_h_end=3), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(pad_w_end=-1), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(pad_w=-1), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(kernel_h=11, pad_h=1), pca.BCONV_XNOR, 0, pca.BCONV_ERR_INVALID_ARGUMENT),
    (dict(in_c=1 << 20, kernel_h=5, kernel_w=5, pad_h=0, pad_w=0), pca.BCONV_XNOR, 0,
     pca.BCONV_ERR_INVALID_ARGUMENT),
])
def test_validate_desc(lib, kw, type, flags, code):
    assert pca.bconv_validate_desc(_desc(**kw), type, flags) == code
    if code != pca.BCONV_OK:
        assert pca.bconv_last_error()


def test_validate_null_desc(lib):
    assert lib.bconv_validate_desc(None, 1, 0) == pca.BCONV_ERR_INVALID_ARGUMENT


def test_status_strings(lib):
    for code, name in ((0, "BCONV_OK"), (2, "BCONV_ERR_UNSUPPORTED"), (5, "BCONV_ERR_HIP")):
        assert pca.bconv_status_string(code) == name


def test_null_handle_calls(lib):
    assert lib.bconv_destroy(None) == pca.BCONV_OK
    assert lib.bconv_get_info(None, None, None, None, None) == pca.BCONV_ERR_INVALID_ARGUMENT
    assert lib.bconv_main_kernel(None, 1) == b""
    for fn in (lib.bconv_forward_packed, lib.bconv_forward_packed_bits):
        assert fn(None, None, 1, None, None, None, 0) == pca.BCONV_ERR_INVALID_ARGUMENT


def test_missing_library_fails_loudly():
    with pytest.raises(pca.BconvLibraryMissing):
        _binding.load_library("/nonexistent/libbconv.so")


def test_workloads_deterministic():
    for i, layer in enumerate(workloads.LAYERS[:2]):
        a = workloads.make_inputs(layer, workloads.layer_seed(i))
        b = workloads.make_inputs(layer, workloads.layer_seed(i))
        for k in a:
            if a[k] is None:
                assert b[k] is None
            else:
                assert np.array_equal(a[k], b[k])
        assert a["x"].dtype == np.float32 and a["x"].shape == (layer.n, layer.in_h, layer.in_w, layer.in_c)
        assert a["weight_bits"].dtype == np.uint32
        assert a["weight_bits"].shape == (layer.out_c, layer.kernel_h, layer.kernel_w, layer.words)


def test_measured_layer_shapes():
    L = workloads.LAYERS
    assert [l.type for l in L] == ["xnor", "xnor", "and", "binary_weights", "xnor"]
    assert L[1].use_beta and L[1].neuron == "relu" and L[1].iscale_dist is not None
    assert (L[3].out_h, L[3].out_w) == (28, 28)
    assert L[4].is_fc and (L[4].out_h, L[4].out_w) == (1, 1)
    assert L[4].nominal_macs() == 256 * 4096 * 25088
    assert L[1].nominal_macs() == 3_699_376_128


def test_calibration_argument_errors(lib):
    """Argument errors of the calibration entry point come back before any launch."""
    for blocks, iters, sink in ((0, 1, 0x1000), (1 << 23, 1, 0x1000), (1, -1, 0x1000), (1, 1, None)):
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_calibrate_popcount(None, blocks, iters, 1, sink)
        assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT
