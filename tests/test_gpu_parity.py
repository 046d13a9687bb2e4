"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case draws seeded host inputs once; the same arrays feed the GPU and the
oracle.  Integer window sums and packed bits must be bit-exact; float results
follow the normwise bounds documented in ``parity.py``.
"""

import numpy as np
import pytest
import torch

import oracle
import parity
import popcount_convolution_amd as pca
from popcount_convolution_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pca.load_library()
    return torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ measured layers

_MEASURED_REF = {}


def measured_reference(index):
    """Seeded inputs of measured layer ``index`` and the oracle's result on the
    whole batch (computed once per test session: the fp32, int8 and sign-bit
    tests of a layer compare against the same reference)."""
    if index not in _MEASURED_REF:
        layer = workloads.LAYERS[index]
        inputs = workloads.make_inputs(layer, workloads.layer_seed(index))
        _MEASURED_REF.clear()  # one layer's reference at a time bounds host memory
        _MEASURED_REF[index] = (inputs, oracle.bconv_layer(layer, inputs))
    return _MEASURED_REF[index]


@pytest.mark.parametrize("index", range(len(workloads.LAYERS)),
                         ids=[l.name for l in workloads.LAYERS])
def test_measured_layer_full(dev, index):
    """Each measured layer at full size, in the launch configuration the
    benchmark times, compared with the oracle on every output of the whole
    batch (every image, so every XCD's share of the strips, and every row
    group of the fully connected product)."""
    layer = workloads.LAYERS[index]
    _log(f"layer {layer.name} seed {workloads.layer_seed(index)}")
    inputs, ref = measured_reference(index)
    got = parity.run_gpu(layer, inputs, dev)
    parity.compare(layer, inputs, got, ref=ref)


def test_small_layer_full(dev):
    """The single-image layer compared on every output, fast and generic paths."""
    layer = workloads.LAYERS[0]
    inputs = workloads.make_inputs(layer, workloads.layer_seed(0))
    ref = oracle.bconv_layer(layer, inputs)
    for generic in (False, True):
        got = parity.run_gpu(layer, inputs, dev, generic=generic)
        parity.compare(layer, inputs, got, ref=ref)


def test_bench_layer_two_full_images(dev):
    """The benchmark layer (XNOR + beta + affine + ReLU) on two whole images,
    every output, fast and generic kernels."""
    layer = workloads.BENCH_LAYER.with_(n=2)
    inputs = workloads.make_inputs(layer, 77)
    ref = oracle.bconv_layer(layer, inputs)
    for generic in (False, True):
        got = parity.run_gpu(layer, inputs, dev, generic=generic)
        parity.compare(layer, inputs, got, ref=ref)


# ---------------------------------------------------------------- sweeps

def _sweep_layers():
    """Geometries that span several channel tiles and strips with ragged
    tails, every word-count tail, all strides/paddings the kernels special-
    case, 1x1 / 2x2 / 3x3 / 5x5 kernels and the FC shape."""
    base = workloads.Layer("sweep", "xnor", 2, 9, 10, 64, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(n=3, in_h=11, in_w=19, in_c=128, out_c=130),             # 3 tiles, ragged strips
        dict(n=1, in_h=5, in_w=7, in_c=33, out_c=65),
        dict(n=2, in_h=8, in_w=8, in_c=100, out_c=1),
        dict(n=2, in_h=14, in_w=14, in_c=256, out_c=64, stride_h=2, stride_w=2),
        dict(n=1, in_h=13, in_w=9, in_c=96, out_c=40, stride_h=2, stride_w=2, pad_h=0, pad_w=0),
        dict(n=2, in_h=6, in_w=21, in_c=31, out_c=17),
        dict(n=1, in_h=1, in_w=1, in_c=64, out_c=8),                  # every tap but one padded
        dict(n=2, in_h=9, in_w=9, in_c=1, out_c=3),                   # Cin = 1
        dict(n=2, in_h=10, in_w=12, in_c=64, out_c=64, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0),
        dict(n=1, in_h=9, in_w=9, in_c=160, out_c=64, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0,
             stride_h=2, stride_w=3),
        dict(n=2, in_h=12, in_w=11, in_c=64, out_c=33, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2),
        dict(n=1, in_h=10, in_w=10, in_c=32, out_c=20, kernel_h=5, kernel_w=5, pad_h=1, pad_w=3),
        dict(n=2, in_h=7, in_w=8, in_c=45, out_c=9, kernel_h=2, kernel_w=2, pad_h=1, pad_w=1),
        dict(n=1, in_h=9, in_w=10, in_c=70, out_c=5, kernel_h=3, kernel_w=1, pad_h=1, pad_w=0,
             stride_h=3, stride_w=1),
        dict(n=3, in_h=4, in_w=5, in_c=37, out_c=66, kernel_h=4, kernel_w=5, pad_h=0, pad_w=0),  # FC
        dict(n=2, in_h=3, in_w=3, in_c=512, out_c=100, kernel_h=3, kernel_w=3, pad_h=0, pad_w=0),  # FC
        dict(n=1, in_h=16, in_w=16, in_c=96, out_c=64),
        dict(n=1, in_h=8, in_w=56, in_c=128, out_c=128),
        dict(n=1, in_h=7, in_w=28, in_c=256, out_c=256),
        dict(n=2, in_h=5, in_w=6, in_c=1000, out_c=40),                # pack: channel chunks in a loop
        dict(n=2, in_h=7, in_w=37, in_c=12, out_c=24),                 # pack: 16 pixels a pass, ragged runs
        dict(n=2, in_h=5, in_w=70, in_c=8, out_c=16),                  # pack: 32 pixels a pass
        dict(n=1, in_h=6, in_w=9, in_c=20, out_c=9),                   # pack: 8 lanes a pixel, idle lanes
        dict(n=3, in_h=3, in_w=5, in_c=768, out_c=24, kernel_h=3, kernel_w=3, pad_h=0, pad_w=0),  # 256-channel parts
    ]
    out = []
    for gi, gd in enumerate(geoms):
        for form in ("xnor", "and", "binary_weights"):
            for variant in range(2):
                kw = dict(gd)
                kw["type"] = form
                kw["name"] = f"g{gi}_{form}_v{variant}"
                if variant == 1:
                    kw.update(use_beta=True, neuron="relu", iscale_dist=("uniform", 0.5, 1.5),
                              ibias_dist=("normal", 0.0, 0.2))
                if (gi + variant) % 3 == 2:
                    kw.update(oscale_dist=None, obias_dist=None, scale_value=0.75)
                out.append(base.with_(**kw))
    return out


SWEEP = _sweep_layers()


@pytest.mark.parametrize("layer", SWEEP, ids=[l.name for l in SWEEP])
def test_sweep(dev, layer):
    inputs = workloads.make_inputs(layer, 5000 + SWEEP.index(layer))
    _log(f"sweep {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev)
    parity.compare(layer, inputs, got, ref=ref)
    gen = parity.run_gpu(layer, inputs, dev, generic=True)
    parity.compare(layer, inputs, gen, ref=ref)


# ------------------------------------------------------- valid-tap beta

_VT = workloads.BENCH_LAYER.with_(n=2, in_h=13, in_w=17, beta_valid_taps=True)
VALID_TAP_CASES = [
    (_VT.with_(name="vt_xnor_k3"), False, False),
    (_VT.with_(name="vt_xnor_k3_generic"), True, False),
    (_VT.with_(name="vt_xnor_k3_int8"), False, True),
    (_VT.with_(name="vt_and_k4_centred", type="and", kernel_h=4, kernel_w=4, pad_h=2, pad_w=2, pad_bottom=1,
               pad_right=1), False, False),
    (_VT.with_(name="vt_xnor_k5_s2", kernel_h=5, kernel_w=5, pad_h=2, pad_w=2, stride_h=2, stride_w=2), False, False),
    (_VT.with_(name="vt_xnor_k2_s2_centred", kernel_h=2, kernel_w=2, pad_h=1, pad_w=1, pad_bottom=0, pad_right=0,
               stride_h=2, stride_w=2, in_c=64), False, False),
    (_VT.with_(name="vt_binary_weights", type="binary_weights", in_c=64), False, False),
    (_VT.with_(name="vt_binary_weights_generic", type="binary_weights", in_c=40, stride_h=2, stride_w=2), True, False),
    (_VT.with_(name="vt_fc", n=3, in_h=4, in_w=5, in_c=96, out_c=70, kernel_h=4, kernel_w=5, pad_h=0, pad_w=0),
     False, False),
]


@pytest.mark.parametrize("layer,generic,int8", VALID_TAP_CASES, ids=[c[0].name for c in VALID_TAP_CASES])
def test_beta_valid_taps(dev, layer, generic, int8):
    """BCONV_FLAG_BETA_VALID_TAPS on every kernel path: beta (from the
    workspace), window sums and outputs against the oracle's valid-tap
    reading; the FC shape has no padding, so the flag changes nothing."""
    inputs = workloads.make_inputs(layer, 3100 + VALID_TAP_CASES.index((layer, generic, int8)))
    _log(f"valid taps {layer.name} generic={generic} int8={int8}")
    got = parity.run_gpu(layer, inputs, dev, generic=generic, int8_mfma=int8)
    ref = parity.compare(layer, inputs, got)
    window = oracle.bconv_layer(layer.with_(beta_valid_taps=False), inputs)
    if layer.pad_h or layer.pad_w:
        assert not np.allclose(ref["beta"], window["beta"])
    else:
        np.testing.assert_array_equal(ref["beta"], window["beta"])


# ------------------------------------------------------- specialised kernels

# (kernel_h, kernel_w, words per pixel, stride) of every compiled instance of
# the specialised XNOR / AND convolution, and its strip widths.
FAST_SHAPES = ([(3, 3, cw, 1) for cw in (1, 2, 3, 4, 8)] + [(3, 3, cw, 2) for cw in (1, 2, 4, 8)]
               + [(1, 1, cw, s) for s in (1, 2) for cw in (1, 2, 4, 8)]
               + [(k, k, cw, s) for k in (2, 4, 5) for s in (1, 2) for cw in (1, 2, 4)])
STRIP_WIDTHS = (4, 6, 7, 8)


def _fast_layer(kh, kw, cw, sw, p, form, variant):
    """Two images, two channel tiles (the second ragged), a ragged last word,
    centred padding (an even kernel pads one less at the end) and rows of
    two whole strips of width p plus a ragged one."""
    ph, pw = kh // 2, kw // 2
    out_w = 2 * p + 3
    in_w = (out_w - 1) * sw + kw - pw - (kw - 1 - pw)
    kwargs = dict(name=f"k{kh}x{kw}_w{cw}_s{sw}_p{p}_{form}_v{variant}", type=form, n=2, in_h=7, in_w=in_w,
                  in_c=32 * cw - 5 if cw > 1 else 27, out_c=70, kernel_h=kh, kernel_w=kw,
                  stride_h=sw, stride_w=sw, pad_h=ph, pad_w=pw, pad_bottom=kh - 1 - ph, pad_right=kw - 1 - pw)
    if variant:
        kwargs.update(use_beta=True, neuron="relu", iscale_dist=("uniform", 0.5, 1.5),
                      ibias_dist=("normal", 0.0, 0.2))
    return workloads.Layer(**kwargs)


@pytest.mark.parametrize("shape", FAST_SHAPES, ids=["k{}x{}_w{}_s{}".format(*s) for s in FAST_SHAPES])
def test_fast_kernel_instances(dev, shape):
    """Every compiled instance (each strip width, XNOR and AND, with and
    without beta / input affine / ReLU) matches the oracle on a layer with
    borders on all sides and ragged strips, tiles and words."""
    kh, kw, cw, sw = shape
    for i, p in enumerate(STRIP_WIDTHS):
        for j, form in enumerate(("xnor", "and")):
            layer = _fast_layer(kh, kw, cw, sw, p, form, (i + j) % 2)
            assert layer.out_w == 2 * p + 3 and (layer.in_c + 31) // 32 == cw
            inputs = workloads.make_inputs(layer, 9000 + 8 * FAST_SHAPES.index(shape) + 2 * i + j)
            _log(f"fast {layer}")
            got = parity.run_gpu(layer, inputs, dev, strip_width=p)
            assert got["main_kernel"] == f"xconv_fast<{kh},{kw},{cw},{sw},{p}>"
            parity.compare(layer, inputs, got)


def test_special_values(dev):
    """Signed zeros, NaN, subnormals and exact ties of the input affine
    binarise as the oracle says (x' < 0 -> -1, else +1)."""
    layer = workloads.Layer("special", "xnor", 1, 4, 4, 64, 64, 3, 3, 1, 1, 1, 1)
    inputs = workloads.make_inputs(layer, 91)
    x = inputs["x"]
    specials = np.array([0.0, -0.0, np.nan, 1e-40, -1e-40, -1e-45, 1e-45, -np.inf, np.inf],
                        np.float32)
    flat = x.reshape(-1)
    flat[: specials.size * 7: 7] = np.resize(specials, flat[: specials.size * 7: 7].shape)
    inputs["x"] = x
    for form in ("xnor", "and"):
        ly = layer.with_(type=form)
        ref = oracle.bconv_layer(ly, inputs)
        # the pack kernel's bits (two-kernel path) ...
        got = parity.run_gpu(ly, inputs, dev, small_fused=False)
        assert np.array_equal(got["acc"], ref["acc"])
        ph, pw = got["bits_pad"]
        assert np.array_equal(got["bits"][:, ph:ph + 4, pw:pw + 4], parity.expected_words(ref["signs"], form))
        # ... and the single-launch kernel's own binarisation
        got = parity.run_gpu(ly, inputs, dev, small_fused=True)
        assert got["main_kernel"].startswith("xconv_small")
        assert np.array_equal(got["acc"], ref["acc"])


def test_binary_weights_special_values(dev):
    """binaryWeights keeps full-precision input: infinities and NaN propagate
    as in the oracle's sum (same sign of infinity, NaN where it has NaN),
    signed zeros and subnormals count at their value, and an image of tiny
    values (whose low-order pieces are subnormal) meets the normwise bound
    with no absolute slack.  Both kernels (matrix-core and VALU)."""
    layer = workloads.Layer("special_bw", "binary_weights", 3, 6, 7, 64, 70, 3, 3, 1, 1, 1, 1)
    inputs = workloads.make_inputs(layer, 92)
    x = inputs["x"]
    specials = np.array([0.0, -0.0, 1e-40, -1e-40, 1e-45, -1e-45, np.inf, -np.inf, np.nan],
                        np.float32)
    img0 = x[0].reshape(-1)
    img0[: specials.size * 97: 97] = specials
    x[1] = x[1] * np.float32(1e-37)       # normal fp32, pieces below bf16's normal range
    x[2] = x[2] * np.float32(1e-41)       # subnormal fp32
    inputs["x"] = x
    ref = oracle.bconv_layer(layer, inputs)
    S = parity.window_abs_sum(layer, inputs)[..., None]
    for generic in (False, True):
        got = parity.run_gpu(layer, inputs, dev, generic=generic)
        for key in ("acc", "out"):
            g, o = got[key].astype(np.float64), ref[key]
            nonfinite = ~np.isfinite(o)
            assert nonfinite[0].any(), "the specials must reach some window"
            assert np.array_equal(np.isnan(g), np.isnan(o)), f"{key}: NaN positions differ"
            inf = np.isinf(o)
            assert np.array_equal(g[inf], o[inf]), f"{key}: infinities differ"
        g, o = got["acc"].astype(np.float64), ref["acc"]
        fin = np.isfinite(o) & np.isfinite(S)
        err = np.abs(g[fin] - o[fin])
        assert np.all(err <= parity.RTOL * np.broadcast_to(S, o.shape)[fin]), \
            f"generic={generic}: sums off by {err.max()}"
        assert np.any(g[1] != 0) and np.any(g[2] != 0), "tiny values must not flush to zero"


# ------------------------------------------------------------ activations

NEURON_PARAMS = {"leaky_relu": (0.1, 0.0), "linear": (0.5, -0.25), "sigmoid": (0.0, 0.0),
                 "hard_sigmoid": (0.2, 0.5), "tanh": (1.5, 0.7), "absolute": (0.0, 0.0),
                 "softplus": (0.8, 1.3), "softsign": (0.0, 0.0), "elu": (0.6, 0.0), "clamp": (-0.5, 0.75),
                 "relu": (0.0, 0.0), "none": (0.0, 0.0)}


def _neuron_layers():
    # output scale ~0.01 so the values sit in every activation's curved range
    xnor = workloads.Layer("act", "xnor", 2, 9, 10, 64, 70, 3, 3, 1, 1, 1, 1,
                           oscale_dist=("uniform", 0.002, 0.02), obias_dist=("normal", 0.0, 1.0))
    bw = xnor.with_(type="binary_weights", in_c=24, oscale_dist=("uniform", 0.1, 0.5))
    out = []
    for name, (a, b) in NEURON_PARAMS.items():
        out.append(xnor.with_(name=f"act_xnor_{name}", neuron=name, neuron_a=a, neuron_b=b))
        out.append(bw.with_(name=f"act_bw_{name}", neuron=name, neuron_a=a, neuron_b=b))
    return out


NEURON_LAYERS = _neuron_layers()


@pytest.mark.parametrize("layer", NEURON_LAYERS, ids=[l.name for l in NEURON_LAYERS])
def test_neuron(dev, layer):
    """Every activation through the specialised and generic kernels (and the
    int8 path for XNOR), fp32 outputs and sign bits."""
    inputs = workloads.make_inputs(layer, 9500 + NEURON_LAYERS.index(layer))
    _log(f"neuron {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    variants = [dict(generic=False), dict(generic=True)]
    if layer.type != "binary_weights":
        variants.append(dict(int8_mfma=True))
    for v in variants:
        got = parity.run_gpu(layer, inputs, dev, **v)
        parity.compare(layer, inputs, got, ref=ref)
    words, out, kernel = _run_bits(layer, inputs, dev)
    assert np.array_equal(parity.unpack_words(words, layer.out_c), (~(out < 0)).astype(np.uint8)), kernel
    parity.compare_bits(layer, inputs, words, ref=ref)


# ------------------------------------------------ asymmetric padding

def _pad_layers():
    base = workloads.Layer("pad", "xnor", 2, 9, 11, 64, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(name="pad_k2_centred", kernel_h=2, kernel_w=2, pad_h=1, pad_w=1, pad_bottom=0, pad_right=0),
        dict(name="pad_k4_centred_beta", kernel_h=4, kernel_w=4, pad_h=2, pad_w=2, pad_bottom=1, pad_right=1,
             use_beta=True, iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2)),
        dict(name="pad_k4_and_cw2", type="and", in_c=50, kernel_h=4, kernel_w=4, pad_h=2, pad_w=2,
             pad_bottom=1, pad_right=1, x_dist=("normal", 0.2, 1.0)),
        dict(name="pad_k2_cw4", in_c=128, out_c=130, kernel_h=2, kernel_w=2, pad_h=1, pad_w=1, pad_bottom=0,
             pad_right=0, n=3, in_h=14, in_w=15),
        dict(name="pad_k3_top_only", pad_h=2, pad_w=0, pad_bottom=0, pad_right=2),
        dict(name="pad_k3_s2_asym", in_c=96, stride_h=2, stride_w=2, pad_h=0, pad_w=1, pad_bottom=2, pad_right=0),
        dict(name="pad_k6_centred", in_c=20, out_c=33, kernel_h=6, kernel_w=6, pad_h=3, pad_w=3, pad_bottom=2,
             pad_right=2),
        dict(name="pad_bw_k4", type="binary_weights", in_c=24, kernel_h=4, kernel_w=4, pad_h=2, pad_w=2,
             pad_bottom=1, pad_right=1, use_beta=True),
        dict(name="pad_bw_k3_asym_s2", type="binary_weights", in_c=64, out_c=128, stride_h=2, stride_w=2,
             pad_h=1, pad_w=0, pad_bottom=0, pad_right=2),
        dict(name="pad_fc_like_trailing", n=3, in_h=4, in_w=5, in_c=40, out_c=20, kernel_h=4, kernel_w=5,
             pad_h=0, pad_w=0, pad_bottom=1, pad_right=2),
    ]
    return [base.with_(**g) for g in geoms]


PAD_LAYERS = _pad_layers()


@pytest.mark.parametrize("layer", PAD_LAYERS, ids=[l.name for l in PAD_LAYERS])
def test_asymmetric_padding(dev, layer):
    """Different leading and trailing padding (the centred window of even
    kernels), on the specialised, generic and int8 paths."""
    inputs = workloads.make_inputs(layer, 9000 + PAD_LAYERS.index(layer))
    _log(f"pad {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    assert ref["out"].shape[1:3] == (layer.out_h, layer.out_w)
    for generic in (False, True):
        got = parity.run_gpu(layer, inputs, dev, generic=generic)
        parity.compare(layer, inputs, got, ref=ref)
    if layer.type != "binary_weights":
        got = parity.run_gpu(layer, inputs, dev, int8_mfma=True)
        parity.compare(layer, inputs, got, ref=ref)


# ------------------------------------------------ int8 matrix-core comparison path

def _int8_layers():
    base = workloads.Layer("i8", "xnor", 2, 9, 10, 64, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(name="i8_bench", **{k: getattr(workloads.BENCH_LAYER, k) for k in (
            "type", "in_h", "in_w", "in_c", "out_c", "use_beta", "neuron", "iscale_dist", "ibias_dist")}),
        dict(name="i8_and", type="and", n=2, in_h=28, in_w=28, in_c=256, out_c=256, x_dist=("normal", 0.2, 1.0)),
        dict(name="i8_small", n=1, in_h=16, in_w=16, in_c=64, out_c=64),
        dict(name="i8_ragged", n=3, in_h=11, in_w=19, in_c=100, out_c=130, use_beta=True, neuron="relu"),
        dict(name="i8_cin33", type="and", n=1, in_h=5, in_w=7, in_c=33, out_c=65),
        dict(name="i8_s2", n=2, in_h=14, in_w=14, in_c=256, out_c=64, stride_h=2, stride_w=2),
        dict(name="i8_1x1", n=2, in_h=10, in_w=12, in_c=64, out_c=64, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0),
        dict(name="i8_5x5", n=1, in_h=12, in_w=11, in_c=64, out_c=33, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2),
        dict(name="i8_fc", n=3, in_h=4, in_w=5, in_c=37, out_c=66, kernel_h=4, kernel_w=5, pad_h=0, pad_w=0),
        dict(name="i8_1px", n=1, in_h=1, in_w=1, in_c=64, out_c=8),
    ]
    return [base.with_(**g) for g in geoms]


INT8_LAYERS = _int8_layers()
INT8_MEASURED = [i for i, l in enumerate(workloads.LAYERS) if l.type != "binary_weights"]


@pytest.mark.parametrize("index", INT8_MEASURED, ids=[workloads.LAYERS[i].name for i in INT8_MEASURED])
def test_int8_mfma_measured_layer_full(dev, index):
    """The int8 path on each XNOR / AND measured layer at full size, every
    output compared with the oracle."""
    layer = workloads.LAYERS[index]
    _log(f"int8 layer {layer.name} seed {workloads.layer_seed(index)}")
    inputs, ref = measured_reference(index)
    got = parity.run_gpu(layer, inputs, dev, int8_mfma=True)
    assert got["main_kernel"] == "i8mma_kernel"
    parity.compare(layer, inputs, got, ref=ref)


@pytest.mark.parametrize("layer", INT8_LAYERS, ids=[l.name for l in INT8_LAYERS])
def test_int8_mfma_path(dev, layer):
    """BCONV_FLAG_INT8_MFMA: the same exact window sums and epilogue as the
    popcount path, and the int8 values of the workspace are the oracle's
    binarised input with a zero halo and zero channel padding."""
    inputs = workloads.make_inputs(layer, 7000 + INT8_LAYERS.index(layer))
    _log(f"int8 {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev, int8_mfma=True)
    assert got["main_kernel"] == "i8mma_kernel"
    parity.compare(layer, inputs, got, ref=ref)


# ------------------------------------------------ packed sign-bit output

def _bits_layers():
    base = workloads.Layer("bits", "xnor", 2, 9, 10, 64, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(name="bits_xnor_o70", use_beta=True, iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2)),
        dict(name="bits_xnor_o33", n=3, in_h=11, in_w=19, in_c=100, out_c=33),
        dict(name="bits_and_o130", type="and", in_c=96, out_c=130, x_dist=("normal", 0.2, 1.0),
             obias_dist=("normal", -20.0, 5.0)),
        dict(name="bits_xnor_relu", out_c=128, neuron="relu"),
        dict(name="bits_xnor_s2_o96", in_h=14, in_w=14, in_c=128, out_c=96, stride_h=2, stride_w=2),
        dict(name="bits_fc_o66", n=5, in_h=4, in_w=5, in_c=37, out_c=66, kernel_h=4, kernel_w=5, pad_h=0, pad_w=0),
        dict(name="bits_bw_o130", type="binary_weights", in_c=64, out_c=130, stride_h=2, stride_w=2),
        dict(name="bits_bw_o40_beta", type="binary_weights", in_c=13, out_c=40, use_beta=True),
        dict(name="bits_1px_o5", n=1, in_h=1, in_w=1, in_c=64, out_c=5),
    ]
    return [base.with_(**g) for g in geoms]


BITS_LAYERS = _bits_layers()


def _run_bits(layer, inputs, dev, generic=False, int8=False, fp4=False):
    with parity.force_generic(generic):
        conv = pca.BinaryConvolution.from_layer(layer, inputs, int8_mfma=int8, fp4_mfma=fp4)
    try:
        x = torch.from_numpy(inputs["x"]).to(dev)
        words = conv.forward_bits(x).cpu().numpy()
        out = conv.forward(x).cpu().numpy()
        torch.cuda.synchronize()
        return words, out, conv.main_kernel(x.shape[0])
    finally:
        conv.close()


@pytest.mark.parametrize("layer", BITS_LAYERS, ids=[l.name for l in BITS_LAYERS])
def test_forward_bits(dev, layer):
    """bconv_forward_bits: the sign bits of the fp32 output, packed for the next
    binary layer, on the specialised and generic kernels (and the int8 path for
    XNOR / AND); exactly the signs of the same kernel's fp32 output, and the
    oracle's signs wherever fp32 rounding cannot decide them."""
    inputs = workloads.make_inputs(layer, 8000 + BITS_LAYERS.index(layer))
    _log(f"bits {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    variants = [dict(generic=False), dict(generic=True)]
    if layer.type != "binary_weights":
        variants.append(dict(int8=True))
    for v in variants:
        words, out, kernel = _run_bits(layer, inputs, dev, **v)
        bits = parity.unpack_words(words, layer.out_c)
        assert np.array_equal(bits, (~(out < 0)).astype(np.uint8)), f"{kernel}: bits differ from its fp32 signs"
        parity.compare_bits(layer, inputs, words, ref=ref)


@pytest.mark.parametrize("index", range(len(workloads.LAYERS)), ids=[l.name for l in workloads.LAYERS])
def test_forward_bits_measured_layer(dev, index):
    """Sign bits on each measured layer at full size, every bit compared with
    the oracle's signs (where fp32 rounding cannot decide them)."""
    layer = workloads.LAYERS[index]
    _log(f"bits layer {layer.name}")
    inputs, ref = measured_reference(index)
    words, out, kernel = _run_bits(layer, inputs, dev)
    bits = parity.unpack_words(words, layer.out_c)
    assert np.array_equal(bits, (~(out < 0)).astype(np.uint8)), f"{kernel}: bits differ from its fp32 signs"
    parity.compare_bits(layer, inputs, words, ref=ref)


# ------------------------------------------------ packed sign-bit input

def _packed_layers():
    base = workloads.Layer("packed", "xnor", 2, 14, 14, 128, 128, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(name="packed_xnor_k3_c128"),
        dict(name="packed_and_k3_c256_o70", type="and", in_c=256, out_c=70, obias_dist=("normal", -20.0, 5.0)),
        dict(name="packed_xnor_tail_c100_o33", n=3, in_h=11, in_w=19, in_c=100, out_c=33, neuron="relu"),
        dict(name="packed_and_tail_c37_s2", type="and", in_h=13, in_w=9, in_c=37, out_c=40, stride_h=2,
             stride_w=2),
        dict(name="packed_fc_c37_o66", n=5, in_h=4, in_w=5, in_c=37, out_c=66, kernel_h=4, kernel_w=5, pad_h=0,
             pad_w=0),
        dict(name="packed_xnor_k5_p2_c64", in_c=64, out_c=64, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2),
        dict(name="packed_xnor_k1_c64_o96", in_c=64, out_c=96, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0),
        dict(name="packed_and_k2x4_asym", type="and", in_c=32, out_c=64, kernel_h=2, kernel_w=4, pad_h=1, pad_w=2,
             pad_bottom=0, pad_right=1),
        dict(name="packed_xnor_1px_c1", n=1, in_h=1, in_w=1, in_c=1, out_c=5),
    ]
    return [base.with_(**g) for g in geoms]


PACKED_LAYERS = _packed_layers()


def _packed_run(layer, inputs, words, dev, generic=False, fp4=False):
    """forward_packed (fp32 and bits) of `words` on a workspace poisoned with
    0xA5, and forward / forward_accum of the +-1 values the words stand for, on
    one handle.  Also returns the padded bit buffer the repad kernel wrote."""
    values = parity.values_from_bits(words, layer.in_c)
    with parity.force_generic(generic):
        conv = pca.BinaryConvolution.from_layer(layer, inputs, fp4_mfma=fp4)
    try:
        n = words.shape[0]
        w = torch.from_numpy(words.view(np.int32)).to(dev)
        x = torch.from_numpy(values).to(dev)
        shape = (n, conv.out_h, conv.out_w, conv.out_c)
        ws = conv.workspace(n, dev)
        ws.fill_(0xA5)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
        conv.forward_packed(w, out, ws)
        torch.cuda.synchronize()
        L = pca.bconv_workspace_layout(conv.handle, n)
        cnt = n * L["bits_rows"] * L["bits_cols"] * L["bits_words"]
        padded = ws.cpu().numpy()[L["bits_offset"]:L["bits_offset"] + 4 * cnt].view("<u4") \
            .reshape(n, L["bits_rows"], L["bits_cols"], L["bits_words"])
        ws.fill_(0xA5)
        out_bits = conv.forward_packed(w, workspace=ws, bits_out=True)
        ref_out = conv.forward(x)
        acc = conv.forward_accum(x)
        torch.cuda.synchronize()
        return dict(out=out.cpu().numpy(), bits=out_bits.cpu().numpy(), values=values,
                    via_values=ref_out.cpu().numpy(), acc=acc.cpu().numpy(), padded=padded,
                    pad=(L["bits_pad_h"], L["bits_pad_w"]), kernel=conv.main_kernel(n))
    finally:
        conv.close()


def _check_packed(layer, inputs, words, r, images=None):
    """The packed-input results against the oracle on the +-1 values."""
    sub = dict(inputs, x=r["values"])
    assert np.array_equal(r["out"].view(np.uint32), r["via_values"].view(np.uint32)), \
        f"{r['kernel']}: packed input and fp32 input with the same signs give different outputs"
    parity.compare(layer, sub, {"out": r["out"], "acc": r["acc"]}, images=images, workspace=False)
    got = parity.unpack_words(r["bits"], layer.out_c)
    assert np.array_equal(got, (~(r["out"] < 0)).astype(np.uint8)), f"{r['kernel']}: output bits differ"
    assert not parity.unpack_words(r["bits"], None)[..., layer.out_c:].any(), "output bits past out_c are set"
    ph, pw = r["pad"]
    h, w = layer.in_h, layer.in_w
    inner = r["padded"][:, ph:ph + h, pw:pw + w, :]
    mask = np.full(layer.words, 0xFFFFFFFF, np.uint32)
    if layer.in_c % 32:
        mask[-1] = (1 << (layer.in_c % 32)) - 1
    assert np.array_equal(inner, words & mask), f"{layer.name}: repadded bits differ from the masked input"
    halo = r["padded"].copy()
    halo[:, ph:ph + h, pw:pw + w, :] = 0
    assert not halo.any(), f"{layer.name}: halo of the repadded input is not zero"


@pytest.mark.parametrize("generic", [False, True], ids=["fast", "generic"])
@pytest.mark.parametrize("layer", PACKED_LAYERS, ids=[l.name for l in PACKED_LAYERS])
def test_forward_packed(dev, layer, generic):
    """bconv_forward_packed / _bits on random words (tail bits past in_c random
    too): the oracle's result on the +-1 input those bits stand for, and
    bit-identical to bconv_forward on that input."""
    seed = 8600 + PACKED_LAYERS.index(layer)
    inputs = workloads.make_inputs(layer, seed)
    words = workloads.make_packed_input(layer, seed + 50)
    _log(f"packed {layer.name} generic={generic}")
    r = _packed_run(layer, inputs, words, dev, generic=generic)
    _check_packed(layer, inputs, words, r)


PACKED_MEASURED = [i for i, l in enumerate(workloads.LAYERS)
                   if l.type != "binary_weights" and not l.use_beta and l.iscale_dist is None]


@pytest.mark.parametrize("index", PACKED_MEASURED, ids=[workloads.LAYERS[i].name for i in PACKED_MEASURED])
def test_forward_packed_measured_layer(dev, index):
    """Packed input on each measured layer it applies to, at full size, every
    output compared with the oracle on the +-1 input the words stand for."""
    layer = workloads.LAYERS[index]
    inputs = workloads.make_inputs(layer, workloads.layer_seed(index))
    words = workloads.make_packed_input(layer, workloads.layer_seed(index) + 77)
    _log(f"packed layer {layer.name}")
    r = _packed_run(layer, inputs, words, dev)
    _check_packed(layer, inputs, words, r)


def test_packed_chain(dev):
    """Two binary layers on bits alone: the first writes packed output sign bits
    (bconv_forward_bits), the second reads them (bconv_forward_packed_bits and
    bconv_forward_packed).  The second layer's result is the oracle's on the
    +-1 input the first layer's bits stand for."""
    l1 = workloads.Layer("chain_xnor", "xnor", 2, 15, 13, 96, 128, 3, 3, 1, 1, 1, 1,
                         obias_dist=("normal", 0.0, 5.0))
    l2 = workloads.Layer("chain_and_s2", "and", 2, 15, 13, 128, 70, 3, 3, 2, 2, 1, 1)
    l3 = workloads.Layer("chain_fc", "xnor", 2, 8, 7, 70, 10, 8, 7, 1, 1, 0, 0)
    in1, in2, in3 = (workloads.make_inputs(l, 8700 + k) for k, l in enumerate((l1, l2, l3)))
    c1, c2, c3 = (pca.BinaryConvolution.from_layer(l, i) for l, i in ((l1, in1), (l2, in2), (l3, in3)))
    try:
        x = torch.from_numpy(in1["x"]).to(dev)
        b1 = c1.forward_bits(x)
        b2 = c2.forward_packed(b1, bits_out=True)
        out3 = c3.forward_packed(b2)
        out2 = c2.forward_packed(b1)
        torch.cuda.synchronize()
        b1h, b2h = b1.cpu().numpy(), b2.cpu().numpy()
        parity.compare_bits(l1, in1, b1h)
        sub2 = dict(in2, x=parity.values_from_bits(b1h, l2.in_c))
        ref2 = oracle.bconv_layer(l2, sub2)
        bound2 = parity.output_bound(l2, sub2, ref2)
        assert np.all(np.abs(out2.cpu().numpy().astype(np.float64) - ref2["out"]) <= bound2)
        assert np.array_equal(parity.unpack_words(b2h, l2.out_c), (~(out2.cpu().numpy() < 0)).astype(np.uint8))
        parity.compare_bits(l2, sub2, b2h, ref=ref2)
        sub3 = dict(in3, x=parity.values_from_bits(b2h, l3.in_c))
        ref3 = oracle.bconv_layer(l3, sub3)
        bound3 = parity.output_bound(l3, sub3, ref3)
        assert np.all(np.abs(out3.cpu().numpy().astype(np.float64) - ref3["out"]) <= bound3)
    finally:
        for c in (c1, c2, c3):
            c.close()


def test_packed_batch_limit(dev):
    """A batch whose padded bit buffer would reach 2^31 words is an argument
    error, found before any launch (a 1x1 image has 9 padded pixels under a
    3x3 window; input and output stay below 2 GiB).  The pointers are never
    dereferenced: without this check the missing workspace is the error."""
    layer = workloads.Layer("tiny_image", "xnor", 1, 1, 1, 32, 1, 3, 3, 1, 1, 1, 1)
    conv = pca.BinaryConvolution.from_layer(layer, workloads.make_inputs(layer, 8802))
    try:
        n = (1 << 31) // 9 + 1
        for fn in (pca.bconv_forward_packed, pca.bconv_forward_packed_bits):
            with pytest.raises(pca.BconvError) as e:
                fn(conv.handle, None, n, 0x10000000000, 0x20000000000, None, 0)
            assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT, pca.bconv_last_error()
            assert "2^31 words" in pca.bconv_last_error()
    finally:
        conv.close()


def test_packed_input_unsupported(dev):
    """Handles that read the full-precision input refuse packed input with
    BCONV_ERR_UNSUPPORTED, before any check of n or pointers."""
    base = workloads.Layer("unsup", "xnor", 1, 6, 6, 64, 32, 3, 3, 1, 1, 1, 1)
    cases = [(base.with_(use_beta=True), False), (base.with_(type="binary_weights"), False),
             (base.with_(iscale_dist=("uniform", 0.5, 1.5)), False),
             (base.with_(ibias_dist=("normal", 0.0, 0.2)), False), (base, True), (base.with_(type="and"), True)]
    for layer, int8 in cases:
        inputs = workloads.make_inputs(layer, 8800)
        conv = pca.BinaryConvolution.from_layer(layer, inputs, int8_mfma=int8)
        try:
            for n in (1, 0):
                for bits_out in (False, True):
                    fn = pca.bconv_forward_packed_bits if bits_out else pca.bconv_forward_packed
                    with pytest.raises(pca.BconvError) as e:
                        fn(conv.handle, None, n, None, None, None, 0)
                    assert e.value.status == pca.BCONV_ERR_UNSUPPORTED, (layer, int8)
        finally:
            conv.close()
    # a supported handle: n == 0 is a no-op, NULL pointers and overlap are argument errors
    inputs = workloads.make_inputs(base, 8801)
    conv = pca.BinaryConvolution.from_layer(base, inputs)
    try:
        pca.bconv_forward_packed(conv.handle, None, 0, None, None, None, 0)
        ws = conv.workspace(1, dev)
        buf = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
        for args in ((None, buf), (buf, None), (buf, buf[1:])):
            with pytest.raises(pca.BconvError) as e:
                pca.bconv_forward_packed(conv.handle, None, 1, args[0], args[1], ws, ws.numel())
            assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward_packed(conv.handle, None, 1, buf, buf[4096:], ws, 16)
        assert e.value.status == pca.BCONV_ERR_WORKSPACE
    finally:
        conv.close()


# ------------------------------------------------------------ robustness

def test_repeat_is_bit_identical(dev):
    layer = workloads.BENCH_LAYER.with_(n=2)
    inputs = workloads.make_inputs(layer, 3)
    a = parity.run_gpu(layer, inputs, dev)
    b = parity.run_gpu(layer, inputs, dev)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    assert np.array_equal(a["beta"].view(np.uint32), b["beta"].view(np.uint32))


REUSE_LAYERS = [workloads.BENCH_LAYER.with_(n=2), workloads.LAYERS[2].with_(n=2),
                 workloads.LAYERS[3].with_(n=2), workloads.LAYERS[4].with_(n=5)]


@pytest.mark.parametrize("layer", REUSE_LAYERS, ids=[l.name for l in REUSE_LAYERS])
def test_new_input_reuses_workspace(dev, layer):
    """One handle and one workspace, two different inputs in turn (forward,
    forward_accum and the event-bracketed forward): every call matches the
    oracle on its own input, so nothing of an earlier call's packed input, A
    map or beta survives into a later one."""
    inputs = [workloads.make_inputs(layer, 21)]
    inputs.append(dict(inputs[0], x=workloads.make_inputs(layer, 22)["x"]))
    refs = [oracle.bconv_layer(layer, inp) for inp in inputs]
    conv = pca.BinaryConvolution.from_layer(layer, inputs[0])
    try:
        n = layer.n
        ws = conv.workspace(n, dev)
        xs = [torch.from_numpy(inp["x"]).to(dev) for inp in inputs]
        shape = (n, conv.out_h, conv.out_w, conv.out_c)
        acc_dtype = torch.float32 if layer.type == "binary_weights" else torch.int32
        begin, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        begin.record(), end.record()
        for rnd in range(3):
            for k in (0, 1):
                out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
                acc = torch.zeros(shape, dtype=acc_dtype, device=dev)
                conv.forward_accum(xs[k], acc, ws)
                if rnd == 1:
                    pca.bconv_forward_profiled(conv.handle, torch.cuda.current_stream().cuda_stream, n, xs[k], out,
                                               ws, ws.numel(), begin.cuda_event, end.cuda_event)
                else:
                    conv.forward(xs[k], out, ws)
                torch.cuda.synchronize()
                _log(f"reuse {layer.name} round {rnd} input {k}")
                parity.compare(layer, inputs[k], {"out": out.cpu().numpy(), "acc": acc.cpu().numpy()}, ref=refs[k],
                               workspace=False)
    finally:
        conv.close()


def test_graph_capture_replays(dev):
    """The forward entry points only launch kernels (no allocation, memset or
    synchronisation inside), so a chain of them records into a HIP graph:
    fp32 output, packed sign bits, and a next layer fed those bits.  Every
    replay, after the outputs and workspaces are poisoned eagerly between
    replays, gives the eager results bit for bit."""
    l1 = workloads.BENCH_LAYER.with_(n=2)
    l2 = workloads.Layer("graph_and_s2", "and", 2, 56, 56, 128, 64, 3, 3, 2, 2, 1, 1)
    in1, in2 = workloads.make_inputs(l1, 8900), workloads.make_inputs(l2, 8901)
    c1, c2 = pca.BinaryConvolution.from_layer(l1, in1), pca.BinaryConvolution.from_layer(l2, in2)
    try:
        x = torch.from_numpy(in1["x"]).to(dev)
        ws1, ws2 = c1.workspace(2, dev), c2.workspace(2, dev)
        out1 = torch.empty((2, c1.out_h, c1.out_w, c1.out_c), dtype=torch.float32, device=dev)
        bits1 = torch.empty((2, c1.out_h, c1.out_w, c1.out_words()), dtype=torch.int32, device=dev)
        out2 = torch.empty((2, c2.out_h, c2.out_w, c2.out_c), dtype=torch.float32, device=dev)

        def chain():
            c1.forward(x, out1, ws1)
            c1.forward_bits(x, bits1, ws1)
            c2.forward_packed(bits1, out2, ws2)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            chain()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        want = [t.clone() for t in (out1, bits1, out2)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            chain()
        torch.cuda.synchronize()
        for replay in range(3):
            out1.fill_(float("nan"))
            bits1.fill_(-1)
            out2.fill_(float("nan"))
            ws1.fill_(0xA5)
            ws2.fill_(0x5A)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            _log(f"graph replay {replay}")
            for got, ref in zip((out1, bits1, out2), want):
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"replay {replay} differs"
        del graph
    finally:
        c1.close()
        c2.close()


def test_two_streams_share_a_handle(dev):
    layer = workloads.LAYERS[2].with_(n=4)
    inputs = workloads.make_inputs(layer, 4)
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    try:
        x = torch.from_numpy(inputs["x"]).to(dev)
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        ws1, ws2 = conv.workspace(4, dev), conv.workspace(4, dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            o1 = conv.forward(x, workspace=ws1, stream=s1)
        with torch.cuda.stream(s2):
            o2 = conv.forward(x, workspace=ws2, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    finally:
        conv.close()


def test_temporaries_on_a_side_stream(dev):
    """forward*(stream=s) with s not the current stream and no workspace or
    output given: the wrapper allocates them on s, so blocks the current
    stream allocates and overwrites right after the launch are never the ones
    the kernels still use.  Every call matches the oracle."""
    layer = workloads.BENCH_LAYER.with_(n=4)
    inputs = workloads.make_inputs(layer, 31)
    ref = oracle.bconv_layer(layer, inputs)
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    try:
        x = torch.from_numpy(inputs["x"]).to(dev)
        side = torch.cuda.Stream()
        nbytes = conv.workspace_bytes(4)
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        outs, accs = [], []
        for _ in range(4):
            outs.append(conv.forward(x, stream=side))
            accs.append(conv.forward_accum(x, stream=side))
            # allocations of the freed temporaries' sizes on the current
            # stream, overwritten at once
            for _ in range(3):
                torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(0x5A)
                torch.empty(outs[-1].shape, dtype=torch.float32, device=dev).fill_(float("nan"))
        side.synchronize()
        torch.cuda.synchronize()
        for out, acc in zip(outs, accs):
            parity.compare(layer, inputs, {"out": out.cpu().numpy(), "acc": acc.cpu().numpy()}, ref=ref,
                           workspace=False)
    finally:
        conv.close()


# ------------------------------------------------------------ maximum sizes

MAX_CHANNELS = 1 << 20   # the C ABI's in_c limit
MAX_EXTENT = 1 << 16     # the C ABI's image extent limit
MAX_CASES = [
    # in_c * kh * kw = 2^24, the largest window the C ABI accepts: FC shape
    # (matrix route) and a conv shape with four outputs (shape-generic kernel)
    workloads.Layer("max_window_fc_xnor", "xnor", 1, 4, 4, MAX_CHANNELS, 3, 4, 4),
    workloads.Layer("max_window_fc_and", "and", 1, 4, 4, MAX_CHANNELS, 3, 4, 4, use_beta=True),
    workloads.Layer("max_window_fc_binary_weights", "binary_weights", 1, 4, 4, MAX_CHANNELS, 3, 4, 4),
    workloads.Layer("max_window_conv_xnor", "xnor", 1, 5, 5, MAX_CHANNELS, 2, 4, 4, use_beta=True),
    # the largest image extent, in either direction
    workloads.Layer("max_width", "xnor", 1, 1, MAX_EXTENT, 32, 70, 3, 3, 1, 1, 1, 1, use_beta=True),
    workloads.Layer("max_height_and", "and", 1, MAX_EXTENT, 1, 40, 5, 3, 3, 2, 1, 1, 1),
]


@pytest.mark.parametrize("layer", MAX_CASES, ids=[l.name for l in MAX_CASES])
def test_maximum_sizes(dev, layer):
    """The C ABI's largest window (2^24 bits: window sums exact in int32 and
    fp32) and largest image extents, against the oracle."""
    inputs = workloads.make_inputs(layer, 4400 + MAX_CASES.index(layer))
    _log(f"max {layer.name}")
    got = parity.run_gpu(layer, inputs, dev)
    parity.compare(layer, inputs, got)


MAX_PACKED = [l for l in MAX_CASES if l.type != "binary_weights" and not l.use_beta]


@pytest.mark.parametrize("layer", MAX_PACKED, ids=[l.name for l in MAX_PACKED])
def test_maximum_sizes_packed(dev, layer):
    """Packed sign-bit input at the largest window and image extent."""
    seed = 4450 + MAX_PACKED.index(layer)
    inputs = workloads.make_inputs(layer, seed)
    words = workloads.make_packed_input(layer, seed + 1)
    _log(f"max packed {layer.name}")
    r = _packed_run(layer, inputs, words, dev)
    _check_packed(layer, inputs, words, r)


def test_maximum_window_is_exact(dev):
    """All 2^24 products of the largest window agree: the XNOR and AND sums
    reach exactly 2^24 (the top of the exact fp32 integers) and the output is
    2^24 * scale."""
    for form in ("xnor", "and"):
        layer = workloads.Layer("max_window_ones", form, 1, 4, 4, MAX_CHANNELS, 2, 4, 4,
                                oscale_dist=None, obias_dist=None, scale_value=0.5)
        inputs = workloads.make_inputs(layer, 1)
        inputs["x"] = np.abs(inputs["x"]) + 0.5
        inputs["weight_bits"][:] = 0xFFFFFFFF
        got = parity.run_gpu(layer, inputs, dev)
        assert np.all(got["acc"] == (1 << 24)), form
        assert np.all(got["out"] == np.float32(1 << 23)), form


def test_calibration_kernel(dev):
    """The popcount calibration kernel does the work its header states: each
    thread's word is sum_k iters * popcount(x[k % 4] ^ w_k), computed here with
    Python integers."""
    blocks, iters, seed = 6, 37, 12345
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
    pca.bconv_calibrate_popcount(torch.cuda.current_stream().cuda_stream, blocks, iters, seed, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    m = 0xFFFFFFFF
    x0 = (seed * 0x9E3779B1) & m
    xs = [x0, x0 ^ 0x85EBCA77, (x0 + 0xC2B2AE3D) & m, x0 ^ 0x27D4EB2F]
    for t in range(blocks * 256):
        want = 0
        for k in range(8):
            w = ((t * 2654435761) & m) ^ ((k * 0x9E3779B9) & m)
            want += iters * bin(xs[k % 4] ^ w).count("1")
        assert int(got[t]) == want & m, t


def test_argument_errors(dev):
    layer = workloads.BENCH_LAYER.with_(n=2)
    inputs = workloads.make_inputs(layer, 5)
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    try:
        x = torch.from_numpy(inputs["x"]).to(dev)
        out = torch.empty((2, 56, 56, 128), device=dev)
        need = conv.workspace_bytes(2)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        s = torch.cuda.current_stream().cuda_stream
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward(conv.handle, s, 2, x, out, ws, need - 1)
        assert e.value.status == pca.BCONV_ERR_WORKSPACE
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward(conv.handle, s, 2, x, x, ws, need)
        assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward(conv.handle, s, -1, x, out, ws, need)
        assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT
        out.fill_(3.0)
        pca.bconv_forward(conv.handle, s, 0, x, out, None, 0)  # empty batch: no-op
        torch.cuda.synchronize()
        assert bool((out == 3.0).all())
    finally:
        conv.close()


def test_fc_entry_point_matches_conv(dev):
    """bconv_create_fc builds the same layer as bconv_create with kernel =
    source size; outputs are identical."""
    layer = workloads.LAYERS[4].with_(n=8, out_c=300)
    inputs = workloads.make_inputs(layer, 12)
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    h = pca.bconv_create_fc(7, 7, 512, 300, pca.BCONV_NEURON_NONE, 1.0, inputs["weight_bits"],
                            inputs["output_scale"], inputs["output_bias"], None, None, pca.BCONV_XNOR,
                            pca.BCONV_FLAG_NONE)
    try:
        x = torch.from_numpy(inputs["x"]).to(dev)
        a = conv.forward(x)
        b = torch.empty_like(a)
        ws = torch.empty(max(1, pca.bconv_workspace_size(h, 8)), dtype=torch.uint8, device=dev)
        pca.bconv_forward(h, torch.cuda.current_stream().cuda_stream, 8, x, b, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert pca.bconv_get_info(h) == (512, 300, 1, 1)
    finally:
        pca.bconv_destroy(h)
        conv.close()


# ------------------------------------- FC shapes whose window is not 4k words

def _fc_tail_layers():
    """Fully connected shapes (kernel = source size, MPSCNNFullyConnected
    conditions) whose K = kh*kw*ceil(in_c/32) words leave 1, 2 or 3 words in
    the matrix kernel's last 4-word step, at batches that are not a multiple of
    its 16-row groups; XNOR and AND, plain and with beta + input affine."""
    base = workloads.Layer("fc_tail", "xnor", 17, 1, 1, 64, 70, 1, 1)
    geoms = [
        dict(in_h=1, in_w=1, in_c=64, out_c=70),                  # K = 2
        dict(in_h=3, in_w=3, in_c=32, out_c=65, n=17),            # K = 9
        dict(in_h=7, in_w=7, in_c=20, out_c=33, n=5),             # K = 49
        dict(in_h=5, in_w=5, in_c=40, out_c=9, n=33),             # K = 50
        dict(in_h=3, in_w=3, in_c=96, out_c=40, n=20),            # K = 27
        dict(in_h=1, in_w=1, in_c=96, out_c=130, n=1),            # K = 3
        dict(in_h=1, in_w=1, in_c=32, out_c=64, n=16),            # K = 1
        dict(in_h=2, in_w=3, in_c=7, out_c=200, n=18),            # K = 6, 7 channels
    ]
    out = []
    for gi, g in enumerate(geoms):
        assert (g["in_h"] * g["in_w"] * ((g["in_c"] + 31) // 32)) % 4 != 0
        for form in ("xnor", "and"):
            kw = dict(g, kernel_h=g["in_h"], kernel_w=g["in_w"], type=form, name=f"fc_tail{gi}_{form}")
            out.append(base.with_(**kw))
            if gi % 2 == 0:
                out.append(base.with_(**dict(kw, name=kw["name"] + "_beta", use_beta=True, neuron="relu",
                                             iscale_dist=("uniform", 0.5, 1.5),
                                             ibias_dist=("normal", 0.0, 0.2))))
    return out


FC_TAIL = _fc_tail_layers()


@pytest.mark.parametrize("layer", FC_TAIL, ids=[l.name for l in FC_TAIL])
def test_fc_partial_k_step(dev, layer):
    """The matrix kernel's partial last K step: fp32 output and window sums
    (matrix route and generic kernel), sign-bit output, and (without beta /
    affine) packed input; every output compared with the oracle."""
    assert layer.is_fc
    inputs = workloads.make_inputs(layer, 9100 + FC_TAIL.index(layer))
    _log(f"fc tail {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev)
    assert got["main_kernel"].startswith("bgemm_kernel"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)
    parity.compare(layer, inputs, parity.run_gpu(layer, inputs, dev, generic=True), ref=ref)
    words, out, kernel = _run_bits(layer, inputs, dev)
    assert np.array_equal(parity.unpack_words(words, layer.out_c), (~(out < 0)).astype(np.uint8)), kernel
    parity.compare_bits(layer, inputs, words, ref=ref)
    if not layer.use_beta:
        pw = workloads.make_packed_input(layer, 9200 + FC_TAIL.index(layer))
        _check_packed(layer, inputs, pw, _packed_run(layer, inputs, pw, dev))


# ------------------------------------- FC product on the fp4 matrix cores

def _fc_f4_layers():
    """Fully connected shapes whose K = kh*kw*ceil(in_c/32) words is a multiple
    of 4 (the fp4 matrix-core route): a lone partial 16-word step, full steps
    only, full steps plus a partial one, batches that leave a ragged 64-row
    block or a single row, channel counts that leave ragged 16- and 64-channel
    tiles, and zero bits past Cin inside a pixel's last word; XNOR and AND,
    plain and with beta + input affine + ReLU."""
    base = workloads.Layer("fc_f4", "xnor", 17, 1, 1, 128, 70, 1, 1)
    geoms = [
        dict(in_h=1, in_w=1, in_c=128, out_c=70, n=17),    # K = 4: one partial step
        dict(in_h=3, in_w=3, in_c=128, out_c=65, n=65),    # K = 36: 2 steps + 1 word group
        dict(in_h=2, in_w=2, in_c=256, out_c=130, n=64),   # K = 32: full steps only
        dict(in_h=7, in_w=7, in_c=512, out_c=100, n=130),  # K = 784: 49 steps, 3 row blocks
        dict(in_h=4, in_w=4, in_c=100, out_c=1, n=3),      # 4 bits of the last word valid
        dict(in_h=1, in_w=2, in_c=255, out_c=64, n=1),     # one row
        dict(in_h=5, in_w=5, in_c=128, out_c=200, n=40),   # K = 100: 6 steps + 1 word group
        dict(in_h=2, in_w=2, in_c=256, out_c=70, n=20, neuron="sigmoid"),
    ]
    out = []
    for gi, g in enumerate(geoms):
        assert (g["in_h"] * g["in_w"] * ((g["in_c"] + 31) // 32)) % 4 == 0
        for form in ("xnor", "and"):
            kw = dict(g, kernel_h=g["in_h"], kernel_w=g["in_w"], type=form, name=f"fc_f4_{gi}_{form}")
            out.append(base.with_(**kw))
            if gi % 2 == 1:
                out.append(base.with_(**dict(kw, name=kw["name"] + "_beta", use_beta=True, neuron="relu",
                                             iscale_dist=("uniform", 0.5, 1.5),
                                             ibias_dist=("normal", 0.0, 0.2))))
    return out


FC_F4 = _fc_f4_layers()


@pytest.mark.parametrize("layer", FC_F4, ids=[l.name for l in FC_F4])
def test_fc_fp4_route(dev, layer):
    """The fully connected product on the fp4 matrix cores
    (BCONV_FLAG_FP4_MFMA): fp32 output and window sums compared with the
    oracle on every output; window sums and fp32 outputs identical to the VALU
    popcount GEMM's; sign-bit output; and (without beta / affine) packed
    input."""
    assert layer.is_fc
    seed = 9400 + FC_F4.index(layer)
    inputs = workloads.make_inputs(layer, seed)
    _log(f"fc fp4 {layer} seed {seed}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev, fp4_mfma=True)
    assert got["main_kernel"].startswith("bgemm_f4_kernel"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)
    pop = parity.run_gpu(layer, inputs, dev)
    assert pop["main_kernel"].startswith("bgemm_kernel"), pop["main_kernel"]
    assert np.array_equal(got["acc"], pop["acc"])
    assert np.array_equal(got["out"].view(np.uint32), pop["out"].view(np.uint32))
    words, out, kernel = _run_bits(layer, inputs, dev, fp4=True)
    assert kernel.startswith("bgemm_f4_kernel"), kernel
    assert np.array_equal(parity.unpack_words(words, layer.out_c), (~(out < 0)).astype(np.uint8)), kernel
    assert not parity.unpack_words(words, None)[..., layer.out_c:].any(), "output bits past out_c are set"
    parity.compare_bits(layer, inputs, words, ref=ref)
    if not layer.use_beta:
        pw = workloads.make_packed_input(layer, 9500 + FC_F4.index(layer))
        r = _packed_run(layer, inputs, pw, dev, fp4=True)
        assert r["kernel"].startswith("bgemm_f4_kernel"), r["kernel"]
        _check_packed(layer, inputs, pw, r)


def test_fc_fp4_measured_layer_full(dev):
    """The measured fully connected layer (256 x 7x7x512 -> 4096) on the fp4
    matrix cores at full size, every output compared with the oracle."""
    index = next(i for i, l in enumerate(workloads.LAYERS) if l.is_fc)
    layer = workloads.LAYERS[index]
    inputs, ref = measured_reference(index)
    got = parity.run_gpu(layer, inputs, dev, fp4_mfma=True)
    assert got["main_kernel"].startswith("bgemm_f4_kernel"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)


def _conv_f4_layers():
    """Convolutions the fp4 matrix-core comparison path takes (a pixel of a
    multiple of 4 words): the XNOR + beta + affine + ReLU form, AND, several
    channel tiles, 5x5 and 7x7 windows (196 word groups), stride 2 without
    padding, a 1x1 window, an even window with the centred padding, and
    channels that leave tail bits in a pixel's last word."""
    base = workloads.Layer("conv_f4", "xnor", 2, 9, 10, 128, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(use_beta=True, neuron="relu", iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2)),
        dict(type="and"),
        dict(),
        dict(n=1, in_h=12, in_w=11, in_c=256, out_c=130, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2, type="and"),
        dict(n=1, in_h=12, in_w=11, in_c=256, out_c=130, kernel_h=5, kernel_w=5, pad_h=2, pad_w=2),
        dict(n=3, in_h=13, in_w=9, out_c=64, stride_h=2, stride_w=2, pad_h=0, pad_w=0),
        dict(n=2, in_h=8, in_w=8, in_c=512, out_c=33, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0),
        dict(n=2, in_h=7, in_w=8, out_c=20, kernel_h=2, kernel_w=2, pad_h=1, pad_w=1, pad_bottom=0, pad_right=0,
             use_beta=True),
        dict(in_c=100, out_c=17),
        dict(in_c=100, out_c=17, type="and"),
        dict(n=1, in_h=10, in_w=10, in_c=512, out_c=16, kernel_h=7, kernel_w=7, pad_h=3, pad_w=3),
        dict(neuron="tanh", neuron_a=1.5, neuron_b=0.5, use_beta=True),   # neurons outside the inline pair
        dict(neuron="elu", neuron_a=0.7, type="and"),
    ]
    return [base.with_(**dict(g, name=f"conv_f4_{i}")) for i, g in enumerate(geoms)]


CONV_F4 = _conv_f4_layers()


@pytest.mark.parametrize("layer", CONV_F4, ids=[l.name for l in CONV_F4])
def test_conv_fp4_route(dev, layer):
    """Convolutions on the fp4 matrix cores (BCONV_FLAG_FP4_MFMA): every output
    compared with the oracle; window sums identical to the popcount path's and
    fp32 outputs to the generic kernel's (same beta summation order); sign-bit
    output; and (without beta / affine) packed input."""
    assert not layer.is_fc
    seed = 9700 + CONV_F4.index(layer)
    inputs = workloads.make_inputs(layer, seed)
    _log(f"conv fp4 {layer} seed {seed}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev, fp4_mfma=True)
    assert got["main_kernel"].startswith("xconv_f4_kernel"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)
    pop = parity.run_gpu(layer, inputs, dev)
    assert np.array_equal(got["acc"], pop["acc"]), pop["main_kernel"]
    gen = parity.run_gpu(layer, inputs, dev, generic=True)
    assert np.array_equal(got["out"].view(np.uint32), gen["out"].view(np.uint32))
    words, out, kernel = _run_bits(layer, inputs, dev, fp4=True)
    assert kernel.startswith("xconv_f4_kernel"), kernel
    assert np.array_equal(parity.unpack_words(words, layer.out_c), (~(out < 0)).astype(np.uint8)), kernel
    assert not parity.unpack_words(words, None)[..., layer.out_c:].any(), "output bits past out_c are set"
    parity.compare_bits(layer, inputs, words, ref=ref)
    if not layer.use_beta and layer.iscale_dist is None:
        pw = workloads.make_packed_input(layer, 9800 + CONV_F4.index(layer))
        r = _packed_run(layer, inputs, pw, dev, fp4=True)
        assert r["kernel"].startswith("xconv_f4_kernel"), r["kernel"]
        _check_packed(layer, inputs, pw, r)


@pytest.mark.parametrize("index", [1, 2], ids=["bench_layer", "and_layer"])
def test_conv_fp4_measured_layer_full(dev, index):
    """The measured XNOR + beta and AND convolutions on the fp4 matrix cores at
    full size, every output compared with the oracle."""
    layer = workloads.LAYERS[index]
    inputs, ref = measured_reference(index)
    got = parity.run_gpu(layer, inputs, dev, fp4_mfma=True)
    assert got["main_kernel"].startswith("xconv_f4_kernel"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)


def test_fc_fp4_unsupported_shapes(dev):
    """BCONV_FLAG_FP4_MFMA on a convolution whose pixel is not a multiple of 4
    words, or on a fully connected window that is not, is refused at
    creation."""
    for layer in (workloads.LAYERS[0], FC_TAIL[0]):
        inputs = workloads.make_inputs(layer, 9600)
        with pytest.raises(pca.BconvError) as e:
            pca.BinaryConvolution.from_layer(layer, inputs, fp4_mfma=True)
        assert e.value.status == pca.BCONV_ERR_UNSUPPORTED, layer.name


@pytest.mark.parametrize("layer", FC_TAIL[:4], ids=[l.name for l in FC_TAIL[:4]])
def test_fc_partial_k_step_int8(dev, layer):
    """The same shapes through the int8 matrix-core comparison path."""
    inputs = workloads.make_inputs(layer, 9100 + FC_TAIL.index(layer))
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev, int8_mfma=True)
    assert got["main_kernel"] == "i8mma_kernel"
    parity.compare(layer, inputs, got, ref=ref)


# --------------------------------------- single-launch small-layer kernel

def _small_layers():
    """Small conv layers (1x1 and 3x3 windows, 1 to 4 words per pixel) that
    the library runs with its single-launch kernel: ragged word and channel
    tiles, strides, no / centred / one-sided padding, a window with every tap
    but one in the padding, Cin = 1; XNOR and AND, plain and with the input
    affine and an activation, and with the scalar output scale."""
    base = workloads.Layer("small", "xnor", 2, 9, 11, 64, 70, 3, 3, 1, 1, 1, 1)
    geoms = [
        dict(in_c=64, out_c=70),
        dict(n=3, in_c=27, out_c=40),
        dict(in_c=100, out_c=64, stride_h=2, stride_w=2),
        dict(in_c=70, out_c=130, pad_h=0, pad_w=0),
        dict(in_c=96, out_c=33, pad_h=1, pad_w=1, pad_bottom=0, pad_right=0),
        dict(in_c=33, out_c=9, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0),
        dict(in_c=128, out_c=64, kernel_h=1, kernel_w=1, pad_h=0, pad_w=0, stride_h=2, stride_w=3),
        dict(n=1, in_h=1, in_w=1, in_c=64, out_c=8),
        dict(in_c=1, out_c=3),
    ]
    out = []
    for gi, g in enumerate(geoms):
        for form in ("xnor", "and"):
            for variant in range(3):
                kw = dict(g, type=form, name=f"small{gi}_{form}_v{variant}")
                if variant == 1:
                    kw.update(neuron="relu", iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2))
                elif variant == 2:
                    kw.update(oscale_dist=None, obias_dist=None, scale_value=0.75, neuron="sigmoid")
                out.append(base.with_(**kw))
    return out


SMALL_LAYERS = _small_layers()


@pytest.mark.parametrize("layer", SMALL_LAYERS, ids=[l.name for l in SMALL_LAYERS])
def test_small_layer_single_launch(dev, layer):
    """The single-launch kernel: window sums bit-exact and outputs within the
    parity bounds of the oracle, bit-identical to the two-kernel path (pack,
    then the convolution) on the same handle inputs, and sign-bit output."""
    inputs = workloads.make_inputs(layer, 9400 + SMALL_LAYERS.index(layer))
    _log(f"small {layer}")
    ref = oracle.bconv_layer(layer, inputs)
    got = parity.run_gpu(layer, inputs, dev, small_fused=True)
    assert got["main_kernel"].startswith("xconv_small"), got["main_kernel"]
    parity.compare(layer, inputs, got, ref=ref)
    two = parity.run_gpu(layer, inputs, dev, small_fused=False)
    assert not two["main_kernel"].startswith("xconv_small")
    assert np.array_equal(got["acc"], two["acc"])
    assert np.array_equal(got["out"].view(np.uint32), two["out"].view(np.uint32))
    with parity.force_generic(False, small_fused=True):
        words, out, kernel = _run_bits(layer, inputs, dev)
    assert kernel.startswith("xconv_small")
    assert np.array_equal(parity.unpack_words(words, layer.out_c), (~(out < 0)).astype(np.uint8))
    parity.compare_bits(layer, inputs, words, ref=ref)


def test_small_route_limits(dev):
    """Beta layers, the fully connected shape, 5x5 windows, more than 128
    input channels and large layers keep the two-kernel path."""
    base = workloads.LAYERS[0]
    assert base.name.startswith("xnor_conv_b1_16x16")
    cases = {
        "default": (base, True),
        "beta": (base.with_(use_beta=True), False),
        "fc": (base.with_(kernel_h=16, kernel_w=16, pad_h=0, pad_w=0), False),
        "k5": (base.with_(kernel_h=5, kernel_w=5, pad_h=2, pad_w=2), False),
        "c160": (base.with_(in_c=160), False),
        "large": (workloads.LAYERS[2], False),
    }
    for name, (layer, small) in cases.items():
        inputs = workloads.make_inputs(layer, 31, n=1)
        with parity.force_generic(False, small_fused=True):
            conv = pca.BinaryConvolution.from_layer(layer, inputs)
        try:
            kernel = conv.main_kernel(layer.n)
            assert kernel.startswith("xconv_small") == small, (name, kernel)
        finally:
            conv.close()
