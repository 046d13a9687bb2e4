"""The packed-bit CPU baseline (``oracle/packed_cpu.c``, a throughput
reference point for the benchmark) against the oracle: window sums bit-exact,
outputs within the fp32 bound."""

import numpy as np
import pytest

import oracle
import parity
from popcount_convolution_amd import workloads

BASE = workloads.Layer("packed", "xnor", 2, 9, 10, 64, 20, 3, 3, 1, 1, 1, 1)
CASES = [
    BASE.with_(name="packed_xnor_beta_affine_relu", use_beta=True, neuron="relu", in_c=100,
               iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2)),
    BASE.with_(name="packed_and", type="and", in_c=70, x_dist=("normal", 0.2, 1.0)),
    BASE.with_(name="packed_xnor_s2_asym", stride_h=2, stride_w=2, pad_h=0, pad_w=1, pad_bottom=2, pad_right=0),
    BASE.with_(name="packed_xnor_k4_centred", kernel_h=4, kernel_w=4, pad_h=2, pad_w=2, pad_bottom=1, pad_right=1,
               in_c=33),
    BASE.with_(name="packed_fc", n=3, in_h=4, in_w=5, in_c=40, out_c=12, kernel_h=4, kernel_w=5, pad_h=0, pad_w=0),
    BASE.with_(name="packed_and_beta_valid_taps", type="and", use_beta=True, beta_valid_taps=True, kernel_h=4,
               kernel_w=4, pad_h=2, pad_w=2, pad_bottom=1, pad_right=1, neuron="relu"),
    workloads.LAYERS[0],
]


@pytest.mark.parametrize("layer", CASES, ids=[c.name for c in CASES])
def test_packed_cpu_matches_oracle(layer):
    inputs = workloads.make_inputs(layer, 700 + CASES.index(layer))
    ref = oracle.bconv_layer(layer, inputs)
    got = oracle.packed_bconv(layer, inputs, threads=2)
    assert np.array_equal(got["acc"], ref["acc"])
    err = np.abs(got["out"].astype(np.float64) - ref["out"])
    assert np.all(err <= parity.output_bound(layer, inputs, ref))


def test_packed_cpu_rejects_binary_weights():
    layer = BASE.with_(type="binary_weights")
    with pytest.raises(ValueError):
        oracle.packed_bconv(layer, workloads.make_inputs(layer, 1))
