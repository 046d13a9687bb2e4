"""Seeded synthetic workloads for binary convolution.

This module only draws random inputs and describes layer shapes. It holds none
of the method's arithmetic (no binarisation, no packing, no convolution): the
same host arrays feed both the HIP path and the CPU oracle.

Shapes follow the five layers the library is measured on (NHWC fp32 input,
weight bits as uint32 words ``[Cout][kh][kw][ceil(Cin/32)]``, channel ``c`` in
bit ``c % 32`` of word ``c // 32``).  Distributions:

* ``("normal", mu, sigma)``  -> ``mu + sigma * randn``
* ``("uniform", a, b)``      -> ``a + (b - a) * rand``

Weight words are uniform 32-bit integers, i.e. i.i.d. Bernoulli(0.5) bits;
bits at channel positions >= Cin in the last word are random as well, so the
consumers' tail masking is exercised.

Draw order with one ``torch.Generator`` seeded per workload: x, weight words,
output scale, output bias, input scale, input bias (absent terms draw nothing).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

TYPES = ("binary_weights", "xnor", "and")
NEURONS = ("none", "relu", "leaky_relu", "linear", "sigmoid", "hard_sigmoid", "tanh", "absolute", "softplus",
           "softsign", "elu", "clamp")


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    type: str
    n: int
    in_h: int
    in_w: int
    in_c: int
    out_c: int
    kernel_h: int
    kernel_w: int
    stride_h: int = 1
    stride_w: int = 1
    pad_h: int = 0
    pad_w: int = 0
    use_beta: bool = False
    neuron: str = "none"
    x_dist: tuple = ("normal", 0.0, 1.0)
    oscale_dist: Optional[tuple] = ("uniform", 0.5, 1.5)
    obias_dist: Optional[tuple] = ("normal", 0.0, 0.1)
    iscale_dist: Optional[tuple] = None
    ibias_dist: Optional[tuple] = None
    scale_value: float = 1.0
    # trailing (bottom / right) zero padding; None = the leading one
    pad_bottom: Optional[int] = None
    pad_right: Optional[int] = None
    # activation parameters (see the neuron list of the C header)
    neuron_a: float = 0.0
    neuron_b: float = 0.0
    # beta divides by the window's in-image taps instead of kh*kw
    beta_valid_taps: bool = False

    @property
    def pad_h_end(self) -> int:
        return self.pad_h if self.pad_bottom is None else self.pad_bottom

    @property
    def pad_w_end(self) -> int:
        return self.pad_w if self.pad_right is None else self.pad_right

    @property
    def out_h(self) -> int:
        return (self.in_h + self.pad_h + self.pad_h_end - self.kernel_h) // self.stride_h + 1

    @property
    def out_w(self) -> int:
        return (self.in_w + self.pad_w + self.pad_w_end - self.kernel_w) // self.stride_w + 1

    @property
    def words(self) -> int:
        return (self.in_c + 31) // 32

    @property
    def is_fc(self) -> bool:
        return (self.kernel_h == self.in_h and self.kernel_w == self.in_w
                and self.stride_h == 1 and self.stride_w == 1
                and self.pad_h == 0 and self.pad_w == 0 and self.pad_h_end == 0 and self.pad_w_end == 0)

    def nominal_macs(self, n: Optional[int] = None) -> int:
        """N*Ho*Wo*Cout*kh*kw*Cin: padded taps counted (bit-MACs, or fp32 MACs
        for binary_weights)."""
        n = self.n if n is None else n
        return (n * self.out_h * self.out_w * self.out_c
                * self.kernel_h * self.kernel_w * self.in_c)

    def with_(self, **kw) -> "Layer":
        return dataclasses.replace(self, **kw)


# The five measured layers.
LAYERS = (
    Layer("xnor_conv_b1_16x16_c64_o64_k3", "xnor", 1, 16, 16, 64, 64, 3, 3, 1, 1, 1, 1),
    Layer("xnor_beta_conv_b8_56x56_c128_o128_k3", "xnor", 8, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1,
          use_beta=True, neuron="relu",
          iscale_dist=("uniform", 0.5, 1.5), ibias_dist=("normal", 0.0, 0.2)),
    Layer("and_conv_b32_28x28_c256_o256_k3", "and", 32, 28, 28, 256, 256, 3, 3, 1, 1, 1, 1,
          x_dist=("normal", 0.2, 1.0)),
    Layer("binary_weights_conv_b16_56x56_c64_o128_k3_s2", "binary_weights", 16, 56, 56, 64, 128,
          3, 3, 2, 2, 1, 1),
    Layer("xnor_fc_b256_7x7x512_o4096", "xnor", 256, 7, 7, 512, 4096, 7, 7, 1, 1, 0, 0),
)

# The XNOR + beta convolution the geometry sweep varies, and the largest
# layer, the fully connected one, which the benchmark's headline quotes.
BENCH_LAYER = LAYERS[1]
HEADLINE_LAYER = LAYERS[4]


def _draw(gen: torch.Generator, dist: tuple, shape) -> np.ndarray:
    kind, a, b = dist
    if kind == "normal":
        t = a + b * torch.randn(shape, generator=gen, dtype=torch.float32)
    elif kind == "uniform":
        t = a + (b - a) * torch.rand(shape, generator=gen, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {kind!r}")
    return t.numpy()


def make_inputs(layer: Layer, seed: int, n: Optional[int] = None) -> dict:
    """Draw every host array a layer needs, deterministically from ``seed``.

    Returns a dict with ``x`` (float32 [n,H,W,Cin]), ``weight_bits`` (uint32
    [Cout,kh,kw,words]) and ``output_scale``/``output_bias`` (float32 [Cout])
    and ``input_scale``/``input_bias`` (float32 [Cin]), each possibly None.
    """
    n = layer.n if n is None else n
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = _draw(gen, layer.x_dist, (n, layer.in_h, layer.in_w, layer.in_c))
    words = torch.randint(0, 2 ** 32, (layer.out_c, layer.kernel_h, layer.kernel_w, layer.words),
                          generator=gen, dtype=torch.int64)
    weight_bits = words.numpy().astype(np.uint32)
    out = {"x": np.ascontiguousarray(x), "weight_bits": np.ascontiguousarray(weight_bits)}
    for key, dist, length in (("output_scale", layer.oscale_dist, layer.out_c),
                              ("output_bias", layer.obias_dist, layer.out_c),
                              ("input_scale", layer.iscale_dist, layer.in_c),
                              ("input_bias", layer.ibias_dist, layer.in_c)):
        out[key] = None if dist is None else np.ascontiguousarray(_draw(gen, dist, (length,)))
    return out


def make_packed_input(layer: Layer, seed: int, n: Optional[int] = None) -> np.ndarray:
    """Uniformly random uint32 words [n,H,W,ceil(Cin/32)] standing for packed
    input sign bits (bit c%32 of word c//32 is channel c).  The bits past Cin
    are random as well: a consumer must ignore them."""
    n = layer.n if n is None else n
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    words = torch.randint(0, 2 ** 32, (n, layer.in_h, layer.in_w, layer.words), generator=gen, dtype=torch.int64)
    return np.ascontiguousarray(words.numpy().astype(np.uint32))


def layer_seed(index: int) -> int:
    """Seed of measured layer ``index``."""
    return 1000 + index
