"""Binary convolution on AMD Instinct MI355X (gfx950).

The forward pass (binarise-and-pack, beta, XNOR/AND popcount convolution,
binaryWeights convolution, fused epilogue) runs in the hand-written HIP kernels
of ``libbconv.so``, reached through its C ABI (``include/bconv.h``).  This
package holds the ctypes binding (``_binding``), a small torch-facing wrapper
(``BinaryConvolution``: torch only provides device memory and the current
stream) and the seeded synthetic workloads (``workloads``).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from ._binding import (  # noqa: F401  (re-exported C ABI names)
    BCONV_AND, BCONV_BINARY_WEIGHTS, BCONV_ERR_ALLOC, BCONV_ERR_HIP, BCONV_ERR_INVALID_ARGUMENT,
    BCONV_ERR_UNSUPPORTED, BCONV_ERR_WORKSPACE, BCONV_FLAG_BETA_VALID_TAPS, BCONV_FLAG_INT8_MFMA, BCONV_FLAG_NONE,
    BCONV_FLAG_USE_BETA_SCALING,
    BCONV_NEURON_NONE, BCONV_NEURON_RELU, BCONV_OK, BCONV_XNOR, NEURON_CODES, TYPE_CODES,
    BconvError, BconvLibraryMissing, bconv_calibrate_popcount, bconv_create, bconv_create_fc, bconv_desc_t,
    bconv_destroy,
    bconv_forward, bconv_forward_accum, bconv_forward_bits, bconv_forward_bits_profiled, bconv_forward_packed,
    bconv_forward_packed_bits, bconv_forward_profiled,
    bconv_get_info, bconv_last_error,
    bconv_main_kernel, bconv_status_string, bconv_validate_desc, bconv_workspace_layout,
    bconv_workspace_size, load_library, make_desc)


class BinaryConvolution:
    """One binary convolution layer on the current GPU.

    ``type`` is ``"xnor"``, ``"and"`` or ``"binary_weights"``; ``weight_bits``
    is a host uint32 array ``[out_c][kernel_h][kernel_w][ceil(in_c/32)]``; the
    scale/bias arrays are host float32 (or None).  ``forward`` takes a CUDA
    (HIP) float32 NHWC tensor and returns the float32 NHWC output.
    """

    def __init__(self, *, in_h: int, in_w: int, in_c: int, out_c: int, kernel: tuple,
                 stride: tuple = (1, 1), pad: tuple = (0, 0), pad_end=None, type: str = "xnor",
                 weight_bits: np.ndarray, output_scale=None, output_bias=None,
                 input_scale=None, input_bias=None, use_beta: bool = False,
                 neuron: str = "none", scale_value: float = 1.0, int8_mfma: bool = False,
                 neuron_a: float = 0.0, neuron_b: float = 0.0, beta_valid_taps: bool = False):
        pe = pad if pad_end is None else pad_end
        self.desc = make_desc(in_h, in_w, in_c, out_c, kernel[0], kernel[1], stride[0], stride[1],
                              pad[0], pad[1], 1, NEURON_CODES[neuron], scale_value, pe[0], pe[1],
                              neuron_a, neuron_b)
        self.type = TYPE_CODES[type]
        self.flags = (BCONV_FLAG_USE_BETA_SCALING if use_beta else BCONV_FLAG_NONE) | \
            (BCONV_FLAG_INT8_MFMA if int8_mfma else BCONV_FLAG_NONE) | \
            (BCONV_FLAG_BETA_VALID_TAPS if beta_valid_taps else BCONV_FLAG_NONE)
        self.handle = bconv_create(self.desc, weight_bits, output_scale, output_bias,
                                   input_scale, input_bias, self.type, self.flags)
        self.in_c, self.out_c, self.out_h, self.out_w = bconv_get_info(self.handle)

    @classmethod
    def from_layer(cls, layer, inputs: dict, int8_mfma: bool = False) -> "BinaryConvolution":
        """Build from a ``workloads.Layer`` and the arrays ``make_inputs`` drew
        (``int8_mfma``: the int8 matrix-core comparison path)."""
        return cls(in_h=layer.in_h, in_w=layer.in_w, in_c=layer.in_c, out_c=layer.out_c,
                   kernel=(layer.kernel_h, layer.kernel_w), stride=(layer.stride_h, layer.stride_w),
                   pad=(layer.pad_h, layer.pad_w), pad_end=(layer.pad_h_end, layer.pad_w_end),
                   type=layer.type,
                   weight_bits=inputs["weight_bits"], output_scale=inputs.get("output_scale"),
                   output_bias=inputs.get("output_bias"), input_scale=inputs.get("input_scale"),
                   input_bias=inputs.get("input_bias"), use_beta=layer.use_beta,
                   neuron=layer.neuron, scale_value=layer.scale_value, int8_mfma=int8_mfma,
                   neuron_a=layer.neuron_a, neuron_b=layer.neuron_b, beta_valid_taps=layer.beta_valid_taps)

    def workspace_bytes(self, n: int) -> int:
        return bconv_workspace_size(self.handle, n)

    def workspace(self, n: int, device=None):
        import torch
        return torch.empty(max(1, self.workspace_bytes(n)), dtype=torch.uint8,
                           device=device or "cuda")

    def _stream(self, stream):
        import torch
        return (stream or torch.cuda.current_stream()).cuda_stream

    def forward(self, x, out=None, workspace=None, stream=None):
        import torch
        n = x.shape[0]
        if out is None:
            out = torch.empty((n, self.out_h, self.out_w, self.out_c), dtype=torch.float32,
                              device=x.device)
        if workspace is None:
            workspace = self.workspace(n, x.device)
        bconv_forward(self.handle, self._stream(stream), n, x, out, workspace,
                      workspace.numel() * workspace.element_size())
        return out

    def forward_accum(self, x, acc=None, workspace=None, stream=None):
        """Window sums before the epilogue: int32 (XNOR/AND) or float32."""
        import torch
        n = x.shape[0]
        if acc is None:
            dt = torch.float32 if self.type == BCONV_BINARY_WEIGHTS else torch.int32
            acc = torch.empty((n, self.out_h, self.out_w, self.out_c), dtype=dt, device=x.device)
        if workspace is None:
            workspace = self.workspace(n, x.device)
        bconv_forward_accum(self.handle, self._stream(stream), n, x, acc, workspace,
                            workspace.numel() * workspace.element_size())
        return acc

    def out_words(self) -> int:
        return (self.out_c + 31) // 32

    def forward_bits(self, x, out_bits=None, workspace=None, stream=None):
        """Packed sign bits of the output (see bconv_forward_bits), as int32
        words [n, out_h, out_w, ceil(out_c/32)] holding the uint32 bit patterns."""
        import torch
        n = x.shape[0]
        if out_bits is None:
            out_bits = torch.empty((n, self.out_h, self.out_w, self.out_words()), dtype=torch.int32,
                                   device=x.device)
        if workspace is None:
            workspace = self.workspace(n, x.device)
        bconv_forward_bits(self.handle, self._stream(stream), n, x, out_bits, workspace,
                           workspace.numel() * workspace.element_size())
        return out_bits

    def forward_packed(self, x_bits, out=None, workspace=None, stream=None, bits_out=False):
        """Forward pass from packed input sign bits (see bconv_forward_packed):
        int32 words [n, in_h, in_w, ceil(in_c/32)], e.g. a previous layer's
        forward_bits.  Returns fp32 NHWC, or packed output bits with bits_out."""
        import torch
        n = x_bits.shape[0]
        if out is None:
            shape = (n, self.out_h, self.out_w, self.out_words() if bits_out else self.out_c)
            out = torch.empty(shape, dtype=torch.int32 if bits_out else torch.float32, device=x_bits.device)
        if workspace is None:
            workspace = self.workspace(n, x_bits.device)
        fn = bconv_forward_packed_bits if bits_out else bconv_forward_packed
        fn(self.handle, self._stream(stream), n, x_bits, out, workspace, workspace.numel() * workspace.element_size())
        return out

    def main_kernel(self, n: int) -> str:
        return bconv_main_kernel(self.handle, n)

    def close(self):
        if getattr(self, "handle", None):
            bconv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
