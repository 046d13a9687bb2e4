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
    BCONV_ERR_UNSUPPORTED, BCONV_ERR_WORKSPACE, BCONV_FLAG_BETA_VALID_TAPS, BCONV_FLAG_FP4_MFMA, BCONV_FLAG_INT8_MFMA, BCONV_FLAG_NONE,
    BCONV_FLAG_USE_BETA_SCALING,
    BCONV_NEURON_NONE, BCONV_NEURON_RELU, BCONV_OK, BCONV_XNOR, NEURON_CODES, TYPE_CODES,
    BconvError, BconvLibraryMissing, bconv_calibrate_popcount, bconv_create, bconv_create_fc, bconv_desc_t,
    bconv_destroy,
    BCONV_SCRATCH_MAX_BYTES, bconv_forward, bconv_forward_accum, bconv_forward_bits, bconv_forward_noalloc, bconv_forward_bits_profiled, bconv_forward_packed,
    bconv_forward_packed_bits, bconv_forward_profiled,
    bconv_get_info, bconv_last_error,
    bconv_main_kernel, bconv_status_string, bconv_validate_desc, bconv_workspace_layout,
    bconv_workspace_size, load_library, make_desc)


def check_tensor(t, name: str, shape, dtypes, device=None) -> None:
    """Raise ValueError unless ``t`` is a contiguous CUDA tensor of exactly
    ``shape`` with one of ``dtypes`` (on ``device`` when given).  The C entry
    points size every buffer from the layer descriptor, so a tensor that is
    smaller, strided or of another element type would be read or written
    past its end, or misread."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: a torch tensor is required, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} is not one of {', '.join(str(d) for d in dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: the tensor must be contiguous (NHWC, dense)")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: a CUDA (HIP) device tensor is required, got device {t.device}")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name}: on {t.device}, the input is on {device}")


def check_workspace(ws, need: int, device) -> None:
    """Raise ValueError unless ``ws`` is a contiguous device tensor on
    ``device`` holding at least ``need`` bytes."""
    import torch
    if not isinstance(ws, torch.Tensor):
        raise ValueError(f"workspace: a torch tensor is required, got {type(ws).__name__}")
    if not ws.is_contiguous():
        raise ValueError("workspace: the tensor must be contiguous")
    if ws.device.type != "cuda" or ws.device != torch.device(device):
        raise ValueError(f"workspace: on {ws.device}, the input is on {device}")
    have = ws.numel() * ws.element_size()
    if have < need:
        raise ValueError(f"workspace: {have} bytes given, {need} needed")


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
                 neuron_a: float = 0.0, neuron_b: float = 0.0, beta_valid_taps: bool = False,
                 fp4_mfma: bool = False):
        pe = pad if pad_end is None else pad_end
        self.desc = make_desc(in_h, in_w, in_c, out_c, kernel[0], kernel[1], stride[0], stride[1],
                              pad[0], pad[1], 1, NEURON_CODES[neuron], scale_value, pe[0], pe[1],
                              neuron_a, neuron_b)
        self.type = TYPE_CODES[type]
        self.flags = (BCONV_FLAG_USE_BETA_SCALING if use_beta else BCONV_FLAG_NONE) | \
            (BCONV_FLAG_INT8_MFMA if int8_mfma else BCONV_FLAG_NONE) | \
            (BCONV_FLAG_BETA_VALID_TAPS if beta_valid_taps else BCONV_FLAG_NONE) | \
            (BCONV_FLAG_FP4_MFMA if fp4_mfma else BCONV_FLAG_NONE)
        self.handle = bconv_create(self.desc, weight_bits, output_scale, output_bias,
                                   input_scale, input_bias, self.type, self.flags)
        self.in_h, self.in_w = in_h, in_w
        self.in_c, self.out_c, self.out_h, self.out_w = bconv_get_info(self.handle)

    @classmethod
    def from_layer(cls, layer, inputs: dict, int8_mfma: bool = False, fp4_mfma: bool = False) -> "BinaryConvolution":
        """Build from a ``workloads.Layer`` and the arrays ``make_inputs`` drew
        (``int8_mfma``: the int8 matrix-core comparison path; ``fp4_mfma``: the
        fp4 matrix-core comparison path of fully connected layers)."""
        return cls(in_h=layer.in_h, in_w=layer.in_w, in_c=layer.in_c, out_c=layer.out_c,
                   kernel=(layer.kernel_h, layer.kernel_w), stride=(layer.stride_h, layer.stride_w),
                   pad=(layer.pad_h, layer.pad_w), pad_end=(layer.pad_h_end, layer.pad_w_end),
                   type=layer.type,
                   weight_bits=inputs["weight_bits"], output_scale=inputs.get("output_scale"),
                   output_bias=inputs.get("output_bias"), input_scale=inputs.get("input_scale"),
                   input_bias=inputs.get("input_bias"), use_beta=layer.use_beta,
                   neuron=layer.neuron, scale_value=layer.scale_value, int8_mfma=int8_mfma,
                   neuron_a=layer.neuron_a, neuron_b=layer.neuron_b, beta_valid_taps=layer.beta_valid_taps,
                   fp4_mfma=fp4_mfma)

    def workspace_bytes(self, n: int) -> int:
        return bconv_workspace_size(self.handle, n)

    def workspace(self, n: int, device=None):
        import torch
        return torch.empty(max(1, self.workspace_bytes(n)), dtype=torch.uint8,
                           device=device or "cuda")

    def out_words(self) -> int:
        return (self.out_c + 31) // 32

    def in_words(self) -> int:
        return (self.in_c + 31) // 32

    def _launch(self, fn, x, x_shape, x_dtypes, out, out_shape, out_dtype, workspace, stream):
        """Checks the tensors against the layer, allocates what the caller did
        not pass on the launch stream itself (so the caching allocator never
        hands those blocks to other work while the kernels still use them),
        then calls the C entry point ``fn``."""
        import torch
        n = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 4 else -1
        check_tensor(x, "input", x_shape(n), x_dtypes)
        s = stream or torch.cuda.current_stream(x.device)
        with torch.cuda.device(x.device), torch.cuda.stream(s):
            if out is None:
                out = torch.empty(out_shape(n), dtype=out_dtype, device=x.device)
            if workspace is None:
                workspace = self.workspace(n, x.device)
        check_tensor(out, "output", out_shape(n), (out_dtype,), device=x.device)
        check_workspace(workspace, self.workspace_bytes(n), x.device)
        fn(self.handle, s.cuda_stream, n, x, out, workspace, workspace.numel() * workspace.element_size())
        return out

    def _in_shape(self, n):
        return (n, self.in_h, self.in_w, self.in_c)

    def _out_shape(self, n):
        return (n, self.out_h, self.out_w, self.out_c)

    def _bits_shape(self, n):
        return (n, self.out_h, self.out_w, self.out_words())

    def forward(self, x, out=None, workspace=None, stream=None):
        """float32 NHWC input [n, in_h, in_w, in_c] -> float32 NHWC output."""
        import torch
        return self._launch(bconv_forward, x, self._in_shape, (torch.float32,), out, self._out_shape,
                            torch.float32, workspace, stream)

    def forward_accum(self, x, acc=None, workspace=None, stream=None):
        """Window sums before the epilogue: int32 (XNOR/AND) or float32."""
        import torch
        dt = torch.float32 if self.type == BCONV_BINARY_WEIGHTS else torch.int32
        return self._launch(bconv_forward_accum, x, self._in_shape, (torch.float32,), acc, self._out_shape, dt,
                            workspace, stream)

    def forward_bits(self, x, out_bits=None, workspace=None, stream=None):
        """Packed sign bits of the output (see bconv_forward_bits), as int32
        words [n, out_h, out_w, ceil(out_c/32)] holding the uint32 bit patterns."""
        import torch
        return self._launch(bconv_forward_bits, x, self._in_shape, (torch.float32,), out_bits, self._bits_shape,
                            torch.int32, workspace, stream)

    def forward_packed(self, x_bits, out=None, workspace=None, stream=None, bits_out=False):
        """Forward pass from packed input sign bits (see bconv_forward_packed):
        int32 words [n, in_h, in_w, ceil(in_c/32)], e.g. a previous layer's
        forward_bits.  Returns fp32 NHWC, or packed output bits with bits_out."""
        import torch
        fn = bconv_forward_packed_bits if bits_out else bconv_forward_packed
        return self._launch(fn, x_bits, lambda n: (n, self.in_h, self.in_w, self.in_words()),
                            (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,),
                            out, self._bits_shape if bits_out else self._out_shape,
                            torch.int32 if bits_out else torch.float32, workspace, stream)

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
