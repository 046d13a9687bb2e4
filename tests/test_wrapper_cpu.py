"""Argument checks of the torch-facing wrapper (no GPU needed).

The C entry points size every buffer from the layer descriptor, so the
wrapper must reject tensors that do not match the layer before anything is
launched: wrong element type, wrong shape, strided views, host tensors and
short workspaces each raise ValueError.
"""

import pytest
import torch

import popcount_convolution_amd as pca


def _fake_layer(type_code=pca.BCONV_XNOR):
    """A BinaryConvolution with the shape attributes of a 2 x 5x6x40 -> 70
    layer and no device handle: only the checks before the launch run."""
    conv = object.__new__(pca.BinaryConvolution)
    conv.handle = None
    conv.type = type_code
    conv.in_h, conv.in_w, conv.in_c = 5, 6, 40
    conv.out_c, conv.out_h, conv.out_w = 70, 5, 6
    return conv


def test_check_tensor_accepts_exact_match_apart_from_device():
    t = torch.zeros((2, 5, 6, 40), dtype=torch.float32)
    with pytest.raises(ValueError, match="CUDA"):
        pca.check_tensor(t, "input", (2, 5, 6, 40), (torch.float32,))


@pytest.mark.parametrize("bad,match", [
    (torch.zeros((2, 5, 6, 40), dtype=torch.float64), "dtype"),
    (torch.zeros((2, 5, 6, 40), dtype=torch.float16), "dtype"),
    (torch.zeros((2, 5, 6, 39), dtype=torch.float32), "shape"),
    (torch.zeros((2, 5, 7, 40), dtype=torch.float32), "shape"),
    (torch.zeros((2 * 5 * 6 * 40,), dtype=torch.float32), "shape"),
    (torch.zeros((2, 40, 5, 6), dtype=torch.float32).permute(0, 2, 3, 1), "contiguous"),
    ([0.0] * 2400, "torch tensor"),
])
def test_forward_rejects_mismatched_input(bad, match):
    conv = _fake_layer()
    with pytest.raises(ValueError, match=match):
        conv.forward(bad)


def test_forward_rejects_host_input():
    conv = _fake_layer()
    with pytest.raises(ValueError, match="CUDA"):
        conv.forward(torch.zeros((2, 5, 6, 40), dtype=torch.float32))


@pytest.mark.parametrize("method,bad,match", [
    ("forward_accum", torch.zeros((2, 5, 6, 40), dtype=torch.int32), "dtype"),
    ("forward_bits", torch.zeros((2, 5, 6, 40), dtype=torch.float64), "dtype"),
    ("forward_packed", torch.zeros((2, 5, 6, 2), dtype=torch.float32), "dtype"),
    ("forward_packed", torch.zeros((2, 5, 6, 40), dtype=torch.int32), "shape"),
    ("forward_packed", torch.zeros((2, 5, 6, 1), dtype=torch.int32), "shape"),
])
def test_other_entry_points_reject_mismatched_input(method, bad, match):
    conv = _fake_layer()
    with pytest.raises(ValueError, match=match):
        getattr(conv, method)(bad)


def test_output_and_workspace_checks():
    ok = torch.zeros((2, 5, 6, 70), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        pca.check_tensor(ok[:, :, :, :69], "output", (2, 5, 6, 70), (torch.float32,))
    with pytest.raises(ValueError, match="contiguous"):
        pca.check_tensor(ok[:, :, ::2], "output", (2, 5, 3, 70), (torch.float32,))
    with pytest.raises(ValueError, match="dtype"):
        pca.check_tensor(ok.int(), "output", (2, 5, 6, 70), (torch.float32,))
    with pytest.raises(ValueError, match="workspace"):
        pca.check_workspace(torch.zeros(64, dtype=torch.uint8), 16, "cpu")
    with pytest.raises(ValueError, match="contiguous"):
        pca.check_workspace(torch.zeros((8, 8), dtype=torch.uint8).t(), 16, "cpu")
    with pytest.raises(ValueError, match="torch tensor"):
        pca.check_workspace(1234, 16, "cpu")
