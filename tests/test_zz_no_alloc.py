"""bconv_forward_noalloc: the forward pass with the library's built-in device
workspace (for callers that cannot allocate), against bconv_forward with a
caller workspace on the same handle and inputs, and against the oracle.

Two calls in a row on one GPU, the second with a smaller batch (and, in the
mixed test, another layer), so what the first left in the shared array must
not leak into the second.  The size limit is checked on the host.
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


def _both(conv, x, n, dev):
    """(bconv_forward with a caller workspace, bconv_forward_noalloc) outputs."""
    s = torch.cuda.current_stream().cuda_stream
    shape = (n, conv.out_h, conv.out_w, conv.out_c)
    ref = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    got = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    ws = conv.workspace(n, dev)
    ws.fill_(0xA5)
    pca.bconv_forward(conv.handle, s, n, x, ref, ws, ws.numel())
    pca.bconv_forward_noalloc(conv.handle, s, n, x, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("index", range(len(workloads.LAYERS)), ids=[l.name for l in workloads.LAYERS])
def test_noalloc_matches_forward(dev, index):
    """Full batch, then a smaller one, on one handle: bit-identical to
    bconv_forward, and the oracle's result within the parity bounds."""
    layer = workloads.LAYERS[index]
    inputs = workloads.make_inputs(layer, workloads.layer_seed(index))
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    try:
        assert conv.workspace_bytes(layer.n) <= pca.BCONV_SCRATCH_MAX_BYTES
        for n in (layer.n, max(1, layer.n // 3)):
            print(f"noalloc {layer.name} n={n}", flush=True)
            x = torch.from_numpy(np.ascontiguousarray(inputs["x"][:n])).to(dev)
            ref, got = _both(conv, x, n, dev)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{layer.name} n={n}"
            sub = parity.slice_inputs(inputs, slice(0, n))
            want = oracle.bconv_layer(layer, sub, want=("out", "acc", "beta"))
            bound = parity.output_bound(layer, sub, want)
            assert np.all(np.abs(got.astype(np.float64) - want["out"]) <= bound), f"{layer.name} n={n}"
    finally:
        conv.close()


def test_noalloc_two_layers_in_a_row(dev):
    """A beta layer with a large bit buffer, then a smaller layer of another
    shape without beta: the second reads none of the first's leftovers."""
    big = workloads.BENCH_LAYER.with_(n=6, name="noalloc_big")
    small = workloads.LAYERS[2].with_(n=2, in_h=9, in_w=13, name="noalloc_small")
    for layer, seed in ((big, 41), (small, 42)):
        inputs = workloads.make_inputs(layer, seed)
        conv = pca.BinaryConvolution.from_layer(layer, inputs)
        try:
            x = torch.from_numpy(inputs["x"]).to(dev)
            ref, got = _both(conv, x, layer.n, dev)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), layer.name
            want = oracle.bconv_layer(layer, inputs, want=("out", "acc", "beta"))
            assert np.all(np.abs(got.astype(np.float64) - want["out"]) <= parity.output_bound(layer, inputs, want))
        finally:
            conv.close()


def test_noalloc_rejects_batches_beyond_the_scratch(dev):
    """A batch whose workspace exceeds BCONV_SCRATCH_MAX_BYTES is refused on
    the host (WORKSPACE) before anything is launched; n = 0 is a no-op."""
    layer = workloads.LAYERS[2]
    inputs = workloads.make_inputs(layer, workloads.layer_seed(2), n=1)
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    try:
        n = 1
        while conv.workspace_bytes(n) <= pca.BCONV_SCRATCH_MAX_BYTES:
            n *= 2
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward_noalloc(conv.handle, None, n, None, None)
        assert e.value.status == pca.BCONV_ERR_WORKSPACE
        pca.bconv_forward_noalloc(conv.handle, None, 0, None, None)
        with pytest.raises(pca.BconvError) as e:
            pca.bconv_forward_noalloc(None, None, 1, None, None)
        assert e.value.status == pca.BCONV_ERR_INVALID_ARGUMENT
    finally:
        conv.close()
