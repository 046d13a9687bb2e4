"""Helpers shared by the GPU parity tests: run a layer through the C ABI,
run the oracle on the same host arrays, and compare.

Comparison rules (the oracle is float64 and exact; the HIP path is fp32):
  * XNOR / AND window sums: bit-exact.
  * packed input bits: bit-exact against the oracle's binarised input.
  * A map and beta image: relative 1e-5 (sums of non-negative terms).
  * final outputs, XNOR / AND: |g - o| <= 1e-5 * (|acc*scale*beta| + |bias|).
  * binaryWeights sums: |g - o| <= 1e-5 * S, S = sum of |x'| over the window;
    final outputs |g - o| <= 1e-5 * (|scale*beta| * S + |bias|).
A purely elementwise relative test is ill-posed where a sum cancels, so the
float bounds are normwise in the terms of each sum.
"""

from __future__ import annotations

import os
from contextlib import contextmanager

import numpy as np
import torch

import oracle
import popcount_convolution_amd as pca
from popcount_convolution_amd import workloads

RTOL = 1e-5
TINY = 1e-30


@contextmanager
def force_generic(on: bool, strip_width: int = 0, small_fused=None):
    """Handles created inside use the generic convolution kernel, or the
    specialised one at the given strip width (0: chosen by cost).  Small
    layers take the single-launch kernel by default; a forced kernel or
    strip width, or small_fused=False, keeps them on the two-kernel path."""
    if small_fused is None:
        small_fused = not on and not strip_width
    values = {"BCONV_FORCE_GENERIC": "1" if on else "0", "BCONV_STRIP_WIDTH": str(strip_width),
              "BCONV_SMALL_FUSED": "1" if small_fused else "0"}
    old = {k: os.environ.get(k) for k in values}
    os.environ.update(values)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def slice_inputs(inputs: dict, images) -> dict:
    out = dict(inputs)
    out["x"] = np.ascontiguousarray(inputs["x"][images])
    return out


def run_gpu(layer: workloads.Layer, inputs: dict, device, generic: bool = False,
            int8_mfma: bool = False, strip_width: int = 0, small_fused=None, fp4_mfma: bool = False) -> dict:
    """Forward and forward_accum through the C ABI; also returns the
    workspace intermediates (bits or int8 values, A map, beta) of the forward
    call.  ``int8_mfma`` selects the int8 matrix-core comparison path;
    ``strip_width`` forces the specialised convolution's pixels per wave;
    ``small_fused`` (None: the library's default) selects or avoids the
    single-launch small-layer kernel, which writes no workspace intermediates;
    ``fp4_mfma`` selects the fp4 matrix-core comparison path of a fully
    connected layer."""
    with force_generic(generic, strip_width, small_fused):
        conv = pca.BinaryConvolution.from_layer(layer, inputs, int8_mfma=int8_mfma, fp4_mfma=fp4_mfma)
    try:
        n = inputs["x"].shape[0]
        x = torch.from_numpy(inputs["x"]).to(device)
        ws = conv.workspace(n, device)
        ws.fill_(0xA5)  # poison: every byte the kernels rely on must be written
        shape = (n, conv.out_h, conv.out_w, conv.out_c)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device=device)
        if layer.type == "binary_weights":
            acc = torch.full(shape, float("nan"), dtype=torch.float32, device=device)
        else:
            acc = torch.full(shape, -(2 ** 31), dtype=torch.int32, device=device)
        conv.forward_accum(x, acc, ws)
        conv.forward(x, out, ws)
        torch.cuda.synchronize()
        res = {"out": out.cpu().numpy(), "acc": acc.cpu().numpy(),
               "main_kernel": conv.main_kernel(n)}
        L = pca.bconv_workspace_layout(conv.handle, n)
        wsh = ws.cpu().numpy()
        if res["main_kernel"].startswith("xconv_small"):
            return res  # binarised in registers: no bit buffer, A map or beta
        if L["bits_offset"] is not None:
            cnt = n * L["bits_rows"] * L["bits_cols"] * L["bits_words"]
            raw = wsh[L["bits_offset"]:L["bits_offset"] + 4 * cnt]
            if int8_mfma:
                res["int8"] = raw.view(np.int8).reshape(n, L["bits_rows"], L["bits_cols"], 4 * L["bits_words"])
            else:
                res["bits"] = raw.view("<u4").reshape(n, L["bits_rows"], L["bits_cols"], L["bits_words"])
            res["bits_pad"] = (L["bits_pad_h"], L["bits_pad_w"])
        if L["a_map_offset"] is not None:
            rows, cols = L["bits_rows"], L["bits_cols"]
            ph, pw = L["bits_pad_h"], L["bits_pad_w"]
            apad = wsh[L["a_map_offset"]:L["a_map_offset"] + 4 * n * rows * cols].view("<f4") \
                .reshape(n, rows, cols)
            res["a_map"] = apad[:, ph:ph + layer.in_h, pw:pw + layer.in_w]
            halo = apad.copy()
            halo[:, ph:ph + layer.in_h, pw:pw + layer.in_w] = 0
            res["a_halo_zero"] = not halo.any()
            nb = n * conv.out_h * conv.out_w
            res["beta"] = wsh[L["beta_offset"]:L["beta_offset"] + 4 * nb].view("<f4") \
                .reshape(n, conv.out_h, conv.out_w)
        return res
    finally:
        conv.close()


def expected_words(signs: np.ndarray, form: str) -> np.ndarray:
    """Pack the oracle's binarised input into little-endian uint32 words,
    channel c at bit c%32 of word c//32, zero tail bits."""
    bits = (signs > 0).astype(np.uint8)
    n, h, w, c = bits.shape
    words = (c + 31) // 32
    padded = np.zeros((n, h, w, words * 32), np.uint8)
    padded[..., :c] = bits
    packed = np.packbits(padded, axis=-1, bitorder="little")
    return packed.view("<u4").reshape(n, h, w, words)


def window_abs_sum(layer: workloads.Layer, inputs: dict) -> np.ndarray:
    """S[n,oy,ox] = sum of |x'| over the in-image taps of the window (float64)."""
    x = inputs["x"].astype(np.float64)
    if inputs.get("input_scale") is not None:
        x = x * inputs["input_scale"].astype(np.float64)
    if inputs.get("input_bias") is not None:
        x = x + inputs["input_bias"].astype(np.float64)
    a = torch.from_numpy(np.abs(x).sum(axis=-1)[:, None])
    a = torch.nn.functional.pad(a, (layer.pad_w, layer.pad_w_end, layer.pad_h, layer.pad_h_end))
    k = torch.ones((1, 1, layer.kernel_h, layer.kernel_w), dtype=torch.float64)
    s = torch.nn.functional.conv2d(a, k, stride=(layer.stride_h, layer.stride_w))
    return s.numpy()[:, 0]


# Lipschitz constant of each activation (a, b its parameters), and whether its
# fp32 evaluation rounds (then 1e-5 of the output is added to the bound).
def _neuron_lipschitz(layer: workloads.Layer):
    a, b = abs(layer.neuron_a), abs(layer.neuron_b)
    return {"none": (1.0, False), "relu": (1.0, False), "absolute": (1.0, False), "clamp": (1.0, False),
            "leaky_relu": (max(1.0, a), True), "linear": (a, True), "sigmoid": (0.25, True),
            "hard_sigmoid": (a, True), "tanh": (a * b, True), "softplus": (a * b, True),
            "softsign": (1.0, True), "elu": (max(1.0, a), True)}[layer.neuron]


def output_bound(layer: workloads.Layer, sub: dict, ref: dict) -> np.ndarray:
    """The normwise fp32 bound on each final output (see the module doc),
    carried through the activation: L * bound + 1e-5 * |out| for an
    activation with Lipschitz constant L whose fp32 evaluation rounds."""
    oc = layer.out_c
    scale = (sub["output_scale"].astype(np.float64) if sub.get("output_scale") is not None
             else np.full(oc, layer.scale_value, np.float64))
    bias = (sub["output_bias"].astype(np.float64) if sub.get("output_bias") is not None
            else np.zeros(oc))
    beta = ref["beta"][..., None]
    if layer.type == "binary_weights":
        S = window_abs_sum(layer, sub)[..., None]
        pre = RTOL * (np.abs(scale * beta) * S + np.abs(bias)) + TINY
    else:
        pre = RTOL * (np.abs(ref["acc"] * scale * beta) + np.abs(bias)) + TINY
    lip, rounds = _neuron_lipschitz(layer)
    return lip * pre + (RTOL * np.abs(ref["out"]) if rounds else 0.0)


def unpack_words(words: np.ndarray, nbits: int) -> np.ndarray:
    """uint32 words [..., W] -> bits [..., 32*W] (bit c%32 of word c//32), as uint8."""
    w = np.ascontiguousarray(words).view("<u4")
    b = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")
    return b[..., :nbits] if nbits is not None else b


def values_from_bits(words: np.ndarray, nbits: int) -> np.ndarray:
    """The fp32 input that packed sign bits stand for: +1 where the bit is 1
    and -1 where it is 0 (any input with these signs gives the same layer
    output under XNOR and AND); bits past ``nbits`` are dropped."""
    return np.where(unpack_words(words, nbits) != 0, 1.0, -1.0).astype(np.float32)


def compare_bits(layer: workloads.Layer, inputs: dict, words: np.ndarray, ref: dict = None, images=None):
    """Packed sign bits of the output against the oracle: bit = !(y < 0).  The
    sign is decided by the fp32 value, so positions whose oracle value lies
    within the fp32 bound of 0 may take either bit; every other bit must match,
    all of them under ReLU (its output is never below 0), and bits past out_c
    must be 0."""
    sub = inputs if images is None else slice_inputs(inputs, images)
    if ref is None:
        ref = oracle.bconv_layer(layer, sub)
    g = words if images is None else words[images]
    oc = layer.out_c
    nw = (oc + 31) // 32
    assert g.shape[-1] == nw, (g.shape, nw)
    allbits = unpack_words(g, None)
    assert not allbits[..., oc:].any(), f"{layer.name}: bits past out_c are set"
    bits = allbits[..., :oc]
    want = (~(ref["out"] < 0)).astype(np.uint8)
    if layer.neuron == "relu":
        certain = np.ones_like(want, dtype=bool)
    else:
        certain = np.abs(ref["out"]) > output_bound(layer, sub, ref)
    bad = certain & (bits != want)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{layer.name}: {int(bad.sum())} sign bits differ, first at {i}: "
                             f"gpu {bits[i]} oracle value {ref['out'][i]}")
    return int((~certain).sum())


def compare(layer: workloads.Layer, inputs: dict, got: dict, ref: dict = None, images=None,
            workspace: bool = True) -> dict:
    """Assert the GPU results (optionally only on `images`) match the oracle;
    ``workspace=False`` checks only the window sums and the output (no packed
    input, A map or beta from the workspace)."""
    sub = inputs if images is None else slice_inputs(inputs, images)
    if ref is None:
        ref = oracle.bconv_layer(layer, sub)
    g = {k: (v if images is None or not isinstance(v, np.ndarray) else v[images])
         for k, v in got.items()}
    if layer.type == "binary_weights":
        S = window_abs_sum(layer, sub)[..., None]
        err = np.abs(g["acc"].astype(np.float64) - ref["acc"])
        assert np.all(err <= RTOL * S + TINY), f"{layer.name}: binaryWeights sums off by {err.max()}"
    else:
        if not np.array_equal(g["acc"], ref["acc"]):
            bad = np.argwhere(g["acc"] != ref["acc"])
            i = tuple(bad[0])
            raise AssertionError(f"{layer.name}: {len(bad)} window sums differ, first at {i}: "
                                 f"gpu {g['acc'][i]} oracle {ref['acc'][i]}")
    bound = output_bound(layer, sub, ref)
    err = np.abs(g["out"].astype(np.float64) - ref["out"])
    ok = err <= bound
    if not np.all(ok):
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{layer.name}: {np.count_nonzero(~ok)} outputs beyond tolerance, "
                             f"first at {i}: gpu {g['out'][i]} oracle {ref['out'][i]}")
    if "bits" in g and ref.get("signs") is not None:
        ph, pw = got["bits_pad"]
        h, w = layer.in_h, layer.in_w
        inner = g["bits"][:, ph:ph + h, pw:pw + w, :]
        want = expected_words(ref["signs"], layer.type)
        assert np.array_equal(inner, want), f"{layer.name}: packed input bits differ"
        halo = g["bits"].copy()
        halo[:, ph:ph + h, pw:pw + w, :] = 0
        assert not halo.any(), f"{layer.name}: halo of the packed input is not zero"
    if "int8" in g and ref.get("signs") is not None:
        ph, pw = got["bits_pad"]
        h, w, c = layer.in_h, layer.in_w, layer.in_c
        neg = 0 if layer.type == "and" else -1
        want = np.where(ref["signs"] > 0, 1, neg).astype(np.int8)
        inner = g["int8"][:, ph:ph + h, pw:pw + w, :c]
        assert np.array_equal(inner, want), f"{layer.name}: int8 input values differ"
        rest = g["int8"].copy()
        rest[:, ph:ph + h, pw:pw + w, :c] = 0
        assert not rest.any(), f"{layer.name}: int8 halo or channel padding is not zero"
    if layer.use_beta and workspace:
        assert got["a_halo_zero"], f"{layer.name}: halo of the A map is not zero"
        np.testing.assert_allclose(g["a_map"], ref["a_map"], rtol=RTOL, atol=0,
                                   err_msg=f"{layer.name}: A map")
        np.testing.assert_allclose(g["beta"], ref["beta"], rtol=RTOL, atol=0,
                                   err_msg=f"{layer.name}: beta")
    return ref
