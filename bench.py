#!/usr/bin/env python3
"""Throughput of the binary-convolution forward pass on one MI355X.

One step = one full forward call (pack + A map, beta, convolution or matrix
kernel with fused epilogue) over one batch of a measured layer, inputs
already resident in HBM.  The default run measures all five measured layers
and prints one JSON line whose headline is the largest of them, the binary
fully connected layer (256 x 7x7x512 -> 4096, 26.3 G bit-MACs per step):
  value      nominal bit-MACs (N*Ho*Wo*Cout*kh*kw*Cin) per second of whole
             steps, in G bit-MAC/s (= binary GOPS);
  roofline   the convolution / matrix kernel alone, timed by hipEvents that its
             dispatch records itself (a second pass over the same K steps, so
             the events do not perturb `value`), against whichever peak binds
             it: the VALU popcount peak (XNOR/AND), the bf16 matrix cores at
             three products per fp32 product (binaryWeights), or HBM;
  pack       the binarise-and-pack kernel (with the A map) of the same steps,
             timed the same way: algorithmic bytes (fp32 input read once,
             packed bits and A map written once) per second against HBM;
  configs    the same figures (and cpu_baseline) for every measured layer;
  comparison    (XNOR / AND) the same layer through the int8 matrix-core
             path (BCONV_FLAG_INT8_MFMA), timed the same way, with its own
             roofline against the dense int8 MFMA peak or HBM; for the fully
             connected layer also through the fp4 matrix-core path
             (BCONV_FLAG_FP4_MFMA), against the dense fp4 peak; and the layer
             with its output written as packed sign bits for a next binary
             layer (bconv_forward_bits), timed the same way; and (XNOR / AND
             without beta or input affine) the layer fed packed sign bits
             (bconv_forward_packed / _bits: repad + convolution), whole steps;
  calibration   measured ceilings of this GPU: the popcount path's two
             instructions on registers (the library's calibration kernel, T
             bit-MAC/s; the roofline object adds the kernel's fraction of it
             beside the published peak) and a 1 GiB device copy (GB/s);
  cpu_baseline  the CPU oracle timed on the layer's whole batch (all host
             cores), with a one-thread one-image per-core figure;
  cpu_packed_baseline  (XNOR / AND) the packed-bit popcount form on the CPU
             (the oracle package's second reference point), whole batch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layer I]
       (--layer I: only measured layer I, which is then the headline)
       python bench.py --sweep   (geometry sweep around the XNOR + beta layer:
                                  strides, paddings, odd and even kernels; one JSON line)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# 256 CUs x 64 lanes per clock x 2.4 GHz = 3.932e13 32-bit VALU lane-ops/s;
# XNOR/AND cost 2 lane-ops (xor/and, then bcnt with accumulate) per 32 bit-MACs.
VALU_LANE_OPS = 256 * 64 * 2.4e9
POPCOUNT_PEAK_TBITMAC = VALU_LANE_OPS * 16 / 1e12          # 629.1
# binaryWeights runs on the bf16 matrix cores (2.5 PFLOP/s dense), three bf16
# products per exact fp32 product: 2500/3 TFLOP/s of fp32-exact work.
BF16X3_PEAK_TFLOPS = 2500.0 / 3
# dense int8 MFMA: 5.0 POP/s = 2.5e15 multiply-accumulates per second
INT8_PEAK_TMAC = 2500.0
# dense fp4 (e2m1) MFMA: 10.1 PFLOP/s
FP4_PEAK_TFLOPS = 10100.0
HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(layer, n, bits_out=False, fp32_input=False):
    """Bytes the convolution / matrix kernel must move at least: its input
    operand once (packed bits for XNOR/AND, fp32 for binaryWeights and for
    the single-launch small-layer kernel, `fp32_input`, which binarises its
    own input), the A map when beta is on, the weight bits and the output
    (fp32, or packed sign bits with `bits_out`)."""
    words = (layer.in_c + 31) // 32
    if layer.is_fc:
        rows, cols = layer.in_h, layer.in_w
    else:
        rows, cols = layer.in_h + layer.pad_h + layer.pad_h_end, layer.in_w + layer.pad_w + layer.pad_w_end
    if layer.type == "binary_weights" or fp32_input:
        src = n * layer.in_h * layer.in_w * layer.in_c * 4
    else:
        src = n * rows * cols * words * 4
    amap = n * rows * cols * 4 if layer.use_beta else 0
    weights = layer.out_c * layer.kernel_h * layer.kernel_w * words * 4
    out = n * layer.out_h * layer.out_w * (((layer.out_c + 31) // 32) if bits_out else layer.out_c) * 4
    return src + amap + weights + out


def int8_algorithmic_bytes(layer, n):
    """Bytes the int8 matrix-core kernel must move at least: the int8 input
    (channels padded to 64, zero halo) once, the A map when beta is on, the
    int8 weights and the fp32 output."""
    cpad = (layer.in_c + 63) // 64 * 64
    if layer.is_fc:
        rows, cols = layer.in_h, layer.in_w
    else:
        rows, cols = layer.in_h + layer.pad_h + layer.pad_h_end, layer.in_w + layer.pad_w + layer.pad_w_end
    src = n * rows * cols * cpad
    amap = n * rows * cols * 4 if layer.use_beta else 0
    weights = layer.out_c * layer.kernel_h * layer.kernel_w * cpad
    out = n * layer.out_h * layer.out_w * layer.out_c * 4
    return src + amap + weights + out


def pack_algorithmic_bytes(layer, n):
    """Bytes the binarise-and-pack kernel must move at least: the fp32 input
    read once, the packed bits (XNOR / AND) and the A map (beta) written once,
    without the zero halo the library adds around them.  None when the layer
    has no pack step (binaryWeights without beta)."""
    pixels = n * layer.in_h * layer.in_w
    bits = pixels * ((layer.in_c + 31) // 32) * 4 if layer.type != "binary_weights" else 0
    amap = pixels * 4 if layer.use_beta else 0
    if not bits and not amap:
        return None
    return pixels * layer.in_c * 4 + bits + amap


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--layer", type=int, default=None,
                   help="measure only this index into workloads.LAYERS (then also the headline)")
    p.add_argument("--cpu-images", type=int, default=256,
                   help="at most this many images of each layer for cpu_baseline (0: skip)")
    p.add_argument("--cpu-repeats", type=int, default=3)
    p.add_argument("--no-int8", action="store_true",
                   help="skip the matrix-core comparisons (int8 for XNOR / AND layers, fp4 for fully connected ones)")
    p.add_argument("--sweep", action="store_true",
                   help="time the convolution over a sweep of strides, paddings and kernel sizes")
    p.add_argument("--sweep-widths", action="store_true",
                   help="with --sweep: also time every strip width of the specialised convolution")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip the measured popcount-peak and HBM-copy calibration")
    p.add_argument("--no-bits", action="store_true",
                   help="skip the packed sign-bit output comparison")
    p.add_argument("--profile-only", action="store_true",
                   help="run warmup + timed steps and print nothing else (for rocprofv3)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="also run one device-to-device copy of this many MiB (calibrates HBM "
                        "byte counters under rocprofv3 --pmc)")
    return p.parse_args()


def cpu_baseline(layer, inputs, images: int, repeats: int):
    """Time the oracle (as it stands) on the first `images` images."""
    import numpy as np

    import oracle
    sub = dict(inputs)
    sub["x"] = np.ascontiguousarray(inputs["x"][:images])
    threads = os.cpu_count() or 1
    oracle.load()
    best = None
    for _ in range(max(1, repeats)):
        t = time.perf_counter()
        oracle.bconv_layer(layer, sub, threads=threads, want=("out",))
        dt = time.perf_counter() - t
        best = dt if best is None else min(best, dt)
    macs = layer.nominal_macs(images)
    # one host thread on one image: the per-core rate
    sub1 = dict(inputs)
    sub1["x"] = np.ascontiguousarray(inputs["x"][:1])
    t = time.perf_counter()
    oracle.bconv_layer(layer, sub1, threads=1, want=("out",))
    one = time.perf_counter() - t
    unit = "GOPS (bit-MAC/s)" if layer.type != "binary_weights" else "GMAC/s (fp32)"
    return {"value": macs / best / 1e9, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{images} of {layer.n} images of {layer.name}, best of {repeats} runs "
                      f"({best:.3f} s each, {macs} nominal MACs)",
            "per_core": {"value": layer.nominal_macs(1) / one / 1e9, "unit": unit, "cores": 1,
                         "sample": f"1 image, 1 thread ({one:.3f} s)"},
            "host": host_cpu(), "build": "gcc -std=c11 -O2 -fopenmp -ffp-contract=off (no intrinsics)"}


def host_cpu() -> str:
    """The host CPU's model name and logical core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical cores"


def cpu_packed_baseline(layer, inputs, repeats: int):
    """Time the packed-bit popcount CPU baseline on the whole batch, all host cores."""
    import oracle
    threads = os.cpu_count() or 1
    oracle.load_packed()
    best = None
    for _ in range(max(1, repeats)):
        t = time.perf_counter()
        oracle.packed_bconv(layer, inputs, threads=threads)
        dt = time.perf_counter() - t
        best = dt if best is None else min(best, dt)
    macs = layer.nominal_macs()
    return {"value": macs / best / 1e9, "unit": "GOPS (bit-MAC/s)", "cores": threads,
            "kind": "packed popcount CPU (oracle/packed_cpu.c)",
            "sample": f"all {layer.n} images of {layer.name}, best of {repeats} runs ({best * 1e3:.3f} ms each)"}


def sweep_layers(workloads):
    """Geometries around the bench layer (XNOR + beta + affine + ReLU, batch 8,
    128 -> 128 channels): strides 1 and 2, paddings none / centred, kernels
    1, 2, 3, 4, 5 (even ones with the centred window's asymmetric padding)."""
    base = workloads.BENCH_LAYER
    out = []
    for k in (1, 2, 3, 4, 5):
        for s in (1, 2):
            for centred in (True, False):
                if k == 1 and not centred:
                    continue
                p, pe = (k // 2, (k - 1) // 2) if centred else (0, 0)
                name = f"xnor_beta_b8_56x56_c128_o128_k{k}_s{s}_p{p}{'' if pe == p else f'-{pe}'}"
                out.append(base.with_(name=name, kernel_h=k, kernel_w=k, stride_h=s, stride_w=s, pad_h=p, pad_w=p,
                                      pad_bottom=pe, pad_right=pe))
    return out


def run_sweep(args):
    import numpy as np
    import torch

    import popcount_convolution_amd as pca
    from popcount_convolution_amd import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    rows = []
    # BCONV_STRIP_WIDTH (read when a handle is created) forces the strip width
    widths = (0, 4, 6, 7, 8) if args.sweep_widths else (0,)
    for i, layer in enumerate(sweep_layers(workloads)):
        inputs = workloads.make_inputs(layer, 4000 + i)
        x = torch.from_numpy(inputs["x"]).to(dev)
        for width in widths:
            os.environ["BCONV_STRIP_WIDTH"] = str(width)
            conv = pca.BinaryConvolution.from_layer(layer, inputs)
            os.environ.pop("BCONV_STRIP_WIDTH")
            kernel = conv.main_kernel(layer.n)
            if width and not kernel.endswith(f",{width}>"):
                conv.close()
                continue
            ms, main_ms, _, out = time_path(pca, torch, np, conv, layer.n, x, stream, args.warmup, args.steps)
            macs = layer.nominal_macs()
            achieved = macs / (main_ms / 1e3) / 1e12
            rows.append({"workload": layer.name, "strip_width": width or "auto", "kernel": kernel,
                         "out_hw": [layer.out_h, layer.out_w], "avg_kernel_us": round(main_ms * 1e3, 3),
                         "ms_per_step": round(ms, 6), "value": round(macs / (ms / 1e3) / 1e9, 3),
                         "achieved": round(achieved, 3), "frac": round(achieved / POPCOUNT_PEAK_TBITMAC, 4)})
            print(f"# {layer.name}: {kernel} {rows[-1]['avg_kernel_us']} us, frac {rows[-1]['frac']}",
                  file=sys.stderr, flush=True)
            del out
            conv.close()
    print(json.dumps({"metric": "binary conv GOPS (bit-MACs/s) over a geometry sweep, 1 MI355X",
                      "unit": "GOPS (bit-MAC/s)", "peak_unit": "Tbit-MAC/s", "peak": POPCOUNT_PEAK_TBITMAC,
                      "steps": args.steps, "warmup": args.warmup, "n_gpus": 1, "data": "synthetic", "sweep": rows}),
          flush=True)


def roofline_of(layer, n, kernel_ms, bits_out=False, kernel=""):
    """Roofline object of a convolution / matrix kernel that ran `kernel_ms`
    per launch: whichever of compute and HBM takes longer at peak binds it."""
    macs = layer.nominal_macs(n)
    nbytes = algorithmic_bytes(layer, n, bits_out=bits_out, fp32_input=kernel.startswith("xconv_small"))
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if layer.type != "binary_weights":
        t_cmp = macs / (POPCOUNT_PEAK_TBITMAC * 1e12)
        cmp = ("alu", macs / (kernel_ms / 1e3) / 1e12, POPCOUNT_PEAK_TBITMAC, "Tbit-MAC/s")
    else:
        t_cmp = 2 * macs / (BF16X3_PEAK_TFLOPS * 1e12)
        cmp = ("mfma", 2 * macs / (kernel_ms / 1e3) / 1e12, BF16X3_PEAK_TFLOPS, "TFLOP/s (fp32-exact, bf16x3)")
    if t_hbm > t_cmp:
        bound, achieved, peak, unit = "hbm", nbytes / (kernel_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = cmp
    return {"bound": bound, "achieved": round(achieved, 3), "peak": round(peak, 3), "unit": unit,
            "frac": round(achieved / peak, 4), "algorithmic_bytes": nbytes,
            "avg_kernel_us": round(kernel_ms * 1e3, 3)}


def fp4_route(layer):
    """Whether the fp4 matrix-core comparison path takes the layer: XNOR / AND
    of the fully connected shape with a window of a multiple of 4 words, or a
    convolution whose pixel is a multiple of 4 words (at most 1024 groups of
    4 words per window)."""
    if layer.type == "binary_weights":
        return False
    words = (layer.in_c + 31) // 32
    if layer.is_fc:
        return (layer.kernel_h * layer.kernel_w * words) % 4 == 0
    return words % 4 == 0 and layer.kernel_h * layer.kernel_w * words // 4 <= 1024


def fp4_roofline(layer, n, kernel_ms):
    """Roofline of the fp4 matrix-core product: two fp4 operations per
    bit-MAC against the dense fp4 peak, or HBM, whichever binds at peak; with
    its rate as a fraction of the VALU popcount peak beside it."""
    macs = layer.nominal_macs(n)
    nbytes = algorithmic_bytes(layer, n)
    if nbytes / (HBM_PEAK_GBS * 1e9) > 2 * macs / (FP4_PEAK_TFLOPS * 1e12):
        bound, achieved, peak, unit = "hbm", nbytes / (kernel_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", 2 * macs / (kernel_ms / 1e3) / 1e12, FP4_PEAK_TFLOPS, "TFLOP/s (fp4)"
    bitmacs = macs / (kernel_ms / 1e3) / 1e12
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "algorithmic_bytes": nbytes, "avg_kernel_us": round(kernel_ms * 1e3, 3),
            "tbitmac_per_s": round(bitmacs, 3), "of_popcount_peak": round(bitmacs / POPCOUNT_PEAK_TBITMAC, 4)}


def pack_entry(layer, n, pack_ms, kernel):
    """The pack kernel of the step against HBM: algorithmic bytes per launch
    over its average dispatch duration."""
    nb = pack_algorithmic_bytes(layer, n)
    if nb is None or pack_ms is None:
        return None
    achieved = nb / (pack_ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes": nb, "avg_kernel_us": round(pack_ms * 1e3, 3),
            "traffic": recorded_traffic(layer.name + "#pack", kernel)}


def measure_layer(pca, torch, np, workloads, index, args, stream):
    """Every figure of one measured layer: whole steps, its main and pack
    kernels, the comparisons, and the CPU baselines."""
    layer = workloads.LAYERS[index]
    inputs = workloads.make_inputs(layer, workloads.layer_seed(index))
    dev = torch.device("cuda:0")
    conv = pca.BinaryConvolution.from_layer(layer, inputs)
    n = layer.n
    x = torch.from_numpy(inputs["x"]).to(dev)
    print(f"# {layer.name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    ms_per_step, main_ms, pack_ms, out = time_path(pca, torch, np, conv, n, x, stream, args.warmup, args.steps)
    if args.profile_only:
        conv.close()
        return None
    macs = layer.nominal_macs()
    binary = layer.type != "binary_weights"
    kernel = conv.main_kernel(n)
    unit = "GOPS (bit-MAC/s)" if binary else "GMAC/s (fp32)"
    entry = {"workload": layer.name, "value": round(macs / (ms_per_step / 1e3) / 1e9, 3), "unit": unit,
             "ms_per_step": round(ms_per_step, 6), "nominal_macs": macs,
             "config": {"workload": layer.name, "type": layer.type, "batch": n,
                        "input_hwc": [layer.in_h, layer.in_w, layer.in_c], "out_c": layer.out_c,
                        "kernel": [layer.kernel_h, layer.kernel_w],
                        "stride": [layer.stride_h, layer.stride_w], "pad": [layer.pad_h, layer.pad_w],
                        "beta": layer.use_beta, "input_affine": layer.iscale_dist is not None,
                        "neuron": layer.neuron, "parallelism": "none (1 GPU)"},
             "roofline": dict(kernel=kernel, **roofline_of(layer, n, main_ms, kernel=kernel),
                              traffic=recorded_traffic(layer.name, kernel)),
             "pack": pack_entry(layer, n, pack_ms, pack_kernel_name(layer)) if pack_ms is not None else None}
    comparison = {}
    if kernel.startswith("xconv_small"):
        # the same layer on the two-kernel path (pack, then the convolution)
        os.environ["BCONV_SMALL_FUSED"] = "0"
        try:
            conv2 = pca.BinaryConvolution.from_layer(layer, inputs)
        finally:
            os.environ.pop("BCONV_SMALL_FUSED", None)
        ms2, main2, pack2, out2 = time_path(pca, torch, np, conv2, n, x, stream, args.warmup, args.steps)
        same = bool(torch.equal(out2, out))
        comparison["two_launch"] = {
            "what": "the same layer as two kernels (binarise-and-pack, then the convolution), the path the "
                    "single-launch small-layer kernel replaces",
            "value": round(macs / (ms2 / 1e3) / 1e9, 3), "unit": unit, "ms_per_step": round(ms2, 6),
            "kernel": conv2.main_kernel(n), "avg_kernel_us": round(main2 * 1e3, 3),
            "pack_avg_kernel_us": round(pack2 * 1e3, 3) if pack2 is not None else None,
            "output_bit_identical": same}
        del out2
        conv2.close()
    if binary and not args.no_int8:
        conv8 = pca.BinaryConvolution.from_layer(layer, inputs, int8_mfma=True)
        ms8, main8, _, out8 = time_path(pca, torch, np, conv8, n, x, stream, args.warmup, args.steps)
        diff8 = float((out8 - out).abs().max()) if out.numel() else 0.0
        del out8
        nb8 = int8_algorithmic_bytes(layer, n)
        if nb8 / (HBM_PEAK_GBS * 1e9) > macs / (INT8_PEAK_TMAC * 1e12):
            r8 = ("hbm", nb8 / (main8 / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s")
        else:
            r8 = ("mfma", macs / (main8 / 1e3) / 1e12, INT8_PEAK_TMAC, "TMAC/s (int8)")
        k8 = conv8.main_kernel(n)
        comparison["int8_mfma"] = {
            "value": round(macs / (ms8 / 1e3) / 1e9, 3), "unit": unit,
            "ms_per_step": round(ms8, 6), "kernel": k8, "avg_kernel_us": round(main8 * 1e3, 3),
            "kernel_speed_vs_popcount": round(main_ms / main8, 4),
            "max_abs_diff_vs_popcount_output": diff8,
            "roofline": {"bound": r8[0], "achieved": round(r8[1], 3), "peak": r8[2], "unit": r8[3],
                         "frac": round(r8[1] / r8[2], 4), "algorithmic_bytes": nb8,
                         "traffic": recorded_traffic(layer.name + "#int8_mfma", k8)}}
        conv8.close()
    if not args.no_int8 and fp4_route(layer):
        conv4 = pca.BinaryConvolution.from_layer(layer, inputs, fp4_mfma=True)
        ms4, main4, _, out4 = time_path(pca, torch, np, conv4, n, x, stream, args.warmup, args.steps)
        same4 = bool(torch.equal(out4, out))
        del out4
        k4 = conv4.main_kernel(n)
        comparison["fp4_mfma"] = {
            "what": "the layer on the fp4 matrix cores (BCONV_FLAG_FP4_MFMA): the 0/1 bit product count as exact "
                    "e2m1 products, XNOR from it and the input and weight bit counts",
            "value": round(macs / (ms4 / 1e3) / 1e9, 3), "unit": unit,
            "ms_per_step": round(ms4, 6), "kernel": k4, "avg_kernel_us": round(main4 * 1e3, 3),
            "kernel_speed_vs_popcount": round(main_ms / main4, 4),
            "output_bit_identical_to_popcount": same4,
            "roofline": dict(fp4_roofline(layer, n, main4), traffic=recorded_traffic(layer.name + "#fp4_mfma", k4))}
        conv4.close()
    if not args.no_bits:
        msb, mainb, _, outb = time_path(pca, torch, np, conv, n, x, stream, args.warmup, args.steps, bits=True)
        del outb
        comparison["packed_bits_output"] = {
            "value": round(macs / (msb / 1e3) / 1e9, 3), "unit": unit,
            "ms_per_step": round(msb, 6), "kernel": kernel, "avg_kernel_us": round(mainb * 1e3, 3),
            "output_bytes": (n * layer.out_h * layer.out_w * ((layer.out_c + 31) // 32) * 4),
            "roofline": roofline_of(layer, n, mainb, bits_out=True, kernel=kernel)}
    if (binary and not layer.use_beta and layer.iscale_dist is None and layer.ibias_dist is None
            and not args.no_bits):
        words = torch.from_numpy(workloads.make_packed_input(layer, workloads.layer_seed(index) + 77).view(np.int32))
        words = words.to(dev)
        msp = {fmt: time_packed(pca, torch, conv, n, words, stream, args.warmup, args.steps, fmt == "bits")
               for fmt in ("fp32", "bits")}
        del words
        comparison["packed_input"] = {
            "what": "bconv_forward_packed: input given as packed sign bits (a previous binary layer's output), "
                    "so the step is repad + convolution, without the fp32 pack",
            "input_bytes": n * layer.in_h * layer.in_w * layer.words * 4,
            "fp32_output": {"value": round(macs / (msp["fp32"] / 1e3) / 1e9, 3), "unit": unit,
                            "ms_per_step": round(msp["fp32"], 6)},
            "bits_output": {"value": round(macs / (msp["bits"] / 1e3) / 1e9, 3), "unit": unit,
                            "ms_per_step": round(msp["bits"], 6)}}
    if comparison:
        entry["comparison"] = comparison
    del out
    conv.close()
    if args.cpu_images > 0:
        print(f"# {layer.name}: CPU oracle", file=sys.stderr, flush=True)
        entry["cpu_baseline"] = cpu_baseline(layer, inputs, min(args.cpu_images, n), args.cpu_repeats)
        if binary and layer.neuron in ("none", "relu"):
            entry["cpu_packed_baseline"] = cpu_packed_baseline(layer, inputs, args.cpu_repeats)
    else:
        entry["cpu_baseline"] = None
    return entry


def pack_kernel_name(layer):
    """Name of the binarise-and-pack kernel the library launches for a layer
    (the fast path takes in_c % 4 == 0 with 16-byte aligned arrays, which torch
    allocations are), or None when it launches none."""
    if pack_algorithmic_bytes(layer, 1) is None:
        return None
    if layer.in_c % 4:
        return "pack_kernel"
    seg = 1
    while seg < (layer.in_c + 3) // 4 and seg < 64:
        seg <<= 1
    nc = 1 if layer.in_c <= 4 * seg else (2 if layer.in_c <= 8 * seg else 0)
    return f"pack_vec4<{seg},{2 if nc == 2 else 4},{nc}>"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not offered, the path runs on a single "
              "MI355X and has no multi-GPU form. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import popcount_convolution_amd as pca
    from popcount_convolution_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.sweep:
        run_sweep(args)
        return
    # a dedicated stream at the default priority
    stream = torch.cuda.Stream()
    indices = range(len(workloads.LAYERS)) if args.layer is None else [args.layer]
    head_index = workloads.LAYERS.index(workloads.HEADLINE_LAYER) if args.layer is None else args.layer
    entries = {i: measure_layer(pca, torch, np, workloads, i, args, stream) for i in indices}
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if args.profile_only:
        return
    head = entries[head_index]
    line = {
        "metric": "binary conv GOPS (bit-MACs/s) and % of VALU popcount peak, 1 MI355X",
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32" if workloads.LAYERS[head_index].type != "binary_weights" else "f32",
        "data": "synthetic (seeded; weight bits Bernoulli(0.5))",
        "config": head["config"],
        "roofline": head["roofline"],
        "pack": head["pack"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for key in ("cpu_packed_baseline", "comparison"):
        if key in head:
            line[key] = head[key]
    if not args.no_calibration:
        cal = calibrate(pca, torch, stream)
        line["calibration"] = cal
        mp = cal["popcount_peak"]["value"]
        for e in entries.values():
            if e["roofline"]["bound"] == "alu":
                e["roofline"]["measured_peak"] = mp
                e["roofline"]["frac_of_measured_peak"] = round(e["roofline"]["achieved"] / mp, 4)
    line["configs"] = [{k: v for k, v in e.items() if k not in ("comparison", "config")}
                       | {"comparison": e.get("comparison")} for i, e in sorted(entries.items())]
    print(json.dumps(line), flush=True)


def calibrate(pca, torch, stream):
    """Measured ceilings on this GPU: the popcount path's instruction pair
    (v_xor_b32 + v_bcnt_u32_b32 on registers, 8 waves per SIMD, the library's
    calibration kernel) in T bit-MAC/s, and a device-to-device copy of 1 GiB
    (torch) in GB/s read + written.  Best of 5 timed runs each."""
    simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * simds, 4096  # 256-thread blocks: 8 waves per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    sptr = stream.cuda_stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    best = None
    for i in range(6):
        ev[0].record(stream)
        pca.bconv_calibrate_popcount(sptr, blocks, iters, 1 + i, sink)
        ev[1].record(stream)
        ev[1].synchronize()
        if i:  # the first run warms up
            t = ev[0].elapsed_time(ev[1]) / 1e3
            best = t if best is None else min(best, t)
    bitmacs = blocks * 256 * iters * 8 * 32
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        tc = None
        for _ in range(5):
            ev[0].record(stream)
            dst.copy_(src)
            ev[1].record(stream)
            ev[1].synchronize()
            t = ev[0].elapsed_time(ev[1]) / 1e3
            tc = t if tc is None else min(tc, t)
    moved = 2 * src.numel() * 4
    del src, dst, sink
    return {"popcount_peak": {"value": round(bitmacs / best / 1e12, 3), "unit": "Tbit-MAC/s",
                              "published": POPCOUNT_PEAK_TBITMAC, "kernel": "popc_peak_kernel",
                              "work": f"{blocks} x 256 threads x {iters} rounds x 8 xor+bcnt pairs"},
            "hbm_copy": {"value": round(moved / tc / 1e9, 1), "unit": "GB/s (read + write)",
                         "published": HBM_PEAK_GBS, "bytes": moved}}


def time_path(pca, torch, np, conv, n, x, stream, warmup, steps, bits=False):
    """Warm up, then (1) time `steps` whole forward calls between two stream
    events, (2) run the same steps again with hipEvents recorded by the main
    kernel's and the input step's own dispatches.  Returns (ms per step, mean
    main-kernel ms, mean input-step ms or None, output).  With `bits` the
    output is the packed sign-bit form (bconv_forward_bits)."""
    dev = x.device
    if bits:
        out = torch.empty((n, conv.out_h, conv.out_w, (conv.out_c + 31) // 32), dtype=torch.int32, device=dev)
        fwd, fwd_prof = pca.bconv_forward_bits, pca.bconv_forward_bits_profiled
    else:
        out = torch.empty((n, conv.out_h, conv.out_w, conv.out_c), dtype=torch.float32, device=dev)
        fwd, fwd_prof = pca.bconv_forward, pca.bconv_forward_profiled
    ws_bytes = max(1, conv.workspace_bytes(n))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    sptr = stream.cuda_stream
    for _ in range(warmup):
        fwd(conv.handle, sptr, n, x, out, ws, ws_bytes)
    torch.cuda.synchronize()

    # timed region 1: K whole forward steps -> value
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fwd(conv.handle, sptr, n, x, out, ws, ws_bytes)
    t1.record(stream)
    torch.cuda.synchronize()

    # timed region 2: the same K steps, each with hipEvents recorded by the
    # input step's and the main kernel's dispatches themselves
    # (hipExtLaunchKernelGGL) -> their durations
    # binaryWeights without beta launches no input step, nor does the
    # single-launch small-layer kernel (it binarises its own input)
    has_input = ((conv.type != pca.BCONV_BINARY_WEIGHTS or bool(conv.flags & pca.BCONV_FLAG_USE_BETA_SCALING))
                 and not conv.main_kernel(n).startswith("xconv_small"))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4 if has_input else 2)] for _ in range(steps)]
    for e in ev:
        for k in e:
            k.record(stream)  # creates the underlying hipEvent
    torch.cuda.synchronize()
    for e in ev:
        fwd_prof(conv.handle, sptr, n, x, out, ws, ws_bytes, e[0].cuda_event, e[1].cuda_event,
                 e[2].cuda_event if has_input else None, e[3].cuda_event if has_input else None)
    torch.cuda.synchronize()
    main_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    pack_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) if has_input else None
    return t0.elapsed_time(t1) / steps, main_ms, pack_ms, out


def time_packed(pca, torch, conv, n, words, stream, warmup, steps, bits_out):
    """ms per step of `steps` bconv_forward_packed (or _bits) calls on packed
    input words, between two stream events, after `warmup` untimed calls."""
    dev = words.device
    if bits_out:
        out = torch.empty((n, conv.out_h, conv.out_w, (conv.out_c + 31) // 32), dtype=torch.int32, device=dev)
        fwd = pca.bconv_forward_packed_bits
    else:
        out = torch.empty((n, conv.out_h, conv.out_w, conv.out_c), dtype=torch.float32, device=dev)
        fwd = pca.bconv_forward_packed
    ws_bytes = max(1, conv.workspace_bytes(n))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    sptr = stream.cuda_stream
    for _ in range(warmup):
        fwd(conv.handle, sptr, n, words, out, ws, ws_bytes)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fwd(conv.handle, sptr, n, words, out, ws, ws_bytes)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


# the source file that defines (and launches) each main kernel, by name prefix
# (first matching prefix wins)
KERNEL_FILES = {"xconv_f4": "gemm_f4.hip", "xconv_fast": "xconv_fast.h", "xconv_generic": "xconv.hip", "xconv_small": "xconv_small.hip",
                "bgemm_f4": "gemm_f4.hip", "bgemm": "gemm.hip", "bwmma": "bwmma.hip", "bwconv": "bwconv.hip", "i8mma": "i8mma.hip",
                "pack_vec4": "pack.hip", "pack_kernel": "pack.hip"}


def _kernel_sha(kernel: str) -> str:
    """Hash of the code a main kernel is built from (its own file and the
    shared internal header, comments and whitespace removed): recorded
    traffic stays valid while it matches."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "popcount_convolution_amd", "csrc")
    base = kernel.split("<")[0]
    prefix = next(p for p in KERNEL_FILES if base.startswith(p))
    for name in (KERNEL_FILES[prefix], "internal.h"):
        with open(os.path.join(csrc, name)) as f:
            code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", f.read(), flags=re.S)
        h.update(name.encode() + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(key: str, kernel: str):
    """HBM bytes per launch recorded under profiles/ for `key`, or None when
    absent or taken from other kernel sources."""
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(tfile):
        return None
    with open(tfile) as f:
        entry = json.load(f).get(key)
    if entry and entry.get("kernel") == kernel and entry.get("source_sha") == _kernel_sha(kernel):
        return entry.get("bytes_per_launch")
    return None


if __name__ == "__main__":
    main()
