"""Host logic of bench.py that needs no GPU: the one-GPU rule, the
algorithmic byte counts of the measured layers, and the source hashes that
keep recorded traffic tied to the kernel code it was measured on."""

import os
import subprocess
import sys

import bench
from popcount_convolution_amd import workloads


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr


def test_bench_layer_algorithmic_bytes():
    """Packed input with its one-pixel zero halo (8 x 58 x 58 pixels x 4
    words), the same-halo A map, the weight bits and the fp32 output, counted
    by hand for the batch-8 56x56 128 -> 128 3x3 layer."""
    layer = workloads.BENCH_LAYER
    bits = 8 * 58 * 58 * 4 * 4
    amap = 8 * 58 * 58 * 4
    weights = 128 * 3 * 3 * 4 * 4
    out = 8 * 56 * 56 * 128 * 4
    assert bench.algorithmic_bytes(layer, 8) == bits + amap + weights + out == 13_401_728
    assert bench.algorithmic_bytes(layer, 8, bits_out=True) == bits + amap + weights + 8 * 56 * 56 * 4 * 4


def test_algorithmic_bytes_count_the_trailing_pad():
    """An even kernel's centred window pads one side less: the halo rows and
    columns counted are the leading plus the trailing pad."""
    layer = workloads.BENCH_LAYER.with_(n=1, kernel_h=2, kernel_w=2, pad_h=1, pad_w=1, pad_bottom=0, pad_right=0,
                                        use_beta=False)
    words_in = 4
    assert bench.algorithmic_bytes(layer, 1) == (57 * 57 * words_in * 4 + 128 * 2 * 2 * 4 * 4
                                                 + layer.out_h * layer.out_w * 128 * 4)


def test_kernel_source_hash(tmp_path, monkeypatch):
    """Comments and whitespace do not change a kernel's source hash, code does;
    kernels from different files hash differently; an unknown record gives
    None."""
    import shutil
    a = bench._kernel_sha("xconv_fast<3,3,4,1,7>")
    csrc = tmp_path / "popcount_convolution_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "popcount_convolution_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = csrc / "xconv_fast.h"
    f.write_text("// a new comment\n/* and a block\n comment */\n" + f.read_text().replace("\n", "\n\n"))
    assert bench._kernel_sha("xconv_fast<3,3,4,1,7>") == a
    f.write_text(f.read_text().replace("acc[p] = 0;", "acc[p] = 1;"))
    assert bench._kernel_sha("xconv_fast<3,3,4,1,7>") != a
    monkeypatch.undo()
    assert a == bench._kernel_sha("xconv_fast<3,3,8,1,7>")  # same source file
    assert a != bench._kernel_sha("bgemm_kernel<false>")
    assert bench._kernel_sha("bgemm_f4_kernel<false>") != bench._kernel_sha("bgemm_kernel<false>")
    assert bench._kernel_sha("xconv_f4_kernel<true>") == bench._kernel_sha("bgemm_f4_kernel<false>")  # one file
    assert bench._kernel_sha("xconv_f4_kernel<true>") != bench._kernel_sha("xconv_fast<3,3,8,1,7>")
    assert bench.recorded_traffic("no such workload", "xconv_fast<3,3,4,1,7>") is None
    assert bench.recorded_traffic(workloads.BENCH_LAYER.name, "bgemm_kernel<false>") is None


def test_pack_algorithmic_bytes():
    """fp32 input read once, packed bits and A map written once, without the
    halo: the per-layer minimum pack bytes, counted by hand."""
    L = workloads.LAYERS
    assert bench.pack_algorithmic_bytes(L[0], 1) == 16 * 16 * 64 * 4 + 16 * 16 * 2 * 4 == 67_584
    assert bench.pack_algorithmic_bytes(L[1], 8) == 8 * 56 * 56 * (128 * 4 + 4 * 4 + 4) == 13_346_816
    assert bench.pack_algorithmic_bytes(L[2], 32) == 32 * 28 * 28 * (256 * 4 + 8 * 4) == 26_492_928
    assert bench.pack_algorithmic_bytes(L[3], 16) is None  # binaryWeights without beta: no pack step
    assert bench.pack_algorithmic_bytes(L[4], 256) == 256 * 49 * (512 * 4 + 16 * 4) == 26_492_928
    assert bench.pack_kernel_name(L[1]) == "pack_vec4<32,4,1>"
    assert bench.pack_kernel_name(L[4]) == "pack_vec4<64,2,2>"
    assert bench.pack_kernel_name(L[3]) is None


def test_headline_is_the_largest_layer():
    """The default line quotes the layer with the most bit-MACs per step."""
    biggest = max(workloads.LAYERS, key=lambda l: l.nominal_macs())
    assert workloads.HEADLINE_LAYER is biggest and biggest.is_fc


def test_fp4_route_and_roofline():
    """The fp4 comparison path takes XNOR / AND layers whose fully connected
    window, or convolution pixel, is a multiple of 4 words; its roofline
    counts two fp4 operations per bit-MAC against the dense fp4 peak, or HBM
    where the layer's bytes take longer."""
    L = workloads.LAYERS
    assert [bench.fp4_route(l) for l in L] == [False, True, True, False, True]
    assert bench.fp4_roofline(L[1], 8, 0.005)["bound"] == "hbm"
    assert not bench.fp4_route(L[4].with_(in_c=96))       # 7*7*3 = 147 words
    assert not bench.fp4_route(L[4].with_(type="binary_weights"))
    r = bench.fp4_roofline(L[4], 256, 0.010)             # 10 us per launch
    macs = 256 * 4096 * 7 * 7 * 512
    assert r["bound"] == "mfma" and r["peak"] == 10100.0
    assert abs(r["achieved"] - 2 * macs / 1e-5 / 1e12) < 1e-2
    assert abs(r["of_popcount_peak"] - macs / 1e-5 / 1e12 / bench.POPCOUNT_PEAK_TBITMAC) < 1e-4
