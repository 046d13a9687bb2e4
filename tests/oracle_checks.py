"""Pins of the CPU oracle against facts fixed outside it.

Every ``check_*`` function takes a loaded oracle library (``ctypes.CDLL``) and
raises ``AssertionError`` on a mismatch.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with a plausible mistake planted, and requires that some check catches each.

What each check compares against (never the oracle's own formula):
  * values printed on the pages (``tests/golden/``): the XNOR truth table, the
    value sets of a 32-bit word dot product, the FC conditions, the beta
    window;
  * the word identities of the pages computed with Python's integer popcount;
  * ``torch.nn.functional.conv2d`` in float64 on +-1 / 0,1 tensors (a textbook
    routine: zero padding in the +-1 domain is "padded taps add nothing");
  * a float64 ``numpy`` matmul of flattened vectors (the FC matrix view);
  * closed forms (all-ones weights, constant inputs, hand-built epilogues);
  * exact rational arithmetic (``fractions``) for the input affine's sign.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def bits_to_values(weight_bits: np.ndarray, in_c: int, form: str) -> np.ndarray:
    """Unpack uint32 words [Cout,kh,kw,words] to [Cout,kh,kw,Cin] with numpy's
    little-endian bit order (byte 0 of a little-endian word holds bits 0..7)."""
    w = np.ascontiguousarray(weight_bits.astype("<u4"))
    b = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")[..., :in_c].astype(np.float64)
    return b if form == "and" else 2.0 * b - 1.0


def conv2d_ref(values_nhwc: np.ndarray, weights_okkc: np.ndarray, stride, pad) -> np.ndarray:
    """float64 torch conv2d, zero padding, NHWC in and out."""
    xt = torch.from_numpy(np.ascontiguousarray(values_nhwc.transpose(0, 3, 1, 2)))
    wt = torch.from_numpy(np.ascontiguousarray(weights_okkc.transpose(0, 3, 1, 2)))
    y = torch.nn.functional.conv2d(xt, wt, stride=tuple(stride), padding=tuple(pad))
    return y.numpy().transpose(0, 2, 3, 1)


def conv2d_ref_pad(values_nhwc: np.ndarray, weights_okkc: np.ndarray, stride, pad, pad_end) -> np.ndarray:
    """float64 torch conv2d after explicit zero padding: `pad` rows / columns
    before (top, left) and `pad_end` after (bottom, right); NHWC in and out."""
    xt = torch.from_numpy(np.ascontiguousarray(values_nhwc.transpose(0, 3, 1, 2)))
    xt = torch.nn.functional.pad(xt, (pad[1], pad_end[1], pad[0], pad_end[0]))
    wt = torch.from_numpy(np.ascontiguousarray(weights_okkc.transpose(0, 3, 1, 2)))
    y = torch.nn.functional.conv2d(xt, wt, stride=tuple(stride))
    return y.numpy().transpose(0, 2, 3, 1)


def _run(lib, x, wbits, form, out_c, k=(1, 1), s=(1, 1), p=(0, 0), **kw):
    return oracle.bconv(x, wbits, type=form, out_c=out_c, kernel=k, stride=s, pad=p, lib=lib,
                        threads=1, **kw)


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_bits(rng, shape):
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)


def _popcount(v: int) -> int:
    return bin(v).count("1")


# ---------------------------------------------------------------- page values

def check_truth_table(lib):
    """Single channel, 1x1 kernel: each (input bit, weight bit) pair gives
    2*XNOR - 1 under the XNOR form and a AND b under the AND form."""
    for a, b, o in ((int(r[0]), int(r[1]), int(r[2])) for r in _rows("xnor_truth_table.txt")):
        x = np.array([[[[1.0 if a else -1.0]]]], np.float32)
        w = np.array([[[[b]]]], np.uint32)
        got = _run(lib, x, w, "xnor", 1)["acc"][0, 0, 0, 0]
        assert got == 2 * o - 1, (a, b, got)
        got_and = _run(lib, x, w, "and", 1)["acc"][0, 0, 0, 0]
        assert got_and == (a & b), (a, b, got_and)


def check_word_identities(lib):
    """Cin = 32, 1x1: the +-1 dot product of one pixel with one weight word is
    32 - 2*popcount(x ^ w); the 0/1 product is popcount(x & w).  Edge words and
    seeded random words; input bit 1 <=> x >= 0."""
    rng = _rng(1)
    edge = [0, 0xFFFFFFFF, 1, 0x80000000, 0x55555555, 0xAAAAAAAA, 0x0000FFFF, 0xFFFF0000]
    xw = [(a, b) for a in edge for b in edge]
    xw += [(int(a), int(b)) for a, b in zip(_rand_bits(rng, 300), _rand_bits(rng, 300))]
    xs = np.empty((len(xw), 1, 1, 32), np.float32)
    for i, (xa, _) in enumerate(xw):
        mags = rng.uniform(0.1, 3.0, 32).astype(np.float32)
        xs[i, 0, 0] = np.where([(xa >> c) & 1 for c in range(32)], mags, -mags)
    for j in range(0, len(xw), 16):
        chunk = xw[j:j + 16]
        wb = np.array([[[[w]]] for _, w in chunk], np.uint32)
        r = _run(lib, xs[j:j + 16], wb, "xnor", len(chunk))["acc"]
        ra = _run(lib, xs[j:j + 16], wb, "and", len(chunk))["acc"]
        for u, (xa, _) in enumerate(chunk):
            for v, (_, wv) in enumerate(chunk):
                assert r[u, 0, 0, v] == 32 - 2 * _popcount(xa ^ wv)
                assert ra[u, 0, 0, v] == _popcount(xa & wv)


def check_word_ranges(lib):
    """The sums a single word can produce are exactly the printed value sets."""
    ranges = {r[0]: set(range(int(r[1]), int(r[2]) + 1, int(r[3])))
              for r in _rows("word_dot_ranges.txt")}
    rng = _rng(2)
    seen = {"xnor": set(), "and": set()}
    # weights with every popcount 0..32 against one all-positive pixel reach
    # every value; random pixels add interior coverage.
    wwords = np.array([(1 << k) - 1 if k < 32 else 0xFFFFFFFF for k in range(33)], np.uint32)
    wb = wwords.reshape(33, 1, 1, 1)
    x = np.concatenate([np.ones((1, 1, 1, 32), np.float32),
                        rng.normal(size=(40, 1, 1, 32)).astype(np.float32)])
    for form in ("xnor", "and"):
        acc = _run(lib, x, wb, form, 33)["acc"]
        seen[form] |= set(int(v) for v in acc.ravel())
        assert seen[form] <= ranges[form], (form, sorted(seen[form] - ranges[form]))
        assert seen[form] == ranges[form], (form, sorted(ranges[form] - seen[form]))


def check_fc_conditions_and_matmul(lib):
    """A kernel the size of the source, stride 1, no padding gives a 1x1
    output equal to a float64 matmul of the NHWC-flattened +-1 input with the
    [No, H*W*Cin] weight matrix (FC matrix view), for all three forms."""
    cond = {r[0]: r[1] for r in _rows("fc_conditions.txt")}
    rng = _rng(3)
    for (h, w, c, no, n) in ((3, 4, 37, 5, 3), (1, 1, 64, 7, 2), (2, 5, 33, 4, 2)):
        x = rng.normal(size=(n, h, w, c)).astype(np.float32)
        wb = _rand_bits(rng, (no, h, w, (c + 31) // 32))
        kh = h if cond["kernel_h"] == "source" else int(cond["kernel_h"])
        kw = w if cond["kernel_w"] == "source" else int(cond["kernel_w"])
        st = (int(cond["stride_h"]), int(cond["stride_w"]))
        for form in ("xnor", "and", "binary_weights"):
            r = _run(lib, x, wb, form, no, k=(kh, kw), s=st)
            assert r["acc"].shape == (n, int(cond["out_h"]), int(cond["out_w"]), no)
            if form == "binary_weights":
                xv = x.astype(np.float64)
            elif form == "xnor":
                xv = np.where(x < 0, -1.0, 1.0)
            else:
                xv = np.where(x < 0, 0.0, 1.0)
            wmat = bits_to_values(wb, c, form).reshape(no, -1)
            want = xv.reshape(n, -1) @ wmat.T
            got = r["acc"][:, 0, 0, :]
            if form == "binary_weights":
                np.testing.assert_allclose(got, want, rtol=0, atol=1e-9)
            else:
                assert np.array_equal(got, want.astype(np.int64)), form


def check_fc_equals_centred_conv(lib):
    """The fully connected page's note: a general convolution centred on the
    source (offset = kernel/2), evaluated at one output, is the FC layer.  With
    odd k = source size and pad = k//2, output (k//2, k//2) of the padded conv
    equals the FC output."""
    rng = _rng(4)
    for (k, c, no) in ((3, 40, 6), (5, 17, 3), (1, 64, 4)):
        x = rng.normal(size=(2, k, k, c)).astype(np.float32)
        wb = _rand_bits(rng, (no, k, k, (c + 31) // 32))
        for form in ("xnor", "and"):
            fc = _run(lib, x, wb, form, no, k=(k, k))["acc"][:, 0, 0, :]
            conv = _run(lib, x, wb, form, no, k=(k, k), p=(k // 2, k // 2))["acc"]
            assert np.array_equal(conv[:, k // 2, k // 2, :], fc), (k, form)


def check_beta_window(lib):
    """Window offsets [-k/2, (k-1)/2] (beta equation): with pad = k//2 and
    stride 1, output y sees exactly the input rows y + first .. y + last.  A
    one-hot input through all-ones binaryWeights reveals the window."""
    for row in _rows("beta_window.txt"):
        k, first, last = int(row[0]), int(row[1]), int(row[2])
        size = 11
        wb = np.full((1, k, k, 1), 1, np.uint32)
        for pos in range(size):
            x = np.zeros((1, size, size, 1), np.float32)
            x[0, pos, pos, 0] = 1.0
            acc = _run(lib, x, wb, "binary_weights", 1, k=(k, k), p=(k // 2, k // 2))["acc"]
            for y in range(min(size, acc.shape[1])):
                inside = first <= pos - y <= last
                assert acc[0, y, y, 0] == (1.0 if inside else 0.0), (k, pos, y)


def check_centred_window_any_kernel(lib):
    """The beta equation's window [-k/2, (k-1)/2] as leading padding k/2 and
    trailing padding (k-1)/2, stride 1: the output keeps the input size for
    even kernels as for odd ones, and output y sees exactly input rows
    y + first .. y + last of the fixture."""
    for row in _rows("beta_window.txt"):
        k, first, last = int(row[0]), int(row[1]), int(row[2])
        size = 9
        wb = np.full((1, k, k, 1), 1, np.uint32)
        for pos in range(size):
            x = np.zeros((1, size, size, 1), np.float32)
            x[0, pos, pos, 0] = 1.0
            acc = _run(lib, x, wb, "binary_weights", 1, k=(k, k), p=(k // 2, k // 2),
                       pad_end=((k - 1) // 2, (k - 1) // 2))["acc"]
            assert acc.shape[1:3] == (size, size), (k, acc.shape)
            for y in range(size):
                inside = first <= pos - y <= last
                assert acc[0, y, y, 0] == (1.0 if inside else 0.0), (k, pos, y)


# ----------------------------------------------------------- textbook routines

def check_bruteforce_conv(lib):
    """XNOR / AND sums equal a float64 conv2d of the binarised input with the
    unpacked weights, zero padding, on small random geometries."""
    rng = _rng(5)
    cases = [(2, 6, 7, 33, 5, 3, 3, 1, 1, 1, 1), (1, 9, 5, 64, 3, 3, 3, 2, 2, 1, 1),
             (3, 5, 5, 1, 4, 1, 1, 1, 1, 0, 0), (1, 8, 8, 31, 2, 5, 5, 3, 2, 2, 1),
             (2, 4, 6, 65, 3, 2, 3, 1, 2, 1, 0), (1, 7, 7, 100, 4, 3, 1, 2, 1, 0, 2)]
    for (n, h, w, c, o, kh, kw, sh, sw, ph, pw) in cases:
        x = rng.normal(size=(n, h, w, c)).astype(np.float32)
        x[rng.random(x.shape) < 0.05] = 0.0
        wb = _rand_bits(rng, (o, kh, kw, (c + 31) // 32))
        for form in ("xnor", "and"):
            got = _run(lib, x, wb, form, o, k=(kh, kw), s=(sh, sw), p=(ph, pw))["acc"]
            xv = np.where(x < 0, -1.0 if form == "xnor" else 0.0, 1.0)
            want = conv2d_ref(xv, bits_to_values(wb, c, form), (sh, sw), (ph, pw))
            assert got.shape == want.shape
            assert np.array_equal(got, np.rint(want).astype(np.int64)), (form, n, h, w, c)


def check_bruteforce_asymmetric_padding(lib):
    """Different leading and trailing padding (even kernels, and odd ones):
    XNOR / AND sums equal a float64 conv2d of the binarised input after
    explicit zero padding, binaryWeights sums its full-precision conv2d, and
    beta the box sum of the A map over the same padded window / (kh*kw)."""
    rng = _rng(15)
    cases = [(2, 6, 7, 33, 5, 2, 2, 1, 1, 1, 1, 0, 0), (1, 9, 8, 64, 3, 4, 4, 1, 1, 2, 2, 1, 1),
             (1, 7, 9, 40, 4, 4, 2, 2, 1, 2, 1, 1, 0), (2, 5, 6, 17, 3, 3, 3, 1, 2, 0, 1, 2, 2),
             (1, 8, 8, 100, 2, 6, 6, 1, 1, 3, 3, 2, 2), (1, 4, 5, 3, 2, 2, 3, 1, 1, 0, 2, 1, 0)]
    for (n, h, w, c, o, kh, kw, sh, sw, ph, pw, phe, pwe) in cases:
        x = rng.normal(size=(n, h, w, c)).astype(np.float32)
        x[rng.random(x.shape) < 0.05] = 0.0
        wb = _rand_bits(rng, (o, kh, kw, (c + 31) // 32))
        geo = dict(k=(kh, kw), s=(sh, sw), p=(ph, pw), pad_end=(phe, pwe))
        for form in ("xnor", "and"):
            got = _run(lib, x, wb, form, o, **geo)["acc"]
            xv = np.where(x < 0, -1.0 if form == "xnor" else 0.0, 1.0)
            want = conv2d_ref_pad(xv, bits_to_values(wb, c, form), (sh, sw), (ph, pw), (phe, pwe))
            assert got.shape == want.shape, (got.shape, want.shape)
            assert np.array_equal(got, np.rint(want).astype(np.int64)), (form, kh, kw, ph, phe)
        r = _run(lib, x, wb, "binary_weights", o, use_beta=True, **geo)
        want = conv2d_ref_pad(x.astype(np.float64), bits_to_values(wb, c, "xnor"), (sh, sw), (ph, pw), (phe, pwe))
        np.testing.assert_allclose(r["acc"], want, rtol=0, atol=1e-12)
        a = np.abs(x.astype(np.float64)).sum(axis=-1, keepdims=True) / c
        box = conv2d_ref_pad(a, np.ones((1, kh, kw, 1)), (sh, sw), (ph, pw), (phe, pwe))[..., 0] / (kh * kw)
        np.testing.assert_allclose(r["beta"], box, rtol=1e-12, atol=0)


def check_binary_weights_conv(lib):
    """binaryWeights: the full-precision input convolved with 2*bit - 1
    weights, float64 conv2d, to 1e-12."""
    rng = _rng(6)
    for (n, h, w, c, o, k, s, p) in ((2, 7, 6, 20, 3, 3, 2, 1), (1, 5, 5, 64, 4, 1, 1, 0),
                                     (1, 9, 9, 3, 2, 5, 1, 2)):
        x = rng.normal(size=(n, h, w, c)).astype(np.float32)
        wb = _rand_bits(rng, (o, k, k, (c + 31) // 32))
        got = _run(lib, x, wb, "binary_weights", o, k=(k, k), s=(s, s), p=(p, p))["acc"]
        want = conv2d_ref(x.astype(np.float64), bits_to_values(wb, c, "xnor"), (s, s), (p, p))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

def check_all_ones_closed_form(lib):
    """3x3, pad 1: with all-ones weights and a non-negative input the XNOR sum
    is Cin times the in-bounds tap count (9 inside, 6 on an edge, 4 in a
    corner); all-zero weights give minus that; AND gives the count itself."""
    c, h, w = 45, 5, 6
    x = np.abs(np.random.default_rng(7).normal(size=(1, h, w, c))).astype(np.float32)
    words = (c + 31) // 32
    ones = np.full((1, 3, 3, words), 0xFFFFFFFF, np.uint32)
    zeros = np.zeros((1, 3, 3, words), np.uint32)
    taps = np.full((h, w), 9)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    a1 = _run(lib, x, ones, "xnor", 1, k=(3, 3), p=(1, 1))["acc"][0, :, :, 0]
    a0 = _run(lib, x, zeros, "xnor", 1, k=(3, 3), p=(1, 1))["acc"][0, :, :, 0]
    aa = _run(lib, x, ones, "and", 1, k=(3, 3), p=(1, 1))["acc"][0, :, :, 0]
    assert np.array_equal(a1, c * taps)
    assert np.array_equal(a0, -c * taps)
    assert np.array_equal(aa, c * taps)


def check_beta_constant_input(lib):
    """Constant post-affine input v: A = |v| everywhere; beta = |v| inside,
    6|v|/9 on edges and 4|v|/9 in corners for 3x3 pad 1; |v| everywhere for
    pad 0 and for the FC shape.  The affine (x*2 - 3 on x = 0.25) runs before
    A, as the input-terms paragraph orders it."""
    h, w, c = 6, 7, 37
    x = np.full((2, h, w, c), 0.25, np.float32)
    isc = np.full(c, 2.0, np.float32)
    ib = np.full(c, -3.0, np.float32)
    v = abs(0.25 * 2.0 - 3.0)
    wb = _rand_bits(_rng(8), (3, 3, 3, 2))
    r = _run(lib, x, wb, "xnor", 3, k=(3, 3), p=(1, 1), use_beta=True, input_scale=isc,
             input_bias=ib)
    np.testing.assert_allclose(r["a_map"], v, rtol=1e-15)
    want = np.full((h, w), 9.0)
    want[0, :] = want[-1, :] = 6.0
    want[:, 0] = want[:, -1] = 6.0
    want[0, 0] = want[0, -1] = want[-1, 0] = want[-1, -1] = 4.0
    np.testing.assert_allclose(r["beta"][0], v * want / 9.0, rtol=1e-15)
    np.testing.assert_allclose(r["beta"][1], v * want / 9.0, rtol=1e-15)
    r0 = _run(lib, x, wb, "and", 3, k=(3, 3), p=(0, 0), use_beta=True, input_scale=isc,
              input_bias=ib)
    np.testing.assert_allclose(r0["beta"], v, rtol=1e-15)
    wfc = _rand_bits(_rng(9), (2, h, w, 2))
    rfc = _run(lib, x, wfc, "binary_weights", 2, k=(h, w), use_beta=True, input_scale=isc,
               input_bias=ib)
    np.testing.assert_allclose(rfc["beta"], v, rtol=1e-15)


def check_beta_valid_taps(lib):
    """The valid-tap reading of beta's divisor (the other reading of the first
    beta equation where the window leaves the image): a mean of A over the
    window's in-image taps.
    - constant post-affine input v: beta = |v| at every position, corners and
      edges included, for odd and even kernels, strides 1 and 2;
    - a 1 x 2 image whose pixels have A = 1 and 3 under a 3x3 window, pad 1:
      both windows see both pixels, so beta = (1 + 3) / 2 = 2 (the kh*kw
      divisor gives 4/9); a single-pixel image gives beta = A of that pixel;
    - windows inside the image read the same beta under both divisors."""
    c = 37
    isc, ib = np.full(c, 2.0, np.float32), np.full(c, -3.0, np.float32)
    v = abs(0.25 * 2.0 - 3.0)
    for (h, w), k, st, p, pe in [((6, 7), 3, 1, 1, 1), ((6, 7), 4, 1, 2, 1), ((7, 9), 2, 2, 1, 0),
                                 ((9, 8), 5, 2, 2, 2), ((5, 5), 1, 1, 0, 0)]:
        x = np.full((2, h, w, c), 0.25, np.float32)
        wb = _rand_bits(_rng(41), (3, k, k, 2))
        r = _run(lib, x, wb, "xnor", 3, k=(k, k), s=(st, st), p=(p, p), pad_end=(pe, pe), use_beta=True,
                 beta_divisor="valid", input_scale=isc, input_bias=ib)
        np.testing.assert_allclose(r["beta"], v, rtol=1e-15, err_msg=f"k{k} s{st} pad {p}/{pe}")
    x = np.empty((1, 1, 2, 4), np.float32)
    x[0, 0, 0] = [1.0, -1.0, 1.0, -1.0]   # A = 1
    x[0, 0, 1] = [3.0, -3.0, -3.0, 3.0]   # A = 3
    wb = _rand_bits(_rng(42), (2, 3, 3, 1))
    r = _run(lib, x, wb, "and", 2, k=(3, 3), p=(1, 1), use_beta=True, beta_divisor="valid")
    np.testing.assert_allclose(r["beta"][0, 0], [2.0, 2.0], rtol=1e-15)
    r9 = _run(lib, x, wb, "and", 2, k=(3, 3), p=(1, 1), use_beta=True)
    np.testing.assert_allclose(r9["beta"][0, 0], [4.0 / 9.0, 4.0 / 9.0], rtol=1e-15)
    r1 = _run(lib, x[:, :, :1], wb, "binary_weights", 2, k=(3, 3), p=(1, 1), use_beta=True,
              beta_divisor="valid")
    np.testing.assert_allclose(r1["beta"][0, 0, 0], 1.0, rtol=1e-15)
    rng = _rng(43)
    x = rng.normal(size=(2, 6, 8, 33)).astype(np.float32)
    wb = _rand_bits(rng, (4, 3, 3, 2))
    rv = _run(lib, x, wb, "xnor", 4, k=(3, 3), p=(1, 1), use_beta=True, beta_divisor="valid")
    rw = _run(lib, x, wb, "xnor", 4, k=(3, 3), p=(1, 1), use_beta=True)
    np.testing.assert_array_equal(rv["beta"][:, 1:-1, 1:-1], rw["beta"][:, 1:-1, 1:-1])
    np.testing.assert_array_equal(rv["acc"], rw["acc"])
    assert not np.array_equal(rv["beta"], rw["beta"])


def check_a_map_definition(lib):
    """A is the mean over channels of |x'| (Nc = Cin, not the padded word
    width), checked with float64 numpy on a random input and affine."""
    rng = _rng(10)
    x = rng.normal(size=(2, 4, 5, 45)).astype(np.float32)
    isc = rng.uniform(0.5, 1.5, 45).astype(np.float32)
    ib = rng.normal(0, 0.2, 45).astype(np.float32)
    r = _run(lib, x, _rand_bits(rng, (2, 3, 3, 2)), "xnor", 2, k=(3, 3), p=(1, 1),
             use_beta=True, input_scale=isc, input_bias=ib)
    xp = np.array([[float(_fma_f32(a, s, b)) for a, s, b in zip(px, isc, ib)]
                   for px in x.reshape(-1, 45)])
    want = np.abs(xp).sum(axis=1) / 45.0
    np.testing.assert_allclose(r["a_map"].ravel(), want, rtol=1e-13)


def check_epilogue_closed_form(lib):
    """Cin = 1, 1x1: acc = +-1, so out = acc*scale*beta + bias by hand, with
    ReLU clamping negatives; a missing output scale uses scale_value and a
    missing bias is 0."""
    x = np.array([2.0, -3.0, 0.5, -0.25], np.float32).reshape(1, 2, 2, 1)
    wb = np.array([1, 0], np.uint32).reshape(2, 1, 1, 1)
    sc = np.array([1.5, 0.75], np.float32)
    bi = np.array([-0.5, 0.25], np.float32)
    sign = np.array([1, -1, 1, -1]).reshape(2, 2)
    wv = np.array([1, -1])
    r = _run(lib, x, wb, "xnor", 2, output_scale=sc, output_bias=bi, neuron="none")
    acc = sign[:, :, None] * wv[None, None, :]
    want = acc * sc.astype(np.float64) + bi.astype(np.float64)
    np.testing.assert_array_equal(r["out"][0], want)
    rr = _run(lib, x, wb, "xnor", 2, output_scale=sc, output_bias=bi, neuron="relu")
    np.testing.assert_array_equal(rr["out"][0], np.maximum(want, 0.0))
    rs = _run(lib, x, wb, "xnor", 2, scale_value=2.5)
    np.testing.assert_array_equal(rs["out"][0], acc * 2.5)
    # with beta on a 1x1 window, beta = A = |x'| of that pixel
    rb = _run(lib, x, wb, "xnor", 2, output_scale=sc, output_bias=bi, use_beta=True)
    absx = np.abs(x[0, :, :, 0].astype(np.float64))
    np.testing.assert_allclose(rb["out"][0], acc * sc * absx[:, :, None] + bi, rtol=1e-15)


# ------------------------------------------------------------------ neurons

_NEURON_RS = np.array([-6.0, -2.5, -1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0, 2.5, 6.0])


def _neuron_outputs(lib, neuron, a=0.0, b=0.0, rs=_NEURON_RS):
    """Outputs of a 1x1 XNOR layer with Cin = 1 whose pre-activation values are
    exactly `rs`: input +1, weight bits 1 (acc = +1), scale 1, bias r - 1."""
    o = len(rs)
    bias = (rs - 1.0).astype(np.float32)
    assert np.array_equal(bias.astype(np.float64) + 1.0, rs)
    r = _run(lib, np.ones((1, 1, 1, 1), np.float32), np.ones((o, 1, 1, 1), np.uint32), "xnor", o,
             output_scale=np.ones(o, np.float32), output_bias=bias, neuron=neuron, neuron_a=a, neuron_b=b)
    return r["out"][0, 0, 0]


def check_neuron_closed_forms(lib):
    """Piecewise-linear and rational activations on exactly representable
    pre-activation values, against hand-computed results."""
    rs = _NEURON_RS
    np.testing.assert_array_equal(_neuron_outputs(lib, "none"), rs)
    np.testing.assert_array_equal(_neuron_outputs(lib, "relu"), [0, 0, 0, 0, 0, 0, 0.25, 0.5, 1, 2.5, 6])
    np.testing.assert_array_equal(_neuron_outputs(lib, "leaky_relu", a=0.125),
                                  [-0.75, -0.3125, -0.125, -0.0625, -0.03125, 0, 0.25, 0.5, 1, 2.5, 6])
    np.testing.assert_array_equal(_neuron_outputs(lib, "linear", a=2.0, b=-0.5),
                                  [-12.5, -5.5, -2.5, -1.5, -1, -0.5, 0, 0.5, 1.5, 4.5, 11.5])
    np.testing.assert_array_equal(_neuron_outputs(lib, "absolute"), [6, 2.5, 1, 0.5, 0.25, 0, 0.25, 0.5, 1, 2.5, 6])
    np.testing.assert_array_equal(_neuron_outputs(lib, "hard_sigmoid", a=0.25, b=0.5),
                                  [0, 0, 0.25, 0.375, 0.4375, 0.5, 0.5625, 0.625, 0.75, 1, 1])
    np.testing.assert_array_equal(_neuron_outputs(lib, "clamp", a=-1.0, b=2.0),
                                  [-1, -1, -1, -0.5, -0.25, 0, 0.25, 0.5, 1, 2, 2])
    np.testing.assert_allclose(_neuron_outputs(lib, "softsign"),
                               [-6 / 7, -5 / 7, -1 / 2, -1 / 3, -1 / 5, 0, 1 / 5, 1 / 3, 1 / 2, 5 / 7, 6 / 7],
                               rtol=1e-15, atol=0)


def check_neuron_identities(lib):
    """The exponential activations through identities that need no math
    library: sigmoid(0) = 1/2 and sigmoid(r) + sigmoid(-r) = 1; a*tanh(b*r) =
    a*(2*sigmoid(2*b*r) - 1); softplus(0) = a*ln 2 and
    softplus(r) - softplus(-r) = a*b*r; elu(r) = a*(e^r - 1) for r < 0 with
    e^r = sigmoid(r) / (1 - sigmoid(r))."""
    rs = _NEURON_RS
    s = _neuron_outputs(lib, "sigmoid")
    assert s[rs == 0][0] == 0.5
    np.testing.assert_allclose(s + s[::-1], 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(s) > 0) and np.all((s > 0) & (s < 1))
    t = _neuron_outputs(lib, "tanh", a=2.0, b=0.5)   # 2*b*r = r
    np.testing.assert_allclose(t, 2.0 * (2.0 * s - 1.0), rtol=0, atol=1e-14)
    sp = _neuron_outputs(lib, "softplus", a=1.5, b=2.0)
    np.testing.assert_allclose(sp[rs == 0][0], 1.5 * 0.6931471805599453, rtol=1e-15)
    np.testing.assert_allclose(sp - sp[::-1], 3.0 * rs, rtol=0, atol=1e-13)
    assert np.all(sp > 0)
    e = _neuron_outputs(lib, "elu", a=0.5)
    neg = rs < 0
    np.testing.assert_array_equal(e[~neg], rs[~neg])
    np.testing.assert_allclose(e[neg], 0.5 * (s[neg] / (1.0 - s[neg]) - 1.0), rtol=1e-13, atol=0)


# -------------------------------------------------------------- sign / affine

def _fma_f32(x, s, b) -> np.float32:
    """Correctly rounded float32 of the exact x*s + b (ties to even)."""
    exact = Fraction(float(x)) * Fraction(float(s)) + Fraction(float(b))
    f = np.float32(float(exact))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        err = abs(Fraction(float(cand)) - exact)
        key = (err, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def check_sign_under_affine(lib):
    """The binarised value is the sign of the exact s*x + b (one rounding keeps
    the sign), with zero counted as +1; adversarial x sit next to -b/s, and
    signed zeros, subnormals and a NaN are included.  A one-hot AND weight
    word reads channel j's 0/1 value alone.  binaryWeights with Cin = 1
    returns x' itself, the correctly rounded fused product-sum."""
    rng = _rng(11)
    c = 24
    s = rng.uniform(0.5, 1.5, c).astype(np.float32)
    b = rng.normal(0, 0.2, c).astype(np.float32)
    xs = []
    for j in range(c):
        root = np.float32(-b[j] / s[j])
        cand = [root, np.nextafter(root, np.float32(1)), np.nextafter(root, np.float32(-1))]
        xs.append(cand[j % 3])
    x = np.array(xs, np.float32).reshape(1, 1, 1, c)
    x2 = np.array([0.0, -0.0, np.nan, 1e-40, -1e-40, -1e-30, 1e-30, 3.0],
                  np.float32).reshape(1, 1, 1, -1)
    for xin, sc, bi in ((x, s, b), (x2, None, None)):
        cc = xin.shape[-1]
        onehot = np.array([1 << j for j in range(cc)], np.uint32).reshape(cc, 1, 1, 1)
        acc = _run(lib, xin, onehot, "and", cc, input_scale=sc, input_bias=bi)["acc"][0, 0, 0]
        for j in range(cc):
            xv = float(xin[0, 0, 0, j])
            if np.isnan(xv):
                want = 1
            elif sc is None:
                want = 0 if xv < 0 else 1
            else:
                exact = Fraction(xv) * Fraction(float(sc[j])) + Fraction(float(bi[j]))
                want = 0 if exact < 0 else 1
            assert acc[j] == want, (j, xv, acc[j], want)
    for j in range(c):
        xi = x[:, :, :, j:j + 1]
        r = _run(lib, xi, np.ones((1, 1, 1, 1), np.uint32), "binary_weights", 1,
                 input_scale=s[j:j + 1], input_bias=b[j:j + 1])["acc"][0, 0, 0, 0]
        assert r == float(_fma_f32(xi[0, 0, 0, 0], s[j], b[j])), j


def check_tail_bits_ignored(lib):
    """Cin not a multiple of 32: weight bits at channel positions >= Cin never
    change the result (all forms)."""
    rng = _rng(12)
    for c in (1, 5, 31, 33, 45, 63):
        words = (c + 31) // 32
        x = rng.normal(size=(1, 4, 4, c)).astype(np.float32)
        wb = _rand_bits(rng, (3, 3, 3, words))
        clean = wb.copy()
        tail = c % 32
        if tail:
            clean[..., -1] &= np.uint32((1 << tail) - 1)
        for form in ("xnor", "and", "binary_weights"):
            a = _run(lib, x, wb, form, 3, k=(3, 3), p=(1, 1))["acc"]
            b_ = _run(lib, x, clean, form, 3, k=(3, 3), p=(1, 1))["acc"]
            assert np.array_equal(a, b_), (c, form)


def check_degenerate_single_channel(lib):
    """Cin = 1, 1x1 kernel: the XNOR sum is the product of the two signs; AND
    is 1 only when both are 1."""
    x = np.array([-1.5, 0.0, 2.0, -0.0], np.float32).reshape(1, 1, 4, 1)
    wb = np.array([0, 1], np.uint32).reshape(2, 1, 1, 1)
    sx = np.array([-1, 1, 1, 1])
    acc = _run(lib, x, wb, "xnor", 2)["acc"][0, 0]
    assert np.array_equal(acc, np.stack([sx * -1, sx * 1], axis=1))
    acca = _run(lib, x, wb, "and", 2)["acc"][0, 0]
    assert np.array_equal(acca, np.stack([sx * 0, (sx > 0).astype(int)], axis=1))


def check_accumulator_parity_and_range(lib):
    """XNOR sums lie in [-Kv, Kv] with the parity of Kv, AND sums in [0, Kv],
    where Kv = Cin times the in-bounds tap count."""
    rng = _rng(13)
    c, h, w = 37, 6, 5
    x = rng.normal(size=(2, h, w, c)).astype(np.float32)
    wb = _rand_bits(rng, (4, 3, 3, 2))
    taps = np.ones((1, h, w, 1), np.float32)
    kv = c * np.rint(conv2d_ref(taps.astype(np.float64), np.ones((1, 3, 3, 1)), (1, 1), (1, 1)))
    ax = _run(lib, x, wb, "xnor", 4, k=(3, 3), p=(1, 1))["acc"]
    aa = _run(lib, x, wb, "and", 4, k=(3, 3), p=(1, 1))["acc"]
    assert np.all(np.abs(ax) <= kv) and np.all((ax - kv) % 2 == 0)
    assert np.all(aa >= 0) and np.all(aa <= kv)


ALL_CHECKS = [
    check_truth_table, check_word_identities, check_word_ranges, check_fc_conditions_and_matmul,
    check_fc_equals_centred_conv, check_beta_window, check_centred_window_any_kernel, check_bruteforce_conv,
    check_bruteforce_asymmetric_padding,
    check_binary_weights_conv, check_all_ones_closed_form, check_beta_constant_input,
    check_a_map_definition, check_epilogue_closed_form, check_sign_under_affine,
    check_tail_bits_ignored, check_degenerate_single_channel,
    check_accumulator_parity_and_range, check_neuron_closed_forms, check_neuron_identities,
    check_beta_valid_taps,
]
