/*
 * Packed-bit CPU baseline of XNOR / AND binary convolution.
 *
 * TEST AND BENCHMARK INFRASTRUCTURE, like the oracle beside it: a reference
 * point for what a CPU does with the packed method, loaded only by the tests
 * (which check it against the oracle) and by the benchmark's CPU leg.  The HIP
 * library never calls it and shares no code with it.
 *
 * The method in the form the "Bitwise XNOR" glossary page describes for
 * CPUs (the XNOR-Net decomposition: XNOR of packed words, then a population
 * count): the input is binarised and packed 32 channels per word, and a
 * window sum is a sum of popcount(x ^ w) (XNOR; value Cin*taps - 2*count,
 * the MPSCNNBinaryConvolution XNOR bullet) or popcount(x & w) (AND bullet)
 * over the window's in-image taps.  Portable C: __builtin_popcount, no SIMD
 * intrinsics, OpenMP over output rows.  Geometry, input affine, sign, beta
 * and epilogue follow the same readings as the oracle (fp32 epilogue here).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PACKED_XNOR 1
#define PACKED_AND 2
#define PACKED_NEURON_NONE 0
#define PACKED_NEURON_RELU 1

static int out_dim(int in, int k, int s, int p, int pe)
{
    if (s <= 0 || k <= 0 || in + p + pe < k) return 0;
    return (in + p + pe - k) / s + 1;
}

/*
 * Forward pass for XNOR / AND with neuron none or ReLU.  Shapes, pointers
 * and use_beta (0, 1: / kh*kw, 2: / in-image taps) as for oracle_bconv;
 * `out` fp32 [n][oh][ow][out_c], `acc_out`
 * (may be NULL) int32 window sums.  Returns 0, or -1 on arguments outside
 * this baseline's scope.
 */
int packed_bconv(int n, int in_h, int in_w, int in_c, int out_c, int kh, int kw, int sh, int sw, int ph, int pw,
                 int phe, int pwe, int type, int use_beta, int neuron, float scale_value, const float *x,
                 const uint32_t *weight_bits, const float *output_scale, const float *output_bias,
                 const float *input_scale, const float *input_bias, float *out, int32_t *acc_out, int n_threads)
{
    if (n < 0 || in_h <= 0 || in_w <= 0 || in_c <= 0 || out_c <= 0 || kh <= 0 || kw <= 0 || sh <= 0 || sw <= 0 ||
        ph < 0 || pw < 0 || phe < 0 || pwe < 0)
        return -1;
    if (type != PACKED_XNOR && type != PACKED_AND) return -1;
    if (neuron != PACKED_NEURON_NONE && neuron != PACKED_NEURON_RELU) return -1;
    if (!x || !weight_bits || !out) return -1;
    const int oh = out_dim(in_h, kh, sh, ph, phe), ow = out_dim(in_w, kw, sw, pw, pwe);
    if (oh <= 0 || ow <= 0) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const int words = (in_c + 31) / 32;
    const long pixels = (long)n * in_h * in_w;
    const int taps = kh * kw;
    uint32_t *bits = (uint32_t *)calloc((size_t)(pixels * words), sizeof(uint32_t));
    float *amap = use_beta ? (float *)malloc(sizeof(float) * (size_t)(pixels > 0 ? pixels : 1)) : NULL;
    uint32_t *wm = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)out_c * taps * words);
    if (!bits || !wm || (use_beta && !amap)) {
        free(bits); free(amap); free(wm);
        return -1;
    }
    /* weight words with the bits past in_c cleared */
    const uint32_t tail = (in_c % 32) ? ((1u << (in_c % 32)) - 1u) : 0xffffffffu;
    for (long i = 0; i < (long)out_c * taps; ++i)
        for (int w = 0; w < words; ++w)
            wm[i * words + w] = weight_bits[i * words + w] & (w == words - 1 ? tail : 0xffffffffu);

    /* binarise and pack: bit = !(x' < 0), x' = fmaf(x, s, b); A = mean |x'| */
#pragma omp parallel for schedule(static)
    for (long p = 0; p < pixels; ++p) {
        const float *xp = x + p * in_c;
        uint32_t *bp = bits + p * words;
        double asum = 0.0;
        for (int c = 0; c < in_c; ++c) {
            float v = xp[c];
            if (input_scale || input_bias)
                v = fmaf(v, input_scale ? input_scale[c] : 1.0f, input_bias ? input_bias[c] : 0.0f);
            if (!(v < 0.0f)) bp[c / 32] |= 1u << (c % 32);
            asum += fabs((double)v);
        }
        if (amap) amap[p] = (float)(asum / in_c);
    }

    const int wpt = words;  /* words per tap */
#pragma omp parallel
    {
        uint32_t *xw = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)taps * wpt);
        int *tw = (int *)malloc(sizeof(int) * (size_t)taps);
#pragma omp for schedule(static)
        for (long row = 0; row < (long)n * oh; ++row) {
            const int img = (int)(row / oh), oy = (int)(row % oh);
            for (int ox = 0; ox < ow; ++ox) {
                /* gather the window's in-image words and their tap numbers */
                int valid = 0;
                double bsum = 0.0;
                for (int ky = 0; ky < kh; ++ky) {
                    const int iy = oy * sh - ph + ky;
                    if (iy < 0 || iy >= in_h) continue;
                    for (int kx = 0; kx < kw; ++kx) {
                        const int ix = ox * sw - pw + kx;
                        if (ix < 0 || ix >= in_w) continue;
                        const long p = ((long)img * in_h + iy) * in_w + ix;
                        memcpy(xw + (size_t)valid * wpt, bits + p * words, sizeof(uint32_t) * wpt);
                        tw[valid] = ky * kw + kx;
                        if (amap) bsum += amap[p];
                        ++valid;
                    }
                }
                const float be = amap ? (float)(bsum / (use_beta == 2 ? valid : taps)) : 1.0f;
                const long o = (((long)img * oh + oy) * ow + ox) * out_c;
                for (int co = 0; co < out_c; ++co) {
                    const uint32_t *wc = wm + (size_t)co * taps * wpt;
                    int cnt = 0;
                    for (int t = 0; t < valid; ++t) {
                        const uint32_t *a = xw + (size_t)t * wpt, *b = wc + (size_t)tw[t] * wpt;
                        if (type == PACKED_XNOR)
                            for (int w = 0; w < wpt; ++w) cnt += __builtin_popcount(a[w] ^ b[w]);
                        else
                            for (int w = 0; w < wpt; ++w) cnt += __builtin_popcount(a[w] & b[w]);
                    }
                    /* XNOR: padded tail bits agree (0 ^ 0), so the count is of disagreeing channels */
                    const int v = type == PACKED_XNOR ? in_c * valid - 2 * cnt : cnt;
                    if (acc_out) acc_out[o + co] = v;
                    const float sc = output_scale ? output_scale[co] : scale_value;
                    const float bi = output_bias ? output_bias[co] : 0.0f;
                    float r = fmaf((float)v * sc, be, bi);
                    if (neuron == PACKED_NEURON_RELU && r < 0.0f) r = 0.0f;
                    out[o + co] = r;
                }
            }
        }
        free(xw);
        free(tw);
    }
    free(bits); free(amap); free(wm);
    return 0;
}
