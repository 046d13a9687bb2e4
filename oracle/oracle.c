/*
 * Plain, slow CPU oracle of binary convolution.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * It is the definition of the method written out, with no bit packing, no
 * popcount and no blocking: the input is turned into a tensor of +-1 (or 0/1)
 * integers, the weight bits into a tensor of +-1 (or 0/1) integers, and every
 * output is a direct sum of products over the in-bounds taps of its window.
 * Page references below are to the Apple developer documentation pages
 * "MPSCNNBinaryConvolution" and "MPSCNNFullyConnected".
 *
 * Readings taken where the pages leave a step open (each is pinned by a CPU
 * test against something other than this file):
 *  - layout NHWC fp32; weights are uint32 words [Cout][kh][kw][ceil(Cin/32)]
 *    with channel c at bit c%32 of word c/32 (the pages only say "32-bit words").
 *  - geometry: ih = oh*stride - pad + ky, out = (in + pad + pad_end - k)/stride + 1,
 *    with pad the leading and pad_end the trailing zero padding (equal for the
 *    odd kernels; the pages' centred window [-k/2, (k-1)/2] of the beta
 *    paragraph gives an even kernel pad = k/2 and pad_end = k/2 - 1).
 *  - padded taps contribute nothing to the sum.
 *  - input affine x' = fmaf(x, inputScale[c], inputBias[c]) in fp32, applied
 *    before the sign and before the A map.
 *  - sign: x' < 0 -> -1 (XNOR) / 0 (AND), otherwise +1 / 1, by IEEE compare
 *    (so -0 and NaN give +1).
 *  - beta divides the window sum of A by kh*kw, out-of-image taps adding 0;
 *    the other reading of that divisor, the count of in-image taps, is
 *    use_beta = 2.
 *  - missing output scale -> scale_value; missing biases -> 0; missing input
 *    scale -> 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Operator forms of MPSCNNBinaryConvolution, Overview, the three type bullets. */
#define ORACLE_BINARY_WEIGHTS 0
#define ORACLE_XNOR 1
#define ORACLE_AND 2

/* Activation applied last (MPSCNNBinaryConvolution, Overview, closing
 * sentence: "the normal activation neuron").  The page names no set; these
 * are the usual element-wise activations, with parameters a and b. */
#define ORACLE_NEURON_NONE 0
#define ORACLE_NEURON_RELU 1
#define ORACLE_NEURON_LEAKY_RELU 2
#define ORACLE_NEURON_LINEAR 3
#define ORACLE_NEURON_SIGMOID 4
#define ORACLE_NEURON_HARD_SIGMOID 5
#define ORACLE_NEURON_TANH 6
#define ORACLE_NEURON_ABSOLUTE 7
#define ORACLE_NEURON_SOFTPLUS 8
#define ORACLE_NEURON_SOFTSIGN 9
#define ORACLE_NEURON_ELU 10
#define ORACLE_NEURON_CLAMP 11
#define ORACLE_NEURON_COUNT 12

/* Each activation from its definition, in double:
 *   relu        r < 0 ? 0 : r              leaky_relu  r < 0 ? a*r : r
 *   linear      a*r + b                    sigmoid     1 / (1 + e^-r)
 *   hard_sigmoid min(max(a*r + b, 0), 1)   tanh        a * tanh(b*r)
 *   absolute    |r|                        softplus    a * log(1 + e^(b*r))
 *   softsign    r / (1 + |r|)              elu         r < 0 ? a*(e^r - 1) : r
 *   clamp       min(max(r, a), b)
 * softplus is evaluated as max(z, 0) + log1p(e^-|z|), the same function
 * without overflow of e^z. */
static double neuron_value(int neuron, double a, double b, double r)
{
    switch (neuron) {
    case ORACLE_NEURON_RELU: return r < 0.0 ? 0.0 : r;
    case ORACLE_NEURON_LEAKY_RELU: return r < 0.0 ? a * r : r;
    case ORACLE_NEURON_LINEAR: return a * r + b;
    case ORACLE_NEURON_SIGMOID: return 1.0 / (1.0 + exp(-r));
    case ORACLE_NEURON_HARD_SIGMOID: return fmin(fmax(a * r + b, 0.0), 1.0);
    case ORACLE_NEURON_TANH: return a * tanh(b * r);
    case ORACLE_NEURON_ABSOLUTE: return fabs(r);
    case ORACLE_NEURON_SOFTPLUS: {
        const double z = b * r;
        return a * (fmax(z, 0.0) + log1p(exp(-fabs(z))));
    }
    case ORACLE_NEURON_SOFTSIGN: return r / (1.0 + fabs(r));
    case ORACLE_NEURON_ELU: return r < 0.0 ? a * expm1(r) : r;
    case ORACLE_NEURON_CLAMP: return fmin(fmax(r, a), b);
    default: return r;
    }
}

int oracle_out_dim2(int in, int k, int stride, int pad, int pad_end)
{
    if (stride <= 0 || k <= 0 || in + pad + pad_end < k) return 0;
    return (in + pad + pad_end - k) / stride + 1;
}

int oracle_out_dim(int in, int k, int stride, int pad) { return oracle_out_dim2(in, k, stride, pad, pad); }

/*
 * Input pre-offset and scale (MPSCNNBinaryConvolution, Overview, paragraph on
 * inputBiasTerms / inputScaleTerms): per input channel, before binarisation
 * and before the beta image.  One fp32 fused multiply-add per element.
 */
static void input_affine(long pixels, int in_c, const float *x, const float *input_scale,
                         const float *input_bias, float *xp)
{
    for (long p = 0; p < pixels; ++p) {
        for (int c = 0; c < in_c; ++c) {
            float v = x[p * in_c + c];
            if (input_scale || input_bias) {
                float s = input_scale ? input_scale[c] : 1.0f;
                float b = input_bias ? input_bias[c] : 0.0f;
                v = fmaf(v, s, b);
            }
            xp[p * in_c + c] = v;
        }
    }
}

/*
 * Value of one weight (MPSCNNBinaryConvolution, Overview, symbol definitions
 * and type bullets): bit 1 is +1 and bit 0 is -1 for XNOR and binaryWeights;
 * for AND the bit itself (0 or 1) is the value.
 */
static int weight_value(const uint32_t *weight_bits, int words, int co, int ky, int kx,
                        int kernel_h, int kernel_w, int c, int type)
{
    long word_index = (((long)co * kernel_h + ky) * kernel_w + kx) * words + c / 32;
    int bit = (int)((weight_bits[word_index] >> (c % 32)) & 1u);
    if (type == ORACLE_AND) return bit;
    return bit ? 1 : -1;
}

/*
 * Binarised input (MPSCNNBinaryConvolution, Overview, XNOR and AND bullets):
 * the sign function gives -1 for x < 0 and +1 otherwise; under AND the two
 * values are read as 0 and 1.
 */
static int input_sign(float v, int type)
{
    if (type == ORACLE_AND) return (v < 0.0f) ? 0 : 1;
    return (v < 0.0f) ? -1 : 1;
}

/*
 * The whole forward pass, following the output equation of
 * MPSCNNBinaryConvolution (Overview):
 *   out = neuron( (sum over window taps and channels of in (x) B) * scale[c]
 *                 * beta[i,x,y] + bias[c] )
 * The fully connected layer of MPSCNNFullyConnected is the same call with a
 * kernel the size of the source image, stride 1 and no padding.
 *
 * Outputs (every pointer but `out` may be NULL):
 *   out       double [n][oh][ow][out_c]   final values
 *   acc_int   int32  [n][oh][ow][out_c]   XNOR/AND sum before the epilogue
 *   acc_real  double [n][oh][ow][out_c]   binaryWeights sum before the epilogue
 *   signs     int8   [n][in_h][in_w][in_c] binarised input (XNOR/AND)
 *   a_map     double [n][in_h][in_w]      A map (only with use_beta)
 *   beta      double [n][oh][ow]          beta image (1 when use_beta is 0)
 * Returns 0, or -1 on an argument the method does not define.
 */
int oracle_bconv(int n, int in_h, int in_w, int in_c, int out_c, int kernel_h, int kernel_w,
                 int stride_h, int stride_w, int pad_h, int pad_w, int pad_h_end, int pad_w_end,
                 int type, int use_beta,
                 int neuron, float scale_value, float neuron_a, float neuron_b, const float *x,
                 const uint32_t *weight_bits,
                 const float *output_scale, const float *output_bias, const float *input_scale,
                 const float *input_bias, double *out, int32_t *acc_int, double *acc_real,
                 int8_t *signs, double *a_map, double *beta, int n_threads)
{
    if (n < 0 || in_h <= 0 || in_w <= 0 || in_c <= 0 || out_c <= 0 || kernel_h <= 0 ||
        kernel_w <= 0 || stride_h <= 0 || stride_w <= 0 || pad_h < 0 || pad_w < 0 || pad_h_end < 0 ||
        pad_w_end < 0)
        return -1;
    if (type != ORACLE_BINARY_WEIGHTS && type != ORACLE_XNOR && type != ORACLE_AND) return -1;
    if (neuron < 0 || neuron >= ORACLE_NEURON_COUNT) return -1;
    if (!x || !weight_bits || !out) return -1;

    const int out_h = oracle_out_dim2(in_h, kernel_h, stride_h, pad_h, pad_h_end);
    const int out_w = oracle_out_dim2(in_w, kernel_w, stride_w, pad_w, pad_w_end);
    if (out_h <= 0 || out_w <= 0) return -1;
    const int words = (in_c + 31) / 32;
    const long in_pixels = (long)n * in_h * in_w;
    const long in_elems = in_pixels * in_c;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    /* Step 1: input affine, in fp32. */
    float *xp = (float *)malloc(sizeof(float) * (size_t)(in_elems > 0 ? in_elems : 1));
    if (!xp) return -1;
    input_affine(in_pixels, in_c, x, input_scale, input_bias, xp);

    /* Step 2: the operand each form multiplies: +-1 / 0,1 integers for
     * XNOR / AND, the full-precision value for binaryWeights. */
    int8_t *s = (int8_t *)malloc((size_t)(in_elems > 0 ? in_elems : 1));
    double *xd = (double *)malloc(sizeof(double) * (size_t)(in_elems > 0 ? in_elems : 1));
    /* Step 3: the weights as small integers, [out_c][kh][kw][in_c]. */
    const long w_elems = (long)out_c * kernel_h * kernel_w * in_c;
    int8_t *wv = (int8_t *)malloc((size_t)w_elems);
    double *bw = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? (long)n * out_h * out_w : 1));
    double *am = (double *)malloc(sizeof(double) * (size_t)(in_pixels > 0 ? in_pixels : 1));
    if (!s || !xd || !wv || !bw || !am) {
        free(xp); free(s); free(xd); free(wv); free(bw); free(am);
        return -1;
    }
    for (long i = 0; i < in_elems; ++i) {
        s[i] = (int8_t)input_sign(xp[i], type);
        xd[i] = (double)xp[i];
    }
    if (signs && type != ORACLE_BINARY_WEIGHTS) memcpy(signs, s, (size_t)in_elems);
    for (int co = 0; co < out_c; ++co)
        for (int ky = 0; ky < kernel_h; ++ky)
            for (int kx = 0; kx < kernel_w; ++kx)
                for (int c = 0; c < in_c; ++c)
                    wv[(((long)co * kernel_h + ky) * kernel_w + kx) * in_c + c] = (int8_t)
                        weight_value(weight_bits, words, co, ky, kx, kernel_h, kernel_w, c, type);

    /* Step 4: the A map and the beta image (MPSCNNBinaryConvolution,
     * Overview, the two beta equations): A is the mean absolute value over
     * channels of the full-precision (post-affine) input; beta is the sum of A
     * over the convolution window divided by kh*kw (use_beta 1) or, in the
     * other reading of that divisor where the window leaves the image, by the
     * number of in-image taps (use_beta 2).  Without the flag beta is 1. */
    for (long p = 0; p < in_pixels; ++p) {
        double sum = 0.0;
        for (int c = 0; c < in_c; ++c) sum += fabs(xd[p * in_c + c]);
        am[p] = sum / (double)in_c;
    }
    for (int i = 0; i < n; ++i)
        for (int oy = 0; oy < out_h; ++oy)
            for (int ox = 0; ox < out_w; ++ox) {
                double b = 1.0;
                if (use_beta) {
                    double sum = 0.0;
                    int valid = 0;
                    for (int ky = 0; ky < kernel_h; ++ky) {
                        int iy = oy * stride_h - pad_h + ky;
                        if (iy < 0 || iy >= in_h) continue;
                        for (int kx = 0; kx < kernel_w; ++kx) {
                            int ix = ox * stride_w - pad_w + kx;
                            if (ix < 0 || ix >= in_w) continue;
                            sum += am[((long)i * in_h + iy) * in_w + ix];
                            ++valid;
                        }
                    }
                    b = sum / (double)(use_beta == 2 ? valid : kernel_h * kernel_w);
                }
                bw[((long)i * out_h + oy) * out_w + ox] = b;
            }
    if (a_map && use_beta) memcpy(a_map, am, sizeof(double) * (size_t)in_pixels);
    if (beta) memcpy(beta, bw, sizeof(double) * (size_t)((long)n * out_h * out_w));

    /* Step 5: the window sums and the epilogue. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int i = 0; i < n; ++i) {
        for (int oy = 0; oy < out_h; ++oy) {
            for (int ox = 0; ox < out_w; ++ox) {
                for (int co = 0; co < out_c; ++co) {
                    int32_t acc = 0;
                    double accd = 0.0;
                    for (int ky = 0; ky < kernel_h; ++ky) {
                        int iy = oy * stride_h - pad_h + ky;
                        if (iy < 0 || iy >= in_h) continue; /* padded tap: nothing */
                        for (int kx = 0; kx < kernel_w; ++kx) {
                            int ix = ox * stride_w - pad_w + kx;
                            if (ix < 0 || ix >= in_w) continue; /* padded tap: nothing */
                            const long xo = (((long)i * in_h + iy) * in_w + ix) * in_c;
                            const long wo = (((long)co * kernel_h + ky) * kernel_w + kx) * in_c;
                            if (type == ORACLE_BINARY_WEIGHTS) {
                                for (int c = 0; c < in_c; ++c) accd += xd[xo + c] * (double)wv[wo + c];
                            } else {
                                for (int c = 0; c < in_c; ++c) acc += (int32_t)s[xo + c] * (int32_t)wv[wo + c];
                            }
                        }
                    }
                    const long oo = (((long)i * out_h + oy) * out_w + ox) * out_c + co;
                    double v = (type == ORACLE_BINARY_WEIGHTS) ? accd : (double)acc;
                    if (acc_int) acc_int[oo] = acc;
                    if (acc_real) acc_real[oo] = accd;
                    double scale = output_scale ? (double)output_scale[co] : (double)scale_value;
                    double bias = output_bias ? (double)output_bias[co] : 0.0;
                    const double r = v * scale * bw[((long)i * out_h + oy) * out_w + ox] + bias;
                    out[oo] = neuron_value(neuron, (double)neuron_a, (double)neuron_b, r);
                }
            }
        }
    }

    free(xp); free(s); free(xd); free(wv); free(bw); free(am);
    return 0;
}
