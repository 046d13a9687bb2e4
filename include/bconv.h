/*
 * bconv.h -- binary convolution on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbconv.so.  The operation is the one defined on Apple's
 * "MPSCNNBinaryConvolution" documentation page (Overview, output equation):
 *
 *   out[i,y,x,c] = neuron( (sum over the window taps (ky,kx) and the input
 *                  channels f of  in'[i,y',x',f] (*) B[c,ky,kx,f])
 *                  * scale[c] * beta[i,y,x] + bias[c] )
 *
 * where (*) is one of the three forms of the page's type bullets:
 *   BCONV_BINARY_WEIGHTS  full-precision input times the weight read as +-1;
 *   BCONV_XNOR            input binarised by its sign, XNOR product read as
 *                         +-1 (a 32-bit word pair gives 32 - 2*popcount(x^w));
 *   BCONV_AND             input binarised, AND product read as 0/1 (a word
 *                         pair gives popcount(x & w)).
 * in' is the input after the optional per-channel input scale and bias (the
 * page's input-terms paragraph), beta is the optional box average of the
 * per-pixel mean |in'| (the page's two beta equations), and the fully
 * connected layer of Apple's "MPSCNNFullyConnected" page (Overview,
 * conditions) is the case kernel = source size, stride 1, no padding.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - Tensors are fp32, NHWC, dense: input [n][in_h][in_w][in_c], output
 *     [n][out_h][out_w][out_c].  x indexes width, y height.
 *   - Weight bits are uint32 words [out_c][kernel_h][kernel_w][ceil(in_c/32)];
 *     input channel f is bit (f % 32) of word (f / 32).  Bit 1 is +1 (XNOR,
 *     binaryWeights) or 1 (AND); bit 0 is -1 or 0.  Bits at positions >= in_c
 *     in the last word are ignored.
 *   - Geometry: out_h = (in_h + pad_h + pad_h_end - kernel_h)/stride_h + 1
 *     (likewise w), with pad_h the leading (top) and pad_h_end the trailing
 *     (bottom) zero padding; tap ky of output y reads input row
 *     y*stride_h - pad_h + ky.  pad = kernel/2, pad_end = (kernel-1)/2 and
 *     stride 1 give the page's centred window [-k/2, (k-1)/2] (the beta
 *     paragraph), for even kernels as well as odd ones.  Taps outside the
 *     image contribute nothing.
 *   - in' = fmaf(in, input_scale[f], input_bias[f]) in fp32; the sign is
 *     taken as (in' < 0) ? -1 : +1 (so -0 and NaN binarise to +1);
 *     subnormals are kept.
 *   - beta[i,y,x] = (sum of A over the window's in-image taps)/(kernel_h *
 *     kernel_w), A[i,y,x] = sum_f |in'[i,y,x,f]| / in_c; beta = 1 without
 *     BCONV_FLAG_USE_BETA_SCALING.  It applies to all three forms.  With
 *     BCONV_FLAG_BETA_VALID_TAPS as well, the divisor is instead the number
 *     of the window's in-image taps (a mean of A over the image part of the
 *     window, so beta stays |c| at the borders for a constant input c).
 *   - A missing output scale array means the scalar desc.scale_value; missing
 *     biases mean 0; a missing input scale means 1.
 *   - neuron: one of bconv_neuron_t, applied last; ReLU is r < 0 ? 0 : r.
 *
 * Results: XNOR/AND window sums are exact integers; the fp32 epilogue and
 * the binaryWeights fp32 accumulation agree with an exact evaluation to a
 * normwise relative 1e-5.
 *
 * Errors: every call returns a bconv_status_t; argument errors are detected
 * on the host before anything is launched.  HIP failures return
 * BCONV_ERR_HIP; bconv_last_error() gives the text (per calling thread).
 */
#ifndef BCONV_H
#define BCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bconv_handle *bconv_t;

typedef enum {
    BCONV_OK = 0,
    BCONV_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or enum out of range */
    BCONV_ERR_UNSUPPORTED = 2,      /* defined by the pages but not offered (groups > 1) */
    BCONV_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    BCONV_ERR_ALLOC = 4,            /* device or host allocation failed at create */
    BCONV_ERR_HIP = 5               /* a HIP runtime call failed; see bconv_last_error() */
} bconv_status_t;

/* The three operator forms (MPSCNNBinaryConvolution, Overview, type bullets). */
typedef enum {
    BCONV_BINARY_WEIGHTS = 0,
    BCONV_XNOR = 1,
    BCONV_AND = 2
} bconv_type_t;

/* Flags (MPSCNNBinaryConvolution, Overview, beta paragraph: beta is not an
 * input; a flag turns it on).
 * BCONV_FLAG_INT8_MFMA selects, for XNOR and AND, a comparison path on the
 * int8 matrix cores instead of the popcount path: the input is stored as one
 * int8 per channel (+-1 for XNOR, 0/1 for AND; the products of the type
 * bullets read on those values), and the window sums are int8 dot products
 * with int32 accumulation.  Results are identical (exact integers, the same
 * fp32 epilogue).  The workspace's bits section then holds those int8 values,
 * channels padded with 0 to a multiple of 64, four per uint32 word
 * (bits_words = padded channels / 4).  Not valid with BCONV_BINARY_WEIGHTS.
 * BCONV_FLAG_BETA_VALID_TAPS divides beta's window sum by the count of
 * in-image taps instead of kernel_h * kernel_w (the other reading of the
 * divisor of the page's first beta equation where the window leaves the
 * image; identical inside the image).  Requires BCONV_FLAG_USE_BETA_SCALING.
 * BCONV_FLAG_FP4_MFMA selects a second comparison path, on the fp4 matrix
 * cores, for XNOR and AND layers: the product count of the 0/1 bits,
 * sum_k x_k * w_k, runs as exact e2m1 products with fp32 accumulation; AND
 * is that count and XNOR follows from it and the counts of set input and
 * weight bits over the window's in-image taps (popcount(x ^ w) = S_x + S_w -
 * 2 S_xw).  It takes layers of the fully connected shape (MPSCNNFullyConnected,
 * Overview, conditions) whose window holds a multiple of 4 words
 * (kernel_h * kernel_w * ceil(in_c / 32) % 4 == 0), and convolutions whose
 * pixel holds a multiple of 4 words (ceil(in_c / 32) % 4 == 0) with at most
 * 4096 words per window; the padded bit buffer must stay below 2 GiB per
 * call (else BCONV_ERR_HIP).  Results are identical (exact integers, the same
 * fp32 epilogue); the workspace is that of the popcount path.  bconv_create
 * returns BCONV_ERR_UNSUPPORTED for other shapes; not valid with
 * BCONV_BINARY_WEIGHTS or BCONV_FLAG_INT8_MFMA. */
enum {
    BCONV_FLAG_NONE = 0u,
    BCONV_FLAG_USE_BETA_SCALING = 1u,
    BCONV_FLAG_INT8_MFMA = 2u,
    BCONV_FLAG_BETA_VALID_TAPS = 4u,
    BCONV_FLAG_FP4_MFMA = 8u
};

/* The activation applied last (MPSCNNBinaryConvolution, Overview, closing
 * sentence of the description: "the normal activation neuron"; the page
 * names no set).  r is the value scale*beta*sum + bias; a and b are
 * desc.neuron_a / desc.neuron_b.  Each is evaluated in fp32 (exp, tanh,
 * log1p and expm1 of the device math library). */
typedef enum {
    BCONV_NEURON_NONE = 0,          /* r */
    BCONV_NEURON_RELU = 1,          /* r < 0 ? 0 : r (NaN passes) */
    BCONV_NEURON_LEAKY_RELU = 2,    /* r < 0 ? a*r : r */
    BCONV_NEURON_LINEAR = 3,        /* a*r + b */
    BCONV_NEURON_SIGMOID = 4,       /* 1 / (1 + e^-r) */
    BCONV_NEURON_HARD_SIGMOID = 5,  /* min(max(a*r + b, 0), 1) */
    BCONV_NEURON_TANH = 6,          /* a * tanh(b*r) */
    BCONV_NEURON_ABSOLUTE = 7,      /* |r| */
    BCONV_NEURON_SOFTPLUS = 8,      /* a * log(1 + e^(b*r)), as max(z,0) + log1p(e^-|z|), z = b*r */
    BCONV_NEURON_SOFTSIGN = 9,      /* r / (1 + |r|) */
    BCONV_NEURON_ELU = 10,          /* r < 0 ? a*(e^r - 1) : r */
    BCONV_NEURON_CLAMP = 11         /* min(max(r, a), b) */
} bconv_neuron_t;
#define BCONV_NEURON_COUNT 12

/* Layer shape (the convolution descriptor of the pages: kernel width/height,
 * strides, groups).  The batch size is given per call. */
typedef struct {
    int32_t in_h, in_w, in_c; /* source image height, width, feature channels (>= 1) */
    int32_t out_c;            /* output feature channels (>= 1) */
    int32_t kernel_h, kernel_w; /* >= 1; kernel_h <= in_h + pad_h + pad_h_end, likewise w */
    int32_t stride_h, stride_w; /* >= 1 */
    int32_t pad_h, pad_w;     /* leading (top, left) zero padding, 0 <= pad < kernel */
    int32_t groups;           /* must be 1 (MPSCNNBinaryConvolution, groups note) */
    int32_t neuron;           /* bconv_neuron_t */
    float scale_value;        /* output scale used when output_scale is NULL */
    int32_t pad_h_end, pad_w_end; /* trailing (bottom, right) zero padding,
                                     0 <= pad_end < kernel; equal to pad_h / pad_w
                                     for the usual symmetric padding */
    float neuron_a, neuron_b;  /* activation parameters a, b (see bconv_neuron_t) */
} bconv_desc_t;

/* Where the per-step intermediates sit in a forward call's workspace, for
 * checking each step on its own.  Offsets are in bytes from the workspace
 * start; SIZE_MAX marks a section the handle does not use.
 *   bits:  uint32 [n][bits_rows][bits_cols][bits_words], the binarised input
 *          with a zero halo of bits_pad_h rows and bits_pad_w columns on each
 *          side; channel f of pixel (y,x) is bit (f%32) of word f/32 at row
 *          y + bits_pad_h, column x + bits_pad_w (XNOR and AND only; with
 *          BCONV_FLAG_INT8_MFMA, byte f%4 of word f/4 holds channel f as int8).
 *   a_map: float [n][bits_rows][bits_cols], the A map with the same zero halo
 *          (only with BCONV_FLAG_USE_BETA_SCALING).
 *   beta:  float [n][out_h][out_w] (only with BCONV_FLAG_USE_BETA_SCALING). */
typedef struct {
    size_t bits_offset;
    int32_t bits_rows, bits_cols, bits_words, bits_pad_h, bits_pad_w;
    size_t a_map_offset;
    size_t beta_offset;
    size_t total_bytes;
} bconv_workspace_layout_t;

/* Checks a descriptor, form and flags without touching any device.
 * INVALID_ARGUMENT for out-of-range values, UNSUPPORTED for groups != 1.
 * Also enforces in_c*kernel_h*kernel_w <= 2^24 so every window sum is exact
 * in int32 and in fp32. */
bconv_status_t bconv_validate_desc(const bconv_desc_t *desc, int32_t type, uint32_t flags);

/* Builds a layer on the current HIP device (MPSCNNBinaryConvolution, Topics,
 * the initializer taking convolution data, output bias/scale, input
 * bias/scale, type and flags; the scaleValue initializer is output_scale =
 * NULL with desc.scale_value).
 *   weight_bits   host, uint32 [out_c][kernel_h][kernel_w][ceil(in_c/32)]
 *   output_scale  host, float [out_c] or NULL (-> desc.scale_value)
 *   output_bias   host, float [out_c] or NULL (-> 0)
 *   input_scale   host, float [in_c]  or NULL (-> 1)
 *   input_bias    host, float [in_c]  or NULL (-> 0)
 * Every array is copied; the caller keeps ownership of its buffers.  The
 * weights are rearranged on the device into the layouts the kernels read.
 * Synchronous.  On success *out receives a handle to release with
 * bconv_destroy.
 * Three environment variables, read here, fix the kernel choice of the
 * handle (for tests and tuning; results do not depend on them):
 *   BCONV_FORCE_GENERIC=1  the shape-generic kernels instead of the
 *                          specialised and matrix routes;
 *   BCONV_SMALL_FUSED=0    small XNOR / AND layers without beta (1x1 or 3x3
 *                          window, in_c <= 128, at most 4096 output pixel x
 *                          64-channel pairs and 2 MiB of input, not the fully
 *                          connected shape) keep the two-kernel path (pack,
 *                          then the convolution) instead of the single kernel
 *                          that binarises its own input (then the workspace
 *                          is still required but left untouched);
 *   BCONV_STRIP_WIDTH=P    the specialised XNOR / AND convolution processes P
 *                          output pixels per wave when a kernel for that width
 *                          is compiled for the shape (otherwise the width is
 *                          chosen by cost). */
bconv_status_t bconv_create(const bconv_desc_t *desc, const uint32_t *weight_bits,
                            const float *output_scale, const float *output_bias,
                            const float *input_scale, const float *input_bias, int32_t type,
                            uint32_t flags, bconv_t *out);

/* The fully connected layer (MPSCNNFullyConnected, Overview and conditions):
 * bconv_create with kernel = source size, stride 1, pad 0, groups 1; the
 * output is [n][1][1][out_c] = [n][out_c].  The weight words are
 * [out_c][in_h][in_w][ceil(in_c/32)], i.e. a row per output over the NHWC
 * flattening of the source (the page's matrix view). */
bconv_status_t bconv_create_fc(int32_t in_h, int32_t in_w, int32_t in_c, int32_t out_c,
                               int32_t neuron, float scale_value, const uint32_t *weight_bits,
                               const float *output_scale, const float *output_bias,
                               const float *input_scale, const float *input_bias, int32_t type,
                               uint32_t flags, bconv_t *out);

/* Channel counts and output extent (MPSCNNBinaryConvolution, Topics,
 * inputFeatureChannels / outputFeatureChannels).  Any pointer may be NULL. */
bconv_status_t bconv_get_info(bconv_t h, int32_t *in_c, int32_t *out_c, int32_t *out_h,
                              int32_t *out_w);

/* Workspace bytes a forward call with batch n needs (0 is possible). */
bconv_status_t bconv_workspace_size(bconv_t h, int32_t n, size_t *bytes);

/* Layout of the workspace for batch n (see bconv_workspace_layout_t). */
bconv_status_t bconv_workspace_layout(bconv_t h, int32_t n, bconv_workspace_layout_t *layout);

/* Forward pass, asynchronous on `stream` (a hipStream_t; NULL = default
 * stream).  `in`, `out` and `workspace` are device pointers owned by the
 * caller and must stay valid until the stream work completes; `in` and `out`
 * must not overlap.  n == 0 is a no-op.  Never allocates and never
 * synchronises.  One handle may serve several streams at once when each call
 * has its own workspace.  Errors: INVALID_ARGUMENT for a NULL handle or
 * pointer, n < 0, overlapping buffers, or a batch too large for one call
 * (n*H*W >= 2^31, input or output of 2 GiB or more, n*Ho*Wo*ceil(Cout/64)
 * >= 2^29, or a padded bit buffer of 2^31 words or more); WORKSPACE for a
 * missing or short workspace; HIP when a launch fails. */
bconv_status_t bconv_forward(bconv_t h, void *stream, int32_t n, const float *in, float *out,
                             void *workspace, size_t workspace_bytes);

/* Bytes of the built-in workspace of bconv_forward_noalloc (16 MiB, one copy
 * per GPU, held until the process ends). */
#define BCONV_SCRATCH_MAX_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * bconv_forward, but the workspace is the library's built-in device array of
 * BCONV_SCRATCH_MAX_BYTES bytes instead of a caller buffer.  Allocates nothing
 * and calls no allocating routine; the array's address on each GPU is taken
 * once, when the first handle is created there.  `in` and `out` are the
 * caller's device buffers as in bconv_forward.  Every call on one GPU shares
 * that GPU's array, so calls that overlap in time on one GPU (two streams,
 * two threads) race and give wrong results: serialise them.  Errors: those of
 * bconv_forward, and WORKSPACE when the batch needs more than
 * BCONV_SCRATCH_MAX_BYTES of workspace (bconv_workspace_size tells how much). */
bconv_status_t bconv_forward_noalloc(bconv_t h, void *stream, int32_t n, const float *in, float *out);

/* As bconv_forward, but writes the window sums instead of the epilogue:
 * int32 for XNOR (the +-1 sum over in-image taps) and AND (the 0/1 sum);
 * float for binaryWeights.  Same shape as the output. */
bconv_status_t bconv_forward_accum(bconv_t h, void *stream, int32_t n, const float *in,
                                   void *acc, void *workspace, size_t workspace_bytes);

/* As bconv_forward, and records hipEvent_t's on `stream` (any may be NULL) at
 * the start and end of two dispatches, so a caller can time each kernel alone:
 * `main_begin` / `main_end` bracket the convolution / matrix kernel,
 * `input_begin` / `input_end` the input step before it (the binarise-and-pack
 * kernel with the A map, or the int8 pack of BCONV_FLAG_INT8_MFMA; binaryWeights
 * has no input step without beta, and then these two are not recorded). */
bconv_status_t bconv_forward_profiled(bconv_t h, void *stream, int32_t n, const float *in,
                                      float *out, void *workspace, size_t workspace_bytes,
                                      void *main_begin, void *main_end, void *input_begin,
                                      void *input_end);

/* As bconv_forward, but the convolution's epilogue writes packed sign bits of
 * its fp32 output instead of the values, in the input encoding of a next
 * binary layer (Apple "MPSCNNBinaryConvolution", Overview: the XNOR and AND
 * bullets read a value as +1 / 1 unless it is below 0).  `out_bits` is device
 * memory of n*out_h*out_w*ceil(out_c/32) uint32 words, NHWC: channel c of
 * pixel (b, y, x) is bit c % 32 (least significant first) of word
 * ((b*out_h + y)*out_w + x)*ceil(out_c/32) + c/32; the bit is 1 unless the
 * value bconv_forward would write is < 0 (so +-0 and NaN give 1, and every bit
 * is 1 under ReLU); bits past out_c are 0.  The fp32 output is not written.
 * Same errors as bconv_forward; `out_bits` must not overlap `in` or the
 * workspace. */
bconv_status_t bconv_forward_bits(bconv_t h, void *stream, int32_t n, const float *in,
                                  uint32_t *out_bits, void *workspace, size_t workspace_bytes);

/* As bconv_forward_bits, with the hipEvents of bconv_forward_profiled. */
bconv_status_t bconv_forward_bits_profiled(bconv_t h, void *stream, int32_t n, const float *in,
                                           uint32_t *out_bits, void *workspace,
                                           size_t workspace_bytes, void *main_begin,
                                           void *main_end, void *input_begin, void *input_end);

/* Forward pass from input that is already binarised and packed, as a previous
 * layer's bconv_forward_bits writes it (Apple "MPSCNNBinaryConvolution",
 * Overview: under XNOR and AND only the sign of each input value enters the
 * product, so the sign bits are the whole input).  `in_bits` is device memory
 * of n*in_h*in_w*ceil(in_c/32) uint32 words, NHWC, channel c of pixel (b, y, x)
 * being bit c % 32 of word ((b*in_h + y)*in_w + x)*ceil(in_c/32) + c/32; a 1
 * stands for an input >= 0 (+1 under XNOR, 1 under AND), a 0 for an input
 * < 0 (-1 under XNOR, 0 under AND).  Bits past in_c are ignored.  The result
 * equals bconv_forward on any fp32 input with those signs.  Workspace as for
 * bconv_forward.  UNSUPPORTED (checked before n) for handles that read the
 * full-precision input: binaryWeights, beta scaling, an input scale or bias,
 * BCONV_FLAG_INT8_MFMA.  Otherwise the errors of bconv_forward. */
bconv_status_t bconv_forward_packed(bconv_t h, void *stream, int32_t n, const uint32_t *in_bits,
                                    float *out, void *workspace, size_t workspace_bytes);

/* As bconv_forward_packed, writing packed sign bits as bconv_forward_bits does,
 * so binary layers chain on bits alone. */
bconv_status_t bconv_forward_packed_bits(bconv_t h, void *stream, int32_t n,
                                         const uint32_t *in_bits, uint32_t *out_bits,
                                         void *workspace, size_t workspace_bytes);

/* Name of the kernel bconv_forward_profiled brackets for batch n (a static
 * string; "" for an invalid handle). */
const char *bconv_main_kernel(bconv_t h, int32_t n);

/* Calibration of the popcount path's instruction pair: launches `blocks`
 * workgroups of 256 threads on `stream` (a hipStream_t; NULL = default
 * stream); every thread runs `iters` rounds of eight independent
 * v_xor_b32 + v_bcnt_u32_b32 pairs on register operands (no memory traffic),
 * then writes one word to `sink` (device memory of blocks*256 uint32, owned by
 * the caller).  Thread t's word is the sum over k = 0..7 of
 *   iters * popcount(x[k % 4] ^ w_k),  w_k = (t * 2654435761) ^ (k * 0x9E3779B9),
 *   x[0] = seed * 0x9E3779B1, x[1] = x[0] ^ 0x85EBCA77, x[2] = x[0] + 0xC2B2AE3D,
 *   x[3] = x[0] ^ 0x27D4EB2F  (all mod 2^32),
 * so a run does blocks*256*iters*8*32 bit-MACs, and timing it gives the VALU
 * popcount rate the chip sustains (the convolution's two instructions per
 * 32-bit word pair).  Asynchronous.  INVALID_ARGUMENT for blocks outside
 * [1, 2^22], iters < 0 or a NULL sink. */
bconv_status_t bconv_calibrate_popcount(void *stream, int32_t blocks, int32_t iters, uint32_t seed,
                                        uint32_t *sink);

/* Releases the handle's device memory.  The caller must make sure no queued
 * forward call still uses it.  NULL is accepted. */
bconv_status_t bconv_destroy(bconv_t h);

/* Static text of a status code. */
const char *bconv_status_string(bconv_status_t s);

/* Text of the last error raised on the calling thread ("" if none). */
const char *bconv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BCONV_H */
