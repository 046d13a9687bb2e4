// Internal declarations shared by the host library and the kernel files of
// libbconv.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bconv.h"

namespace bconv {

// Output channels handled by one wave in the lane-per-channel kernels.
constexpr int kTile = 64;

// Geometry of one forward call, resolved on the host.
struct Geom {
    int n, in_h, in_w, in_c, out_c;
    int kh, kw, sh, sw, ph, pw;
    int out_h, out_w;
    int words;        // ceil(in_c / 32)
    int tiles;        // ceil(out_c / kTile)
    // binarised-input buffer with a zero halo
    int bits_rows;    // in_h + ph + trailing pad
    int bits_cols;    // in_w + pw + trailing pad
    int bits_halo_h, bits_halo_w;
    long long bits_slack_words;  // zero words after the last image (strip over-reads)
    int simds;        // SIMD units of the device (4 per compute unit)
    int strip_p;      // strip width the specialised convolution must use (0: by cost)
};

// Raw buffer descriptor word 3 for gfx9-family targets (32-bit data format).
constexpr int kBufferFlags = 0x00020000;
// Buffer cache policy: agent-scope write-through (sc1).
constexpr int kStoreSc1 = 16;

// Agent-scope relaxed store: written through to memory while the kernel runs,
// so it does not sit dirty in one XCD's L2 until the end-of-kernel write-back.
template <typename T>
__device__ __forceinline__ void store_through(T *p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The activation applied last: type (a bconv_neuron_t value) and parameters.
struct Neuron {
    int type;
    float a, b;
};
constexpr int kNeuronNone = 0;
constexpr int kNeuronRelu = 1;

// neuron(r), in fp32 with the device math library (the definitions are listed
// with bconv_neuron_t).
__device__ __forceinline__ float apply_neuron(const Neuron &n, float r)
{
    switch (n.type) {
    case 1: return (r < 0.0f) ? 0.0f : r;
    case 2: return (r < 0.0f) ? n.a * r : r;
    case 3: return __builtin_fmaf(n.a, r, n.b);
    case 4: return 1.0f / (1.0f + expf(-r));
    case 5: return fminf(fmaxf(__builtin_fmaf(n.a, r, n.b), 0.0f), 1.0f);
    case 6: return n.a * tanhf(n.b * r);
    case 7: return fabsf(r);
    case 8: {
        const float z = n.b * r;
        return n.a * (fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))));
    }
    case 9: return r / (1.0f + fabsf(r));
    case 10: return (r < 0.0f) ? n.a * expm1f(r) : r;
    case 11: return fminf(fmaxf(r, n.a), n.b);
    default: return r;
    }
}

// The fused epilogue's output value: neuron(v * scale * beta + bias).
__device__ __forceinline__ float epilogue_value(float v, float sc, float be, float bi, const Neuron &n)
{
    return apply_neuron(n, __builtin_fmaf(v * sc, be, bi));
}

// apply_neuron as one out-of-line copy per translation unit.
static __device__ __attribute__((noinline)) float apply_neuron_outline(int type, float na, float nb, float r)
{
    return apply_neuron(Neuron{type, na, nb}, r);
}

// epilogue_value for kernels that form many values per lane: identity and
// ReLU inline, every other neuron through the one out-of-line copy (the whole
// switch inlined at each value would overflow the instruction cache).  The
// same arithmetic, so the same results.
__device__ __forceinline__ float epilogue_value_compact(float v, float sc, float be, float bi, const Neuron &n)
{
    const float r = __builtin_fmaf(v * sc, be, bi);
    if (n.type == kNeuronNone) return r;
    if (n.type == kNeuronRelu) return (r < 0.0f) ? 0.0f : r;
    return apply_neuron_outline(n.type, n.a, n.b, r);
}

// Sign bit of an output value, in the input encoding of the next binary
// layer: 1 unless y < 0 (so +-0 and NaN give 1).
__device__ __forceinline__ bool sign_bit(float y) { return !(y < 0.0f); }

// Packed sign bits of one output pixel over a 64-channel tile held one
// channel per lane (`bit` already 0 for channels past out_c).  Every lane of
// the wave must call it.  Lanes 0 and 1 write words 2*tile and 2*tile + 1 of
// the pixel's `out_words` words, where those exist.
__device__ __forceinline__ void store_tile_bits(uint32_t *bits, long long pixel, int out_words, int tile, bool bit)
{
    const unsigned long long m = __ballot(bit);
    const int lane = threadIdx.x & 63;
    const int wi = 2 * tile + lane;
    if (lane < 2 && wi < out_words)
        store_through(&bits[pixel * out_words + wi], lane ? (uint32_t)(m >> 32) : (uint32_t)m);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, kBufferFlags);
}

// Stream plus the optional hipEvents that bracket one kernel dispatch: with
// events, the kernel is launched by hipExtLaunchKernelGGL, which records
// them at the dispatch's own start and completion.
struct Launch {
    hipStream_t stream;
    hipEvent_t begin, end;
};

template <typename... Args, typename F>
hipError_t launch_kernel(const Launch &L, F kernel, dim3 grid, dim3 block, uint32_t lds, Args... args)
{
    if (L.begin || L.end)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, L.stream, L.begin, L.end, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, L.stream, args...);
    return hipGetLastError();
}

// Per-lane weight words, grouped by kernel row: [tiles][kh][kwc4][64][4],
// kwc4 = ceil(kw*words / 4).  Within row ky, word r = kx*words + w; lane l
// of tile t holds output channel t*64 + l, so a wave reads 256 contiguous
// bytes per 4 words.  Channels >= out_c and words past kw*words are zero; bits
// >= in_c are cleared.
struct LaneWeights {
    const uint32_t *words;  // device
    const int32_t *rect;    // [tiles][64][(kh+1)*rect_row]: prefix sums of tap popcounts
    int kwc4;
};

// Entries per row of a lane's prefix-sum table: kw+1 rounded up to a multiple
// of 4, so each table row is whole 16-byte loads.
__host__ __device__ inline int rect_row(int kw) { return (kw + 1 + 3) / 4 * 4; }

// Unsigned division by a runtime divisor d (1 <= d < 2^31) of numerators
// n < 2^31 as a multiply-high and a shift: with l = ceil(log2 d) >= 1,
// m = floor(2^(31+l) / d) + 1 fits 32 bits and n/d = mulhi(n, m) >> (l-1)
// (the error term n*(m*d - 2^(31+l)) / (d*2^(31+l)) stays below 1/d).  d = 1
// is m = 0: the quotient is n.
struct FastDiv {
    uint32_t m;
    int s;
    uint32_t id;  // all ones for d <= 1 (m = 0, quotient = n), else 0
};
inline FastDiv make_fastdiv(uint32_t d)
{
    if (d <= 1) return FastDiv{0u, 0, 0xffffffffu};
    int l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned long long m = (1ull << (31 + l)) / d + 1;
    return FastDiv{(uint32_t)m, l - 1, 0u};
}
// Branch-free: for d <= 1 the product term is 0 and the mask passes n.
__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f)
{
    return (__umulhi(n, f.m) >> f.s) | (n & f.id);
}

// Epilogue operands.  With a_pad set, the convolution kernels form beta as
// the window sum of the zero-halo A map / (kh*kw) and also store it to
// beta_out ([n][out_h][out_w]); without it beta is 1.
struct Epilogue {
    const float *scale;  // [out_c] or nullptr -> scale_value
    const float *bias;   // [out_c] or nullptr -> 0
    float scale_value;
    const float *a_pad;  // [n][bits_rows][bits_cols] or nullptr
    float *beta_out;     // [n][out_h][out_w] (used when a_pad is set)
    Neuron neuron;
    // Packed sign bits of the output instead of fp32 values: [n][out_h][out_w]
    // [out_words] words, channel c at bit c % 32 of word c / 32, bit = !(y < 0)
    // for the value y the fp32 output would hold, bits past out_c zero.
    uint32_t *bits_out;
    int out_words;
    // beta divides by the window's in-image tap count instead of kh*kw
    int beta_valid_taps;
};

// Number of taps of output pixel (oy, ox)'s window that lie inside the image
// (at least 1: every window holds an in-image tap since pads < kernel).
__device__ __forceinline__ int window_valid_taps(int oy, int ox, int sh, int sw, int ph, int pw, int kh, int kw,
                                                 int in_h, int in_w)
{
    const int iy0 = oy * sh - ph, ix0 = ox * sw - pw;
    const int r0 = iy0 < 0 ? -iy0 : 0, r1 = in_h - iy0 < kh ? in_h - iy0 : kh;
    const int c0 = ix0 < 0 ? -ix0 : 0, c1 = in_w - ix0 < kw ? in_w - ix0 : kw;
    const int v = (r1 - r0) * (c1 - c0);
    return v > 0 ? v : 1;
}

// Launchers (each returns the hipGetLastError() of its launch).
hipError_t launch_pack(const Geom &g, const Launch &L, const float *x, const float *in_scale,
                       const float *in_bias, uint32_t *bits, float *a_map);
// Copies caller-packed input bits ([n][in_h][in_w][words]) into the padded bit
// buffer, zeroing the halo, the slack and the bits past in_c.
hipError_t launch_repad(const Geom &g, const Launch &L, const uint32_t *src, uint32_t *bits);
hipError_t launch_prepack(const Geom &g, hipStream_t s, const uint32_t *user_bits, uint32_t *lane_words,
                          int32_t *lane_popc, float *pm_weights, int pm_cols, int type);
// Returns true when a specialised convolution kernel exists for this shape.
bool xconv_fast_available(const Geom &g);
const char *xconv_kernel_name(const Geom &g);
hipError_t launch_xconv(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits,
                        const LaneWeights &w, const Epilogue &e, float *out, int32_t *acc_out,
                        bool allow_fast);
// Single-launch XNOR / AND convolution for small layers (binarises its own
// input; no pack kernel, no bit buffer): 1x1 and 3x3 windows, in_c <= 128,
// not the fully connected shape, at most kSmallMaxWaves (output pixel,
// 64-channel tile) pairs and kSmallMaxInputBytes of fp32 input.
constexpr long long kSmallMaxWaves = 4096;
constexpr long long kSmallMaxInputBytes = 2ll << 20;
bool small_route(const Geom &g);
const char *small_kernel_name(const Geom &g, int and_mode);
hipError_t launch_xconv_small(const Geom &g, const Launch &L, int and_mode, const float *x, const float *in_scale,
                              const float *in_bias, const LaneWeights &w, const Epilogue &e, float *out,
                              int32_t *acc_out);
// Columns of the +-1.0f binaryWeights table (out_c rounded up to the channel block).
int bwconv_pm_cols(int out_c);
const char *bwconv_kernel_name(const Geom &g);
// Fully connected shape (kernel = source, stride 1, no padding): binary GEMM.
bool gemm_route(const Geom &g);
size_t gemm_weight_words(const Geom &g);
hipError_t launch_prepack_flat(const Geom &g, hipStream_t s, const uint32_t *user_bits, uint32_t *flat);
const char *gemm_kernel_name(const Geom &g, int and_mode);
hipError_t launch_gemm(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const uint32_t *wflat,
                       const Epilogue &e, float *out, int32_t *acc_out);
// XNOR / AND on the fp4 matrix cores (comparison path; 0/1 bit counts, exact
// in fp32): the fully connected product when its row is a multiple of 4
// words, a convolution when a pixel is (at most 1024 word groups per window).
bool f4_route(const Geom &g);
size_t f4_bytes(const Geom &g);
hipError_t launch_prepack_f4(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *tab);
const char *f4_kernel_name(const Geom &g, int and_mode);
hipError_t launch_f4(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const void *tab,
                     const Epilogue &e, float *out, int32_t *acc_out);
hipError_t launch_bwconv(const Geom &g, const Launch &L, const float *x, const float *in_scale,
                         const float *in_bias, const float *pm_weights, int pm_cols,
                         const Epilogue &e, float *out, float *acc_out);

// binaryWeights on the bf16 matrix cores (exact three-way split of the input).
size_t bwmma_frag_bytes(const Geom &g);
hipError_t launch_prepack_bwmma(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *frag);
// `affine`: the layer has an input scale/bias (then both device arrays exist).
const char *bwmma_kernel_name(const Geom &g, bool affine);
hipError_t launch_bwmma(const Geom &g, const Launch &L, const float *x, const float *in_scale, const float *in_bias,
                        const void *frag, const Epilogue &e, float *out, float *acc_out);

// XNOR / AND on the int8 matrix cores (comparison path).
int i8_cpad(int in_c);  // channels padded to a multiple of 64
size_t i8_act_bytes(const Geom &g);
size_t i8_frag_bytes(const Geom &g);
hipError_t launch_prepack_i8(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *frag, int and_mode);
hipError_t launch_pack_i8(const Geom &g, const Launch &L, const float *x, const float *in_scale, const float *in_bias,
                          int and_mode, int8_t *act, float *a_map);
const char *i8mma_kernel_name();
// Calibration kernel: blocks x 256 lanes, each running iters rounds of eight
// v_xor_b32 + v_bcnt_u32_b32 pairs on registers; one sum per lane to sink.
hipError_t launch_popc_peak(hipStream_t stream, int blocks, int iters, uint32_t seed, uint32_t *sink);
hipError_t launch_i8mma(const Geom &g, const Launch &L, const int8_t *act, const void *frag, const Epilogue &e,
                        float *out, int32_t *acc_out);

}  // namespace bconv
