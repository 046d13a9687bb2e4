// Single-launch XNOR / AND binary convolution for small layers.
//
// Apple "MPSCNNBinaryConvolution" (Overview): the input terms paragraph
// (in' = in * inputScale + inputBias per channel), the XNOR and AND bullets
// (bin(x) = x < 0 ? -1 : 1, then 32 - 2*popcount(x ^ w) or popcount(x & w)
// per 32-bit word pair) and the output equation with its fused epilogue
// neuron(v * scale[c] + bias[c]) (no beta on this path).
//
// A small layer spends most of a two-kernel step (binarise-and-pack, then the
// convolution) on two launches and two memory round trips.  Here one kernel
// does both: one wave per (output pixel, 64-channel tile).
//  * Binarise in registers: for each tap of the window, lane l reads channel
//    64*c + l of the input pixel (256 contiguous bytes per wave), applies the
//    input affine and compares; a wave ballot of the 64 signs is exactly the
//    two packed 32-channel words of that pixel (bit f % 32 of word f / 32 is
//    channel f), already in SGPRs.
//  * Convolve: lane l is output channel 64*tile + l; its weight words come
//    from the lane-major table of the specialised kernel; v_xor/v_and with the
//    ballot word as the scalar operand, v_bcnt to count and accumulate.  Taps
//    outside the image are skipped (the window holds the same pixel for the
//    whole wave), so the XNOR value is Cin*valid_taps - 2*acc with no border
//    correction.
//  * Every input load of the window is issued before any is used.
// Each input value is read once per window that holds it (kh*kw/stride^2
// times) instead of once, which is why this path is only taken for layers
// whose input is small.
#include "internal.h"

namespace bconv {
namespace {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: loads return 0

struct SArgs {
    const float *x;
    const float *in_scale, *in_bias;  // both or neither
    const uint32_t *wlane;            // [tiles][kh][kwc4][64][4]
    const float *scale, *bias;
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;
    int out_words;
    int in_h, in_w, in_c, out_c, out_h, out_w;
    int sh, sw, ph, pw, kwc4, tiles;
    int waves;  // n * out_h * out_w * tiles
    int x_bytes, wlane_bytes;
};

// KH x KW window, WORDS = ceil(in_c / 32) words per pixel (channels read in
// chunks of 64, one per lane).
template <int KH, int KW, int WORDS, bool AND>
__global__ __launch_bounds__(256) void xconv_small(SArgs a)
{
    constexpr int NCH = (WORDS + 1) / 2;    // 64-channel chunks per pixel
    constexpr int RW4 = (KW * WORDS + 3) / 4;  // 16-byte weight groups per kernel row
    const int lane = threadIdx.x & 63;
    // wave -> (output pixel, channel tile); all uniform
    const int gw = (int)(blockIdx.x * 4u) + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (gw >= a.waves) return;
    const int tile = gw % a.tiles;
    const int pix = gw / a.tiles;
    const int hw = a.out_h * a.out_w;
    const int img = pix / hw, rem = pix - img * hw;
    const int oy = rem / a.out_w, ox = rem - oy * a.out_w;
    const int iy0 = oy * a.sh - a.ph, ix0 = ox * a.sw - a.pw;

    // every input value of the window (0 outside the image or past in_c)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    float v[KH * KW][NCH];
#pragma unroll
    for (int t = 0; t < KH * KW; ++t) {
        const int iy = iy0 + t / KW, ix = ix0 + t % KW;
        const bool inside = (unsigned)iy < (unsigned)a.in_h && (unsigned)ix < (unsigned)a.in_w;
        const uint32_t base = (uint32_t)(((img * a.in_h + iy) * a.in_w + ix) * a.in_c) * 4u;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const int c = ch * 64 + lane;
            const uint32_t off = (inside && c < a.in_c) ? base + (uint32_t)c * 4u : kOob;
            v[t][ch] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0));
        }
    }
    // the lane's input affine (per input channel) and output channel's weights
    float isc[NCH], ibi[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int c = ch * 64 + lane;
        const int cc = c < a.in_c ? c : 0;
        isc[ch] = a.in_scale ? a.in_scale[cc] : 1.0f;
        ibi[ch] = a.in_bias ? a.in_bias[cc] : 0.0f;
    }
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wlane, a.wlane_bytes);
    uint32_t w[KH][RW4 * 4];
#pragma unroll
    for (int ky = 0; ky < KH; ++ky)
#pragma unroll
        for (int q = 0; q < RW4; ++q) {
            // rows hold kwc4 >= RW4 groups when in_c rounds up to WORDS words
            const uint32_t off = (uint32_t)((((tile * KH + ky) * a.kwc4 + q) * 64 + lane) * 16);
            const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
            w[ky][4 * q] = u.x;
            w[ky][4 * q + 1] = u.y;
            w[ky][4 * q + 2] = u.z;
            w[ky][4 * q + 3] = u.w;
        }
    const int co = tile * kTile + lane;
    const bool co_ok = co < a.out_c;
    const float sc = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
    const float bi = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;

    uint32_t acc = 0;
    int valid = 0;
#pragma unroll
    for (int t = 0; t < KH * KW; ++t) {
        const int ky = t / KW, kx = t % KW;
        const int iy = iy0 + ky, ix = ix0 + kx;
        if ((unsigned)iy >= (unsigned)a.in_h || (unsigned)ix >= (unsigned)a.in_w) continue;  // uniform
        ++valid;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const int c = ch * 64 + lane;
            const float xv = __builtin_fmaf(v[t][ch], isc[ch], ibi[ch]);
            // bit = !(x' < 0): -0 and NaN give 1; channels past in_c give 0
            const unsigned long long m = __ballot(c < a.in_c && !(xv < 0.0f));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int wd = 2 * ch + h;
                if (wd >= WORDS) break;
                const uint32_t word = h ? (uint32_t)(m >> 32) : (uint32_t)m;
                const uint32_t wv = w[ky][kx * WORDS + wd];
                acc += __builtin_popcount(AND ? (word & wv) : (word ^ wv));
            }
        }
    }
    const int value = AND ? (int)acc : a.in_c * valid - 2 * (int)acc;
    const long long o = (long long)pix * a.out_c + co;
    if (a.acc_out) {
        if (co_ok) store_through(&a.acc_out[o], value);
        return;
    }
    // beta = 1 as a value the compiler cannot see: fma(v*scale, 1, bias) must
    // round as in the other kernels (v*scale rounded, then one fma), not be
    // folded and contracted into fma(v, scale, bias)
    float be = 1.0f;
    asm volatile("" : "+v"(be));
    const float res = epilogue_value((float)value, sc, be, bi, a.neuron);
    if (a.bits_out) {
        store_tile_bits(a.bits_out, pix, a.out_words, tile, co_ok && sign_bit(res));
        return;
    }
    if (co_ok) store_through(&a.out[o], res);
}

typedef void (*small_kernel)(SArgs);

template <bool AND>
small_kernel pick(int k, int words)
{
    if (k == 1) {
        switch (words) {
        case 1: return xconv_small<1, 1, 1, AND>;
        case 2: return xconv_small<1, 1, 2, AND>;
        case 3: return xconv_small<1, 1, 3, AND>;
        case 4: return xconv_small<1, 1, 4, AND>;
        }
    } else if (k == 3) {
        switch (words) {
        case 1: return xconv_small<3, 3, 1, AND>;
        case 2: return xconv_small<3, 3, 2, AND>;
        case 3: return xconv_small<3, 3, 3, AND>;
        case 4: return xconv_small<3, 3, 4, AND>;
        }
    }
    return nullptr;
}

}  // namespace

bool small_route(const Geom &g)
{
    if (!(g.kh == g.kw && (g.kh == 1 || g.kh == 3)) || g.words > 4) return false;
    if (gemm_route(g)) return false;  // fully connected shapes have their own matrix kernel
    const long long waves = (long long)g.n * g.out_h * g.out_w * g.tiles;
    const long long x_bytes = (long long)g.n * g.in_h * g.in_w * g.in_c * 4;
    return waves <= kSmallMaxWaves && x_bytes <= kSmallMaxInputBytes;
}

const char *small_kernel_name(const Geom &g, int and_mode)
{
    static const char *const names[2][2][4] = {
        {{"xconv_small<1,1,1,false>", "xconv_small<1,1,2,false>", "xconv_small<1,1,3,false>",
          "xconv_small<1,1,4,false>"},
         {"xconv_small<3,3,1,false>", "xconv_small<3,3,2,false>", "xconv_small<3,3,3,false>",
          "xconv_small<3,3,4,false>"}},
        {{"xconv_small<1,1,1,true>", "xconv_small<1,1,2,true>", "xconv_small<1,1,3,true>", "xconv_small<1,1,4,true>"},
         {"xconv_small<3,3,1,true>", "xconv_small<3,3,2,true>", "xconv_small<3,3,3,true>",
          "xconv_small<3,3,4,true>"}}};
    if (!small_route(g)) return "";
    return names[and_mode ? 1 : 0][g.kh == 3 ? 1 : 0][g.words - 1];
}

hipError_t launch_xconv_small(const Geom &g, const Launch &L, int and_mode, const float *x, const float *in_scale,
                              const float *in_bias, const LaneWeights &w, const Epilogue &e, float *out,
                              int32_t *acc_out)
{
    if (!small_route(g)) return hipErrorInvalidValue;
    SArgs a{};
    a.x = x;
    a.in_scale = in_scale;
    a.in_bias = in_bias;
    a.wlane = w.words;
    a.scale = e.scale;
    a.bias = e.bias;
    a.scale_value = e.scale_value;
    a.neuron = e.neuron;
    a.out = out;
    a.acc_out = acc_out;
    a.bits_out = e.bits_out;
    a.out_words = e.out_words;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.in_c = g.in_c;
    a.out_c = g.out_c;
    a.out_h = g.out_h;
    a.out_w = g.out_w;
    a.sh = g.sh;
    a.sw = g.sw;
    a.ph = g.ph;
    a.pw = g.pw;
    a.kwc4 = w.kwc4;
    a.tiles = g.tiles;
    a.waves = (int)((long long)g.n * g.out_h * g.out_w * g.tiles);
    a.x_bytes = (int)((long long)g.n * g.in_h * g.in_w * g.in_c * 4);
    a.wlane_bytes = (int)((long long)g.tiles * g.kh * w.kwc4 * 256 * 4);
    if (a.waves == 0) return hipSuccess;
    const small_kernel k = and_mode ? pick<true>(g.kh, g.words) : pick<false>(g.kh, g.words);
    if (!k) return hipErrorInvalidValue;
    return launch_kernel(L, k, dim3((unsigned)((a.waves + 3) / 4)), dim3(256), 0, a);
}

}  // namespace bconv
