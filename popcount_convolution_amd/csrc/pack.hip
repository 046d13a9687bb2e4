// Binarise-and-pack of the input, with the fused A map, and the beta box
// filter.
//
// Input affine and sign: Apple "MPSCNNBinaryConvolution", Overview (input
// terms paragraph; XNOR and AND bullets).  A map and beta: same page, the two
// beta equations.
#include "internal.h"

namespace bconv {
namespace {

struct PackArgs {
    const float *x;
    const float *in_scale;  // [in_c] or nullptr
    const float *in_bias;   // [in_c] or nullptr
    uint32_t *bits;         // padded bit buffer or nullptr (A only)
    float *a_map;           // [pixels] or nullptr
    long long pixels;       // n*in_h*in_w
    int in_h, in_w, in_c, words;
    int rows, cols, halo_h, halo_w;
    int pack_blocks;        // blocks doing the packing; the rest clear the halo
    long long halo_pixels_per_image;
    long long halo_words;   // n*halo_pixels_per_image*words
    long long slack_words;  // zero words after the last image
    long long image_words;  // rows*cols*words
    int n;
};

// Zero the halo of every image and the slack after the last image, so that
// padded taps and strip over-reads see 0 bits.
__device__ void clear_halo(const PackArgs &a, long long t)
{
    if (t >= a.halo_words + a.slack_words) return;
    if (t >= a.halo_words) {
        a.bits[(long long)a.n * a.image_words + (t - a.halo_words)] = 0u;
        return;
    }
    const long long per_image = a.halo_pixels_per_image * a.words;
    const long long img = t / per_image;
    long long r = t % per_image;
    const int word = (int)(r % a.words);
    long long i = r / a.words;  // halo pixel within the image
    int row, col;
    const long long top = (long long)a.halo_h * a.cols;
    const long long bottom = (long long)(a.rows - a.halo_h - a.in_h) * a.cols;
    if (i < top) {
        row = (int)(i / a.cols);
        col = (int)(i % a.cols);
    } else if (i - top < bottom) {
        i -= top;
        row = a.halo_h + a.in_h + (int)(i / a.cols);
        col = (int)(i % a.cols);
    } else {
        i -= top + bottom;
        const int side = a.cols - a.in_w;
        row = a.halo_h + (int)(i / side);
        const int j = (int)(i % side);
        col = j < a.halo_w ? j : a.in_w + j;
    }
    a.bits[img * a.image_words + ((long long)row * a.cols + col) * a.words + word] = 0u;
}

// One pass of a wave covers 64/SEG pixels; each pixel's channels are spread
// over SEG lanes, VEC consecutive channels per lane.  The channel signs of a
// 32-channel word are gathered with an OR across the 32/VEC lanes holding it;
// |x'| is summed per lane and then across the pixel's lanes (a fixed
// butterfly, so the result is deterministic).
template <int VEC, int SEG>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a)
{
    if ((int)blockIdx.x >= a.pack_blocks) {
        clear_halo(a, (long long)(blockIdx.x - a.pack_blocks) * blockDim.x + threadIdx.x);
        return;
    }
    constexpr int PPW = 64 / SEG;
    constexpr int CHUNK = SEG * VEC;
    constexpr int LPW = (32 / VEC) < SEG ? (32 / VEC) : SEG;
    const int lane = threadIdx.x & 63;
    const int slot = lane / SEG;
    const int sl = lane % SEG;
    const long long wave = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const long long pix = wave * PPW + slot;
    const bool live = pix < a.pixels;
    const bool affine = a.in_scale != nullptr || a.in_bias != nullptr;
    const float *xp = a.x + (live ? pix : 0) * a.in_c;

    long long dst = 0;
    if (a.bits && live) {
        const long long img = pix / ((long long)a.in_h * a.in_w);
        const int rem = (int)(pix % ((long long)a.in_h * a.in_w));
        const int y = rem / a.in_w, x = rem % a.in_w;
        dst = img * a.image_words +
              ((long long)(y + a.halo_h) * a.cols + (x + a.halo_w)) * a.words;
    }

    float asum = 0.0f;
    for (int c0 = 0; c0 < a.in_c; c0 += CHUNK) {
        const int c = c0 + sl * VEC;
        const bool act = live && c < a.in_c;
        uint32_t nib = 0;
        if (act) {
            float v[VEC];
            if constexpr (VEC == 4) {
                const float4 q = *reinterpret_cast<const float4 *>(xp + c);
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            } else {
                v[0] = xp[c];
            }
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                float t = v[j];
                if (affine) {
                    const float s = a.in_scale ? a.in_scale[c + j] : 1.0f;
                    const float b = a.in_bias ? a.in_bias[c + j] : 0.0f;
                    t = __builtin_fmaf(t, s, b);
                }
                nib |= (t < 0.0f ? 0u : 1u) << j;
                asum += fabsf(t);
            }
        }
        if (a.bits) {
            uint32_t part = nib << ((sl * VEC) & 31);
#pragma unroll
            for (int off = 1; off < LPW; off <<= 1) part |= __shfl_xor(part, off, 64);
            if (act && (sl % LPW) == 0) a.bits[dst + c / 32] = part;
        }
    }
    if (a.a_map) {
#pragma unroll
        for (int off = 1; off < SEG; off <<= 1) asum += __shfl_xor(asum, off, 64);
        if (live && sl == 0) a.a_map[pix] = asum / (float)a.in_c;
    }
}

template <int VEC, int SEG>
hipError_t launch_pack_t(const PackArgs &a, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL((pack_kernel<VEC, SEG>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// beta[i,y,x] = sum of A over the in-image taps of the window / (kh*kw).
__global__ __launch_bounds__(256) void beta_kernel(const float *__restrict__ a_map,
                                                   float *__restrict__ beta, int n, int in_h,
                                                   int in_w, int out_h, int out_w, int kh, int kw,
                                                   int sh, int sw, int ph, int pw)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)n * out_h * out_w;
    if (t >= total) return;
    const int ox = (int)(t % out_w);
    const int oy = (int)((t / out_w) % out_h);
    const long long img = t / ((long long)out_w * out_h);
    const float *am = a_map + img * in_h * in_w;
    float sum = 0.0f;
    for (int ky = 0; ky < kh; ++ky) {
        const int iy = oy * sh - ph + ky;
        if (iy < 0 || iy >= in_h) continue;
        for (int kx = 0; kx < kw; ++kx) {
            const int ix = ox * sw - pw + kx;
            if (ix < 0 || ix >= in_w) continue;
            sum += am[(long long)iy * in_w + ix];
        }
    }
    beta[t] = sum / (float)(kh * kw);
}

}  // namespace

hipError_t launch_pack(const Geom &g, hipStream_t s, const float *x, const float *in_scale,
                       const float *in_bias, uint32_t *bits, float *a_map)
{
    PackArgs a{};
    a.x = x;
    a.in_scale = in_scale;
    a.in_bias = in_bias;
    a.bits = bits;
    a.a_map = a_map;
    a.n = g.n;
    a.pixels = (long long)g.n * g.in_h * g.in_w;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.in_c = g.in_c;
    a.words = g.words;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    a.halo_h = g.bits_halo_h;
    a.halo_w = g.bits_halo_w;
    a.image_words = (long long)g.bits_rows * g.bits_cols * g.words;
    a.halo_pixels_per_image = (long long)g.bits_rows * g.bits_cols - (long long)g.in_h * g.in_w;
    a.halo_words = bits ? (long long)g.n * a.halo_pixels_per_image * g.words : 0;
    a.slack_words = bits ? g.bits_slack_words : 0;

    const int vec = (g.in_c % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0) ? 4 : 1;
    int need = (g.in_c + vec - 1) / vec;
    int seg = 1;
    while (seg < need && seg < 64) seg <<= 1;
    const long long ppw = 64 / seg;
    const long long waves = (a.pixels + ppw - 1) / ppw;
    const long long pack_blocks = (waves + 3) / 4;
    const long long halo_blocks = (a.halo_words + a.slack_words + 255) / 256;
    if (pack_blocks + halo_blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    a.pack_blocks = (int)pack_blocks;
    const int blocks = (int)(pack_blocks + halo_blocks);
    if (blocks == 0) return hipSuccess;
#define BCONV_PACK_CASE(V, S) \
    if (vec == V && seg == S) return launch_pack_t<V, S>(a, blocks, s);
    BCONV_PACK_CASE(4, 1) BCONV_PACK_CASE(4, 2) BCONV_PACK_CASE(4, 4) BCONV_PACK_CASE(4, 8)
    BCONV_PACK_CASE(4, 16) BCONV_PACK_CASE(4, 32) BCONV_PACK_CASE(4, 64)
    BCONV_PACK_CASE(1, 1) BCONV_PACK_CASE(1, 2) BCONV_PACK_CASE(1, 4) BCONV_PACK_CASE(1, 8)
    BCONV_PACK_CASE(1, 16) BCONV_PACK_CASE(1, 32) BCONV_PACK_CASE(1, 64)
#undef BCONV_PACK_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_beta(const Geom &g, hipStream_t s, const float *a_map, float *beta)
{
    const long long total = (long long)g.n * g.out_h * g.out_w;
    if (total == 0) return hipSuccess;
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(beta_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a_map, beta, g.n,
                       g.in_h, g.in_w, g.out_h, g.out_w, g.kh, g.kw, g.sh, g.sw, g.ph, g.pw);
    return hipGetLastError();
}

}  // namespace bconv
