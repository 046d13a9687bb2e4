// Binarise-and-pack of the input, with the fused A map.
//
// Input affine and sign: Apple "MPSCNNBinaryConvolution", Overview (input
// terms paragraph; XNOR and AND bullets).  A map: same page, second beta
// equation (mean over channels of |in'|).  The A map is written with the
// same zero halo as the bit buffer, so the convolution kernels form beta (the
// window sum of A over kh*kw, first beta equation) without bounds checks.
// The repad kernel at the end serves input that arrives already packed (a
// previous layer's sign bits): it only moves words into the padded buffer.
#include "internal.h"

namespace bconv {
namespace {

struct PackArgs {
    const float *x;
    int x_bytes;            // input size in bytes (< 2^31, checked by the host)
    const float *in_scale;  // [in_c] or nullptr
    const float *in_bias;   // [in_c] or nullptr
    uint32_t *bits;         // padded bit buffer or nullptr (A only)
    float *a_map;           // padded [n][rows][cols] or nullptr
    long long pixels;       // n*in_h*in_w
    int in_h, in_w, in_c, words;
    int rows, cols, halo_h, halo_w;
    int pack_blocks;        // blocks doing the packing; the rest clear the halo
    long long halo_pixels_per_image;
    long long halo_words;   // n*halo_pixels_per_image*words
    long long slack_words;  // zero words after the last image
    long long image_words;  // rows*cols*words
    long long halo_a;       // n*halo_pixels_per_image (A map halo entries)
    int n;
};

__device__ __forceinline__ void halo_pixel(const PackArgs &a, unsigned i, int &row, int &col)
{
    const unsigned cols = (unsigned)a.cols;
    const unsigned top = (unsigned)a.halo_h * cols;
    const unsigned bottom = (unsigned)(a.rows - a.halo_h - a.in_h) * cols;
    if (i < top) {
        row = (int)(i / cols);
        col = (int)(i % cols);
    } else if (i - top < bottom) {
        i -= top;
        row = a.halo_h + a.in_h + (int)(i / cols);
        col = (int)(i % cols);
    } else {
        i -= top + bottom;
        const unsigned side = (unsigned)(a.cols - a.in_w);
        row = a.halo_h + (int)(i / side);
        const int j = (int)(i % side);
        col = j < a.halo_w ? j : a.in_w + j;
    }
}

// Zero the halo of every image (bit words, then A entries) and the slack
// after the last image, so that padded taps and strip over-reads see 0.
__device__ void clear_halo(const PackArgs &a, long long t)
{
    // halo and slack counts fit 31 bits (they are below the padded buffer size)
    if (t >= a.halo_words + a.slack_words) {
        const unsigned u = (unsigned)(t - a.halo_words - a.slack_words);
        if ((long long)u >= a.halo_a) return;
        const unsigned per = (unsigned)a.halo_pixels_per_image;
        const unsigned img = u / per;
        int row, col;
        halo_pixel(a, u - img * per, row, col);
        store_through(&a.a_map[((long long)img * a.rows + row) * a.cols + col], 0.0f);
        return;
    }
    if (t >= a.halo_words) {
        store_through(&a.bits[(long long)a.n * a.image_words + (t - a.halo_words)], 0u);
        return;
    }
    const unsigned u = (unsigned)t;
    const unsigned per_image = (unsigned)(a.halo_pixels_per_image * a.words);
    const unsigned img = u / per_image;
    const unsigned r = u - img * per_image;
    const unsigned word = r % (unsigned)a.words;
    int row, col;
    halo_pixel(a, r / (unsigned)a.words, row, col);
    store_through(&a.bits[(long long)img * a.image_words + ((long long)row * a.cols + col) * a.words + word], 0u);
}

// Pixel indices fit 31 bits (the host checks), so the decomposition uses
// 32-bit divisions; 64-bit ones expand to long VALU sequences.
__device__ __forceinline__ long long padded_pixel(const PackArgs &a, long long pix)
{
    const unsigned p = (unsigned)pix;
    const unsigned hw = (unsigned)a.in_h * (unsigned)a.in_w;
    const unsigned img = p / hw;
    const unsigned rem = p - img * hw;
    const unsigned y = rem / (unsigned)a.in_w;
    const unsigned x = rem - y * (unsigned)a.in_w;
    return ((long long)img * a.rows + y + a.halo_h) * a.cols + x + a.halo_w;
}

// DPP lane exchanges within rows of 16 lanes (gfx9 encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// OR over aligned groups of N lanes (N <= 8); every lane gets its group's OR.
template <int N>
__device__ __forceinline__ uint32_t group_or(uint32_t v)
{
    if (N >= 2) v |= dpp_u32<kDppXor1>(v);
    if (N >= 4) v |= dpp_u32<kDppXor2>(v);
    if (N >= 8) v |= dpp_u32<kDppHalfMirror>(v);
    return v;
}
// Sum over aligned groups of N lanes (N <= 64), in a fixed order.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    if (N >= 2) v += dpp_f32<kDppXor1>(v);
    if (N >= 4) v += dpp_f32<kDppXor2>(v);
    if (N >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if (N >= 16) v += dpp_f32<kDppMirror>(v);
    if (N >= 32) v += __shfl_xor(v, 16, 64);
    if (N >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Fast path: in_c % 4 == 0 and a 16-byte aligned input.  A pixel's channels
// are spread over SEG lanes, four consecutive channels (one float4) per lane
// and SEG*4 channels per chunk; a wave pass covers 64/SEG pixels and a wave
// makes U passes, so it owns a run of G*U consecutive pixels of one image
// row, located once with scalar arithmetic (no per-lane division).  Loads and
// stores go through buffer descriptors: a scalar base plus a lane offset.  The
// input scale and bias of a lane's channels are loaded once per chunk.  A
// 32-channel word is the OR of 8 lanes' 4-bit groups (DPP), |x'| is summed per
// lane and then over the pixel's lanes in a fixed order.
template <int SEG, int U>
__global__ __launch_bounds__(256) void pack_vec4(PackArgs a)
{
    if ((int)blockIdx.x >= a.pack_blocks) {
        clear_halo(a, (long long)(blockIdx.x - a.pack_blocks) * blockDim.x + threadIdx.x);
        return;
    }
    constexpr int G = 64 / SEG;
    constexpr int RUN = G * U;  // pixels per wave
    constexpr int LPW = SEG < 8 ? SEG : 8;
    const int lane = threadIdx.x & 63;
    const int slot = lane / SEG;
    const int sl = lane % SEG;
    // wave -> (image row, run of RUN pixels in it); all uniform
    const unsigned wave = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned runs_per_row = ((unsigned)a.in_w + RUN - 1) / RUN;
    const unsigned row_id = wave / runs_per_row;  // img * in_h + y
    if (row_id >= (unsigned)a.n * (unsigned)a.in_h) return;
    const int x0 = (int)(wave - row_id * runs_per_row) * RUN;
    const unsigned img = row_id / (unsigned)a.in_h;
    const unsigned y = row_id - img * (unsigned)a.in_h;
    const uint32_t in_base = (row_id * (unsigned)a.in_w + (unsigned)x0) * (unsigned)a.in_c * 4u;
    const uint32_t pad_base = ((img * (unsigned)a.rows + y + (unsigned)a.halo_h) * (unsigned)a.cols +
                               (unsigned)(x0 + a.halo_w));  // padded pixel index of x0
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const bool affine = a.in_scale != nullptr || a.in_bias != nullptr;
    float asum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) asum[u] = 0.0f;
    for (int c0 = 0; c0 < a.in_c; c0 += SEG * 4) {
        const int c = c0 + sl * 4;
        const bool cact = c < a.in_c;
        float4 s4 = make_float4(1.f, 1.f, 1.f, 1.f), b4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (cact && a.in_scale) s4 = *reinterpret_cast<const float4 *>(a.in_scale + c);
        if (cact && a.in_bias) b4 = *reinterpret_cast<const float4 *>(a.in_bias + c);
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int px = x0 + u * G + slot;
            v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (cact && px < a.in_w)
                v[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       xr, (uint32_t)((u * G + slot) * a.in_c + c) * 4u, in_base, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int px = x0 + u * G + slot;
            float t[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            if (affine) {
                t[0] = __builtin_fmaf(t[0], s4.x, b4.x);
                t[1] = __builtin_fmaf(t[1], s4.y, b4.y);
                t[2] = __builtin_fmaf(t[2], s4.z, b4.z);
                t[3] = __builtin_fmaf(t[3], s4.w, b4.w);
            }
            uint32_t nib = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                nib |= (t[j] < 0.0f ? 0u : 1u) << j;
                asum[u] += fabsf(t[j]);
            }
            if (!cact) nib = 0;  // channels past in_c are zero bits, not signs of 0
            if (a.bits) {
                const uint32_t word = group_or<LPW>(nib << ((sl * 4) & 31));
                if (cact && px < a.in_w && (sl % LPW) == 0)
                    store_through(&a.bits[((long long)pad_base + u * G + slot) * a.words + c / 32], word);
            }
        }
    }
    if (a.a_map) {
        const float inv_c = 1.0f / (float)a.in_c;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float s = group_sum<SEG>(asum[u]);
            if (sl == 0 && x0 + u * G + slot < a.in_w) store_through(&a.a_map[(long long)pad_base + u * G + slot], s * inv_c);
        }
    }
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

    const long long dst = live ? padded_pixel(a, pix) * a.words : 0;

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
            if (act && (sl % LPW) == 0) store_through(&a.bits[dst + c / 32], part);
        }
    }
    if (a.a_map) {
#pragma unroll
        for (int off = 1; off < SEG; off <<= 1) asum += __shfl_xor(asum, off, 64);
        if (live && sl == 0) store_through(&a.a_map[padded_pixel(a, pix)], asum / (float)a.in_c);
    }
}

template <int VEC, int SEG>
hipError_t launch_pack_t(PackArgs a, long long pack_blocks, long long halo_blocks, hipStream_t s)
{
    if (pack_blocks + halo_blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    a.pack_blocks = (int)pack_blocks;
    hipLaunchKernelGGL((pack_kernel<VEC, SEG>), dim3((unsigned)(pack_blocks + halo_blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

constexpr int kPackPasses = 4;  // wave passes per wave in the vec4 path

template <int SEG>
hipError_t launch_vec4_t(PackArgs a, long long halo_blocks, hipStream_t s)
{
    const long long per_wave = (64 / SEG) * kPackPasses;
    const long long waves = (long long)a.n * a.in_h * ((a.in_w + per_wave - 1) / per_wave);
    const long long pack_blocks = (waves + 3) / 4;
    if (pack_blocks + halo_blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    a.pack_blocks = (int)pack_blocks;
    hipLaunchKernelGGL((pack_vec4<SEG, kPackPasses>), dim3((unsigned)(pack_blocks + halo_blocks)), dim3(256),
                       0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const Geom &g, hipStream_t s, const float *x, const float *in_scale,
                       const float *in_bias, uint32_t *bits, float *a_map)
{
    PackArgs a{};
    a.x = x;
    a.x_bytes = (int)((long long)g.n * g.in_h * g.in_w * g.in_c * 4 < 0x7fffffffLL
                          ? (long long)g.n * g.in_h * g.in_w * g.in_c * 4 : 0x7fffffffLL);
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
    a.halo_a = a_map ? (long long)g.n * a.halo_pixels_per_image : 0;
    const long long halo_blocks = (a.halo_words + a.slack_words + a.halo_a + 255) / 256;
    if (a.pixels == 0) return hipSuccess;

    const bool vec4 = g.in_c % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                      (long long)g.n * g.in_h * g.in_w * g.in_c * 4 < 0x7fffffffLL &&
                      (reinterpret_cast<uintptr_t>(in_scale) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(in_bias) & 15) == 0;
    const int vec = vec4 ? 4 : 1;
    int need = (g.in_c + vec - 1) / vec;
    int seg = 1;
    while (seg < need && seg < 64) seg <<= 1;
    if (vec4) {
        switch (seg) {
        case 1: return launch_vec4_t<1>(a, halo_blocks, s);
        case 2: return launch_vec4_t<2>(a, halo_blocks, s);
        case 4: return launch_vec4_t<4>(a, halo_blocks, s);
        case 8: return launch_vec4_t<8>(a, halo_blocks, s);
        case 16: return launch_vec4_t<16>(a, halo_blocks, s);
        case 32: return launch_vec4_t<32>(a, halo_blocks, s);
        default: return launch_vec4_t<64>(a, halo_blocks, s);
        }
    }
    const long long waves = (a.pixels + (64 / seg) - 1) / (64 / seg);
    const long long pack_blocks = (waves + 3) / 4;
    switch (seg) {
    case 1: return launch_pack_t<1, 1>(a, pack_blocks, halo_blocks, s);
    case 2: return launch_pack_t<1, 2>(a, pack_blocks, halo_blocks, s);
    case 4: return launch_pack_t<1, 4>(a, pack_blocks, halo_blocks, s);
    case 8: return launch_pack_t<1, 8>(a, pack_blocks, halo_blocks, s);
    case 16: return launch_pack_t<1, 16>(a, pack_blocks, halo_blocks, s);
    case 32: return launch_pack_t<1, 32>(a, pack_blocks, halo_blocks, s);
    default: return launch_pack_t<1, 64>(a, pack_blocks, halo_blocks, s);
    }
}

namespace {

struct RepadArgs {
    const uint32_t *src;    // [n][in_h][in_w][words]
    uint32_t *bits;         // padded [n][rows][cols][words] + slack
    unsigned image_words;   // rows*cols*words
    unsigned total;         // n*image_words + slack (< 2^31, checked by the host)
    unsigned image_count;   // n
    int in_h, in_w, words, cols, halo_h, halo_w;
    uint32_t tail_mask;     // valid bits of a pixel's last word
};

// One thread per word of the padded buffer: the caller's word where the pixel
// is inside the image (the last word of a pixel masked to in_c bits), else 0
// (halo and the slack after the last image).  Consecutive threads read
// consecutive words of an image row.
__global__ __launch_bounds__(256) void repad_kernel(RepadArgs a)
{
    const unsigned t = blockIdx.x * 256u + threadIdx.x;
    if (t >= a.total) return;
    uint32_t v = 0;
    const unsigned img = t / a.image_words;
    if (img < a.image_count) {
        const unsigned r = t - img * a.image_words;
        const unsigned pix = r / (unsigned)a.words;
        const unsigned w = r - pix * (unsigned)a.words;
        const unsigned row = pix / (unsigned)a.cols;
        const unsigned col = pix - row * (unsigned)a.cols;
        const int y = (int)row - a.halo_h, x = (int)col - a.halo_w;
        if (y >= 0 && y < a.in_h && x >= 0 && x < a.in_w) {
            v = a.src[(((unsigned long long)img * a.in_h + y) * a.in_w + x) * a.words + w];
            if ((int)w == a.words - 1) v &= a.tail_mask;
        }
    }
    store_through(&a.bits[t], v);
}

}  // namespace

hipError_t launch_repad(const Geom &g, hipStream_t s, const uint32_t *src, uint32_t *bits)
{
    const long long image_words = (long long)g.bits_rows * g.bits_cols * g.words;
    const long long total = (long long)g.n * image_words + g.bits_slack_words;
    if (g.n <= 0) return hipSuccess;
    if (total >= 0x7fffffffLL) return hipErrorInvalidValue;
    RepadArgs a{};
    a.src = src;
    a.bits = bits;
    a.image_words = (unsigned)image_words;
    a.total = (unsigned)total;
    a.image_count = (unsigned)g.n;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.words = g.words;
    a.cols = g.bits_cols;
    a.halo_h = g.bits_halo_h;
    a.halo_w = g.bits_halo_w;
    a.tail_mask = g.in_c % 32 ? (1u << (g.in_c % 32)) - 1u : 0xffffffffu;
    hipLaunchKernelGGL(repad_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bconv
