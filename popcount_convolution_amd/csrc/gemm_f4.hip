// XNOR / AND on the fp4 matrix cores: the fully connected product, and the
// convolution as an implicit product (second kernel, below).
//
// Apple "MPSCNNFullyConnected" (Overview, conditions, matrix view): with the
// kernel the size of the source image, stride 1 and no padding, every output
// is the dot product of the NHWC-flattened image (K = H*W*Cin channels) with
// one row of a [No][K] weight matrix.  "MPSCNNBinaryConvolution" (Overview,
// XNOR and AND bullets) defines the binary forms over 32-bit words:
// K - 2*popcount(x ^ w) (XNOR) and popcount(x & w) (AND).
//
// Both are exact integer functions of three counts over the valid bits: the
// product count S_xw = sum_k x_k*w_k of the 0/1 bits, the row count S_x and
// the channel count S_w.  AND is S_xw; XNOR is
//     K - 2*(S_x + S_w - 2*S_xw),  since popcount(x ^ w) = S_x + S_w - 2*S_xw.
// S_xw is a dense contraction of 0/1 values, which the gfx950 matrix cores
// run at their fp4 rate: 0, 0.5, 1 and 2 are exact e2m1 values, a product of
// two of them below is always 0 or 1, and fp32 accumulation of integers below
// 2^24 (K <= 2^24 here) is exact in any order.  Zero bits (the channels past
// Cin of a pixel's last word, and the zero-filled tail of K) add nothing, so
// no correction term is needed for them.
//
// Encoding (v_mfma_f32_16x16x128_f8f6f4 with both operands fp4): lane l of a
// wave holds row (A) or column (B) l % 16 and 32 values of the 128-deep step,
// as 4 dwords of 8 nibbles.  The 32 values of a lane are one 32-bit bit word,
// spread by masks alone: for the activation word x, dword d nibble i holds
// bit 4i + d at nibble position d (values 0.5, 1, 2 for d = 0, 1, 2) and, for
// d = 3, bit 4i + 3 shifted to position 1 (value 1).  The weight table stores
// every word with bits 0 and 2 of each nibble swapped, so its masks give the
// reciprocal values 2, 1, 0.5, 1: every product of two set bits is exactly 1.
// Four mask-and operations and one shift per 32 values on each side.
//
// Mapping on gfx950: M = batch rows, N = output channels, K = words.
//  * A workgroup (8 waves, 2 per SIMD) owns a 64-row x 64-channel block; its
//    waves split K and each holds the whole block as 4 x 4 fragments of
//    16 x 16 fp32 accumulators, so one expanded activation word serves four
//    channel fragments and one weight word four row fragments.
//  * K advances 16 words per step (4 matrix steps of 128 values): each lane
//    loads 16 bytes per fragment (row-major activations; a fragment-ordered
//    weight table), the next step's while the current one computes.
//  * The partial blocks meet in LDS (128 KB, which also keeps one workgroup
//    per compute unit); the block's rows are counted (S_x) during the loop,
//    the channel counts S_w come with the weight table.
//  * Workgroups are dealt to the eight XCDs round-robin; the row blocks of one
//    channel tile run on the same XCD, so its weights cross HBM once.
#include "internal.h"

namespace bconv {
namespace {

constexpr int kF4Waves = 8;  // waves per workgroup (K shares)
constexpr int kF4Rows = 64;  // batch rows per workgroup
constexpr int kF4Xcds = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct F4Args {
    const float *scale, *bias;
    const float *a_pad;     // A map [n][H*W] or nullptr (beta = 1)
    float *beta_out;        // [n]
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;     // packed sign bits instead of out
    int out_words;
    const int32_t *wcount;  // S_w of channel c at wcount[4 c]
    int out_c, hw;
    int kbits;              // valid bits per row (H*W*Cin)
};

// Activation word -> the four fp4 dwords of one lane (values 0.5, 1, 2, 1).
__device__ __forceinline__ v8i spread_x(uint32_t x)
{
    v8i r = {(int)(x & 0x11111111u), (int)(x & 0x22222222u), (int)(x & 0x44444444u), (int)((x >> 2) & 0x22222222u),
             0, 0, 0, 0};
    return r;
}
// Weight word (nibble bits 0 and 2 swapped) -> fp4 dwords (values 2, 1, 0.5, 1).
__device__ __forceinline__ v8i spread_w(uint32_t w)
{
    v8i r = {(int)(w & 0x44444444u), (int)(w & 0x22222222u), (int)(w & 0x11111111u), (int)((w >> 2) & 0x22222222u),
             0, 0, 0, 0};
    return r;
}

__device__ __forceinline__ v4f mma(v8i a, v8i b, v4f c)
{
    // cbsz = blgp = 4: both operands e2m1; zero scale operands select the
    // unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, 0, 0, 0);
}

// One 16-word step: 4 matrix steps x (R row x 4 channel fragments).
template <bool AND, int R>
__device__ __forceinline__ void f4_step(const uint4 (&xa)[R], const uint4 (&wb)[4], v4f (&acc)[R][4],
                                        uint32_t (&rowcnt)[R])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v8i ex[R], ew[4];
#pragma unroll
        for (int f = 0; f < R; ++f) {
            const uint32_t x = j == 0 ? xa[f].x : j == 1 ? xa[f].y : j == 2 ? xa[f].z : xa[f].w;
            ex[f] = spread_x(x);
            if (!AND) rowcnt[f] += __builtin_popcount(x);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t w = j == 0 ? wb[g].x : j == 1 ? wb[g].y : j == 2 ? wb[g].z : wb[g].w;
            ew[g] = spread_w(w);
        }
#pragma unroll
        for (int f = 0; f < R; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[f][g] = mma(ex[f], ew[g], acc[f][g]);
    }
}

// Leading scalar arguments (preloaded in SGPRs) are what the main loop needs.
// bits: activations [n][kw4 * 4] words (rows 16-byte aligned; x_bytes their
// size, reads past it return zero); wtab:
// [tiles][steps][4][64] uint4 (see prepack_f4_kernel); kw4 = K words / 4;
// steps = ceil(kw4 / 4).
template <bool AND>
__global__ __launch_bounds__(64 * kF4Waves) void bgemm_f4_kernel(const uint4 *bits, int x_bytes, const uint4 *wtab,
                                                                 int kw4, int steps, int n, int mblocks, int tiles,
                                                                 F4Args a)
{
    __shared__ v4f part[kF4Waves][16][64];  // partial blocks, fragment order
    __shared__ uint4 rowpart[kF4Waves][16];  // partial S_x of the 64 rows
    __shared__ float rbeta[kF4Rows];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned b = blockIdx.x;
    const unsigned xcd = b % kF4Xcds, local = b / kF4Xcds;
    const unsigned lq = local / (unsigned)mblocks;
    const int mb = (int)(local - lq * (unsigned)mblocks);
    const int tile = (int)(xcd + kF4Xcds * lq);
    if (tile >= tiles) return;  // whole block uniform
    const int m0 = mb * kF4Rows;
    const int r16 = lane & 15, kq = lane >> 4;

    // this wave's steps; the last, partial one (K words not a multiple of 16)
    // is taken after the loop, with its missing word groups masked
    const int t0 = (steps * wave) / kF4Waves, t1 = (steps * (wave + 1)) / kF4Waves;
    const int tfull = kw4 / 4;  // steps whose four word groups all lie inside K
    const int tend = t1 < tfull ? t1 : tfull;
    // lane's 16-byte word group: row m0 + 16f + r16 (the last row stands in
    // for rows past the batch), words 16t + 4kq .. + 3; the step enters as a
    // scalar offset, so every load is issued unconditionally
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(bits, x_bytes);
    uint32_t xoff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int m = m0 + 16 * f + r16 < n ? m0 + 16 * f + r16 : n - 1;
        xoff[f] = ((uint32_t)m * (uint32_t)kw4 + (uint32_t)kq) * 16u;
    }
    const uint4 *wl = wtab + (long long)tile * steps * 256 + lane;

    v4f acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t rowcnt[4] = {0u, 0u, 0u, 0u};

    auto load = [&](int t, uint4 (&xa)[4], uint4 (&wb)[4]) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
            xa[f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[f], (uint32_t)t * 64u, 0));
#pragma unroll
        for (int g = 0; g < 4; ++g) wb[g] = wl[((long long)t * 4 + g) * 64];
    };
    int t = t0;
    if (t0 < tend) {
        // two buffers in turn: step t computes while step t + 1 loads (the
        // last prefetch repeats the final step and goes unused)
        uint4 x0[4], w0[4], x1[4], w1[4];
        load(t, x0, w0);
        for (; t + 1 < tend; t += 2) {
            load(t + 1, x1, w1);
            f4_step<AND, 4>(x0, w0, acc, rowcnt);
            load(t + 2 < tend ? t + 2 : tend - 1, x0, w0);
            f4_step<AND, 4>(x1, w1, acc, rowcnt);
        }
        if (t < tend) {
            f4_step<AND, 4>(x0, w0, acc, rowcnt);
            ++t;
        }
    }
    if (t < t1) {
        // the partial step: word groups past K read zero weights; the
        // activation words there belong to the next row and are cleared
        uint4 xa[4], wb[4];
        load(t, xa, wb);
        if (4 * t + kq >= kw4) {
#pragma unroll
            for (int f = 0; f < 4; ++f) xa[f] = make_uint4(0u, 0u, 0u, 0u);
        }
        f4_step<AND, 4>(xa, wb, acc, rowcnt);
    }

    // beta of the block's rows: mean of the A map over the whole image, in
    // the order of the other kernels (sequential sum, then / (H*W))
    if (a.a_pad && wave == 0) {
        const int m = m0 + lane < n ? m0 + lane : n - 1;
        const float *ap = a.a_pad + (long long)m * a.hw;
        float sum = 0.0f;
        for (int i = 0; i < a.hw; ++i) sum += ap[i];
        const float be = sum / (float)a.hw;
        rbeta[lane] = be;
        if (tile == 0 && m0 + lane < n) a.beta_out[m0 + lane] = be;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) part[wave][f * 4 + g][lane] = acc[f][g];
    if (!AND) {
        // a row's count over the four lane groups, then one lane per row
        uint32_t c[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            c[f] = rowcnt[f];
            c[f] += (uint32_t)__shfl_xor((int)c[f], 16, 64);
            c[f] += (uint32_t)__shfl_xor((int)c[f], 32, 64);
        }
        if (lane < 16) {
            uint32_t *rp = reinterpret_cast<uint32_t *>(&rowpart[wave][0]);
#pragma unroll
            for (int f = 0; f < 4; ++f) rp[16 * f + lane] = c[f];
        }
    }
    __syncthreads();

    // epilogue, by pairs of channel fragments: pair q is row fragment q / 2
    // with channel fragments 2 (q % 2) and 2 (q % 2) + 1, i.e. 32 channels =
    // one output sign-bit word; wave w takes pairs w * kPairs ... ; lane =
    // column r16 of rows 4 kq .. 4 kq + 3 of the fragment
    constexpr int kPairs = 8 / kF4Waves;
#pragma unroll
    for (int pi = 0; pi < kPairs; ++pi) {
        const int q = wave * kPairs + pi;
        const int f = q >> 1;
        const int rbase = 16 * f + 4 * kq;  // first of the lane's 4 rows in the block
        uint4 sx = make_uint4(0u, 0u, 0u, 0u);
        if (!AND) {
#pragma unroll
            for (int w = 0; w < kF4Waves; ++w) {
                const uint4 p = rowpart[w][rbase / 4];
                sx.x += p.x;
                sx.y += p.y;
                sx.z += p.z;
                sx.w += p.w;
            }
        }
        const uint32_t sxr[4] = {sx.x, sx.y, sx.z, sx.w};
        float be[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (a.a_pad) {
#pragma unroll
            for (int j = 0; j < 4; ++j) be[j] = rbeta[rbase + j];
        }
        bool bit[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int g = 2 * (q & 1) + h;
            v4f s = part[0][f * 4 + g][lane];
#pragma unroll
            for (int w = 1; w < kF4Waves; ++w) s += part[w][f * 4 + g][lane];
            const int co = tile * kTile + 16 * g + r16;
            const bool co_ok = co < a.out_c;
            const int sw = co_ok && !AND ? a.wcount[4 * co] : 0;
            const float sc = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
            const float bi = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = m0 + rbase + j;
                const int sxw = (int)s[j];  // exact: an integer below 2^24
                const int v = AND ? sxw : a.kbits - 2 * ((int)sxr[j] + sw - 2 * sxw);
                bit[h][j] = false;
                if (m >= n || !co_ok) continue;
                const long long o = (long long)m * a.out_c + co;
                if (a.acc_out) {
                    store_through(&a.acc_out[o], v);
                    continue;
                }
                const float res = epilogue_value_compact((float)v, sc, be[j], bi, a.neuron);
                if (a.bits_out) {
                    bit[h][j] = sign_bit(res);
                    continue;
                }
                store_through(&a.out[o], res);
            }
        }
        if (a.bits_out) {
            // output word 2 * tile + (q & 1) of each row: low half from the
            // pair's first channel fragment, high half from its second
            const int wi = 2 * tile + (q & 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned long long lo = __ballot(bit[0][j]), hi = __ballot(bit[1][j]);
                // lane c < 4 writes row 4c + j of the fragment
                if (lane < 4 && wi < a.out_words) {
                    const int m = m0 + 16 * f + 4 * lane + j;
                    const uint32_t word = (uint32_t)((lo >> (16 * lane)) & 0xffffu) |
                                          ((uint32_t)((hi >> (16 * lane)) & 0xffffu) << 16);
                    if (m < n) store_through(&a.bits_out[(long long)m * a.out_words + wi], word);
                }
            }
        }
    }
}

// Convolution as an implicit product on the same matrix cores.  Rows are
// output pixels; K runs over the window's taps in (ky, kx) order and, within a
// tap, over the pixel's words, so the weight table above serves unchanged.
// A lane's 16-byte word group G = 4 step + kq is 4 words of one tap pixel of
// the zero-halo bit buffer: its offset from the window's first word comes from
// a table in LDS.  Taps in the padding read zero words and add nothing to
// S_xw or S_x; XNOR then needs S_w over the window's in-image taps only, a
// rectangle of taps whose count comes from per-channel 2-D prefix sums.
struct CF4Args {
    const float *scale, *bias;
    const float *a_pad;     // zero-halo A map [n][rows][cols] or nullptr (beta = 1)
    float *beta_out;        // [n][out_h][out_w]
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;     // packed sign bits instead of out
    int out_words;
    const int32_t *wrect;   // per channel: set weight bits of taps [0,y) x [0,x) at y*(kw+1)+x
    int out_c, in_c, in_h, in_w, out_h, out_w;
    int kh, kw, sh, sw, ph, pw, rows, cols, words;
    int beta_valid;         // beta divides by the in-image tap count
    FastDiv div_ohw, div_ow;
};

constexpr int kCF4Waves = 4;         // waves per workgroup
constexpr int kCF4R = 2;             // row fragments (16 pixels each) per wave
constexpr int kCF4MaxGroups = 1024;  // word groups per window
constexpr int kCF4MaxRect = 128;     // prefix-table entries per channel, (kh+1)*(kw+1)
constexpr int kCF4BetaTaps = 25;     // beta windows up to this many taps load all taps at once

// Pixel m -> (image, oy, ox).
__device__ __forceinline__ void cf4_pixel(const CF4Args &a, int m, int &img, int &oy, int &ox)
{
    img = (int)fastdiv((uint32_t)m, a.div_ohw);
    const int rem = m - img * a.out_h * a.out_w;
    oy = (int)fastdiv((uint32_t)rem, a.div_ow);
    ox = rem - oy * a.out_w;
}

// Leading scalar arguments (preloaded in SGPRs) are what the main loop needs.
// bits: the zero-halo bit buffer (bits_bytes long, reads past it return
// zero); wtab: the weight table; groups = kh*kw*words/4; npix = n*out_h*out_w.
// Every global load the epilogue needs (scale, bias, the beta window) is
// issued before the main loop and the prefix table sits in LDS, so the
// epilogue waits on nothing but arithmetic.
template <bool AND>
__global__ __launch_bounds__(64 * kCF4Waves) void xconv_f4_kernel(const uint32_t *bits, int bits_bytes,
                                                                  const uint4 *wtab, int groups, int steps, int npix,
                                                                  int tiles, CF4Args a)
{
    constexpr int R = kCF4R;
    __shared__ int goff[kCF4MaxGroups];  // word offset of group G from the window's first word
    __shared__ int prect[AND ? 1 : 64 * (kCF4MaxRect + 1)];  // the tile's channels' prefix tables
    __shared__ int aoff[kCF4BetaTaps];   // A-map offset of tap t from the window's first entry
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = (int)(blockIdx.x % (unsigned)tiles);
    const int m0 = (int)(blockIdx.x / (unsigned)tiles) * (16 * R * kCF4Waves) + 16 * R * wave;
    const int E = (a.kh + 1) * (a.kw + 1);
    const int ES = E | 1;  // odd row length: lanes 16 rows apart fall in different banks
    const int taps = a.kh * a.kw;
    {
        const int wpt = a.words / 4;
        for (int G = threadIdx.x; G < groups; G += 64 * kCF4Waves) {
            const int t = G / wpt, sub = G - t * wpt;
            const int ky = t / a.kw, kx = t - ky * a.kw;
            goff[G] = (ky * a.cols + kx) * a.words + 4 * sub;
        }
        if (!AND) {
            for (int i = threadIdx.x; i < 64 * E; i += 64 * kCF4Waves) {
                const int c = i / E, co = tile * kTile + c;
                prect[c * ES + (i - c * E)] = co < a.out_c ? a.wrect[(long long)co * E + (i - c * E)] : 0;
            }
        }
        if ((int)threadIdx.x < taps && taps <= kCF4BetaTaps) {
            const int ky = (int)threadIdx.x / a.kw, kx = (int)threadIdx.x - ky * a.kw;
            aoff[threadIdx.x] = ky * a.cols + kx;
        }
    }
    const int r16 = lane & 15, kq = lane >> 4;
    // channel constants of the lane's four channel fragments (requested now,
    // used by the epilogue)
    float sc[4], bi[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int co = tile * kTile + 16 * g + r16;
        const bool co_ok = co < a.out_c;
        sc[g] = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
        bi[g] = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;
    }
    uint32_t wbase[R];  // byte offset of the window's first word, pixels m0 + 16 f + r16
#pragma unroll
    for (int f = 0; f < R; ++f) {
        const int m = m0 + 16 * f + r16 < npix ? m0 + 16 * f + r16 : npix - 1;
        int img, oy, ox;
        cf4_pixel(a, m, img, oy, ox);
        wbase[f] = (uint32_t)(((img * a.rows + oy * a.sh) * a.cols + ox * a.sw) * a.words) * 4u;
    }
    __syncthreads();
    // the beta window of pixel m0 + lane (lanes < 16 R): all taps requested
    // now, summed after the main loop in the order of the generic kernel
    const bool beta_lane = a.a_pad != nullptr && lane < 16 * R;
    const int mb = m0 + lane < npix ? m0 + lane : npix - 1;
    const float *apw = nullptr;
    float av[kCF4BetaTaps];
    if (beta_lane) {
        int img, oy, ox;
        cf4_pixel(a, mb, img, oy, ox);
        apw = a.a_pad + ((long long)img * a.rows + oy * a.sh) * a.cols + ox * a.sw;
        if (taps <= kCF4BetaTaps) {
#pragma unroll
            for (int t = 0; t < kCF4BetaTaps; ++t) av[t] = t < taps ? apw[aoff[t]] : 0.0f;
        }
    }

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(bits, bits_bytes);
    const uint4 *wl = wtab + (long long)tile * steps * 256 + lane;
    v4f acc[R][4];
#pragma unroll
    for (int f = 0; f < R; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t rowcnt[R];
#pragma unroll
    for (int f = 0; f < R; ++f) rowcnt[f] = 0u;

    // every load is issued; groups past the window read offset 0 and are
    // cleared after they arrive
    auto load = [&](int t, uint4 (&xa)[R], uint4 (&wb)[4], bool &live) {
        const int G = 4 * t + kq;
        live = G < groups;
        const uint32_t off = (uint32_t)goff[live ? G : 0] * 4u;
#pragma unroll
        for (int f = 0; f < R; ++f)
            xa[f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, wbase[f] + off, 0, 0));
#pragma unroll
        for (int g = 0; g < 4; ++g) wb[g] = wl[((long long)t * 4 + g) * 64];
    };
    auto clear_dead = [](uint4 (&xa)[R], bool live) {
#pragma unroll
        for (int f = 0; f < R; ++f)
            if (!live) xa[f] = make_uint4(0u, 0u, 0u, 0u);
    };
    {
        uint4 x0[R], w0[4], x1[R], w1[4];
        bool l0, l1;
        int t = 0;
        load(0, x0, w0, l0);
        for (; t + 1 < steps; t += 2) {
            load(t + 1, x1, w1, l1);
            clear_dead(x0, l0);
            f4_step<AND, R>(x0, w0, acc, rowcnt);
            load(t + 2 < steps ? t + 2 : steps - 1, x0, w0, l0);
            clear_dead(x1, l1);
            f4_step<AND, R>(x1, w1, acc, rowcnt);
        }
        if (t < steps) {
            clear_dead(x0, l0);
            f4_step<AND, R>(x0, w0, acc, rowcnt);
        }
    }

    float beta_l = 1.0f;
    if (beta_lane) {
        int img, oy, ox;
        cf4_pixel(a, mb, img, oy, ox);
        float sum = 0.0f;
        if (taps <= kCF4BetaTaps) {
#pragma unroll
            for (int t = 0; t < kCF4BetaTaps; ++t)
                if (t < taps) sum += av[t];
        } else {
            for (int ky = 0; ky < a.kh; ++ky)
                for (int kx = 0; kx < a.kw; ++kx) sum += apw[ky * a.cols + kx];
        }
        beta_l = sum / (float)(a.beta_valid ? window_valid_taps(oy, ox, a.sh, a.sw, a.ph, a.pw, a.kh, a.kw, a.in_h,
                                                                a.in_w)
                                           : taps);
        if (tile == 0 && m0 + lane < npix) a.beta_out[m0 + lane] = beta_l;
    }
    // a row's S_x over the four lane groups
    uint32_t sxl[R];
#pragma unroll
    for (int f = 0; f < R; ++f) {
        sxl[f] = rowcnt[f];
        if (!AND) {
            sxl[f] += (uint32_t)__shfl_xor((int)sxl[f], 16, 64);
            sxl[f] += (uint32_t)__shfl_xor((int)sxl[f], 32, 64);
        }
    }

    // epilogue: lane = column r16 of rows 4 kq .. 4 kq + 3 of each fragment;
    // channel fragments in pairs (one output sign-bit word each)
#pragma unroll
    for (int f = 0; f < R; ++f) {
        int sx[4], kvalid[4], y0[4], y1[4], x0[4], x1[4];
        bool inner[4];
        float be[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * kq + j;  // row in the fragment
            sx[j] = (int)__shfl((int)sxl[f], r, 64);
            be[j] = __shfl(beta_l, 16 * f + r, 64);
            const int m = m0 + 16 * f + r < npix ? m0 + 16 * f + r : npix - 1;
            int img, oy, ox;
            cf4_pixel(a, m, img, oy, ox);
            const int iy0 = oy * a.sh - a.ph, ix0 = ox * a.sw - a.pw;
            y0[j] = iy0 < 0 ? -iy0 : 0;
            y1[j] = a.in_h - iy0 < a.kh ? a.in_h - iy0 : a.kh;
            x0[j] = ix0 < 0 ? -ix0 : 0;
            x1[j] = a.in_w - ix0 < a.kw ? a.in_w - ix0 : a.kw;
            kvalid[j] = a.in_c * (y1[j] - y0[j]) * (x1[j] - x0[j]);
            inner[j] = y0[j] == 0 && x0[j] == 0 && y1[j] == a.kh && x1[j] == a.kw;
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            bool bit[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = 2 * pr + h;
                const int co = tile * kTile + 16 * g + r16;
                const bool co_ok = co < a.out_c;
                const int *P = prect + (AND ? 0 : (16 * g + r16) * ES);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = m0 + 16 * f + 4 * kq + j;
                    const int sxw = (int)acc[f][g][j];  // exact: an integer below 2^24
                    int v = sxw;
                    if (!AND) {
                        const int w1 = a.kw + 1;
                        const int swv = inner[j] ? P[E - 1]
                                                 : P[y1[j] * w1 + x1[j]] - P[y0[j] * w1 + x1[j]] -
                                                       P[y1[j] * w1 + x0[j]] + P[y0[j] * w1 + x0[j]];
                        v = kvalid[j] - 2 * (sx[j] + swv - 2 * sxw);
                    }
                    bit[h][j] = false;
                    if (m >= npix || !co_ok) continue;
                    const long long o = (long long)m * a.out_c + co;
                    if (a.acc_out) {
                        store_through(&a.acc_out[o], v);
                        continue;
                    }
                    const float res = epilogue_value_compact((float)v, sc[g], be[j], bi[g], a.neuron);
                    if (a.bits_out) {
                        bit[h][j] = sign_bit(res);
                        continue;
                    }
                    store_through(&a.out[o], res);
                }
            }
            if (a.bits_out) {
                const int wi = 2 * tile + pr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned long long lo = __ballot(bit[0][j]), hi = __ballot(bit[1][j]);
                    // lane c < 4 writes row 4c + j of the fragment
                    if (lane < 4 && wi < a.out_words) {
                        const int m = m0 + 16 * f + 4 * lane + j;
                        const uint32_t word = (uint32_t)((lo >> (16 * lane)) & 0xffffu) |
                                              ((uint32_t)((hi >> (16 * lane)) & 0xffffu) << 16);
                        if (m < npix) store_through(&a.bits_out[(long long)m * a.out_words + wi], word);
                    }
                }
            }
        }
    }
}

// Weight table: [tiles][steps][4][64] uint4.  Entry (tile, t, g, lane) holds
// words 16t + 4(lane / 16) .. + 3 of channel 64 tile + 16 g + lane % 16 (k =
// (ky*kw + kx)*words + w), bits >= in_c of each pixel's last word cleared,
// zero past K and for channels >= out_c, and bits 0 and 2 of every nibble
// swapped (the reciprocal encoding above).
__global__ void prepack_f4_kernel(const uint32_t *__restrict__ user, uint4 *__restrict__ tab, int out_c, int K,
                                  int words, int in_c, int tiles, int steps)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)tiles * steps * 256;
    if (t >= total) return;
    const int lane = (int)(t % 64);
    const int g = (int)((t / 64) % 4);
    const int step = (int)((t / 256) % steps);
    const int tile = (int)(t / (256LL * steps));
    const int co = tile * kTile + 16 * g + lane % 16;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = 16 * step + 4 * (lane / 16) + j;
        uint32_t x = 0;
        if (co < out_c && k < K) {
            x = user[(long long)co * K + k];
            const int tail = in_c - 32 * (k % words);
            if (tail < 32) x &= (tail <= 0) ? 0u : ((1u << tail) - 1u);
        }
        v[j] = (x & 0xAAAAAAAAu) | ((x & 0x11111111u) << 2) | ((x >> 2) & 0x11111111u);
    }
    tab[t] = make_uint4(v[0], v[1], v[2], v[3]);
}

// Set bits of each channel's valid weight bits (0 past out_c), as 2-D prefix
// sums over the taps: entry y*(qw+1)+x counts taps [0,y) x [0,x).  With qh =
// qw = 1 (the fully connected route) the one tap is the whole window and the
// entry 3 the total.
__global__ void weight_count_kernel(const uint32_t *__restrict__ user, int32_t *__restrict__ cnt, int out_c, int K,
                                    int words, int in_c, int channels, int qh, int qw)
{
    const int co = blockIdx.x * blockDim.x + threadIdx.x;
    if (co >= channels) return;
    const int E = (qh + 1) * (qw + 1);
    int32_t *P = cnt + (long long)co * E;
    const int tap_words = K / (qh * qw);
    for (int x = 0; x <= qw; ++x) P[x] = 0;
    for (int y = 0; y < qh; ++y) {
        P[(y + 1) * (qw + 1)] = 0;
        int row = 0;  // taps [y] x [0, x)
        for (int x = 0; x < qw; ++x) {
            int s = 0;
            if (co < out_c) {
                for (int i = 0; i < tap_words; ++i) {
                    const int k = (y * qw + x) * tap_words + i;
                    uint32_t v = user[(long long)co * K + k];
                    const int tail = in_c - 32 * (k % words);
                    if (tail < 32) v &= (tail <= 0) ? 0u : ((1u << tail) - 1u);
                    s += __builtin_popcount(v);
                }
            }
            row += s;
            P[(y + 1) * (qw + 1) + x + 1] = P[y * (qw + 1) + x + 1] + row;
        }
    }
}

int f4_groups(const Geom &g) { return g.kh * g.kw * g.words / 4; }
int f4_steps(const Geom &g) { return (f4_groups(g) + 3) / 4; }
// taps of the count table: the whole window as one tap for the product route
int f4_qh(const Geom &g) { return gemm_route(g) ? 1 : g.kh; }
int f4_qw(const Geom &g) { return gemm_route(g) ? 1 : g.kw; }
size_t f4_table_bytes(const Geom &g) { return (size_t)g.tiles * f4_steps(g) * 256 * 16; }

}  // namespace

bool f4_route(const Geom &g)
{
    if ((g.kh * g.kw * g.words) % 4 != 0) return false;  // 16-byte word groups within a tap or row
    if (gemm_route(g)) return true;
    return (g.words % 4) == 0 && f4_groups(g) <= kCF4MaxGroups && (g.kh + 1) * (g.kw + 1) <= kCF4MaxRect;
}

size_t f4_bytes(const Geom &g)
{
    return f4_table_bytes(g) + (size_t)g.tiles * kTile * (f4_qh(g) + 1) * (f4_qw(g) + 1) * 4;
}

hipError_t launch_prepack_f4(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *tab)
{
    const int K = g.kh * g.kw * g.words;
    const int steps = f4_steps(g);
    const long long total = (long long)g.tiles * steps * 256;
    uint4 *t = static_cast<uint4 *>(tab);
    int32_t *cnt = reinterpret_cast<int32_t *>(static_cast<char *>(tab) + f4_table_bytes(g));
    hipLaunchKernelGGL(prepack_f4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, user_bits, t,
                       g.out_c, K, g.words, g.in_c, g.tiles, steps);
    const int channels = g.tiles * kTile;
    hipLaunchKernelGGL(weight_count_kernel, dim3((unsigned)((channels + 63) / 64)), dim3(64), 0, s, user_bits, cnt,
                       g.out_c, K, g.words, g.in_c, channels, f4_qh(g), f4_qw(g));
    return hipGetLastError();
}

const char *f4_kernel_name(const Geom &g, int and_mode)
{
    if (gemm_route(g)) return and_mode ? "bgemm_f4_kernel<true>" : "bgemm_f4_kernel<false>";
    return and_mode ? "xconv_f4_kernel<true>" : "xconv_f4_kernel<false>";
}

namespace {

hipError_t launch_gemm_f4(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const void *tab,
                          const Epilogue &e, float *out, int32_t *acc_out)
{
    const int K = g.kh * g.kw * g.words;
    const int steps = f4_steps(g);
    F4Args a{};
    a.scale = e.scale;
    a.bias = e.bias;
    a.a_pad = e.a_pad;
    a.beta_out = e.beta_out;
    a.scale_value = e.scale_value;
    a.neuron = e.neuron;
    a.out = out;
    a.acc_out = acc_out;
    a.bits_out = e.bits_out;
    a.out_words = e.out_words;
    // totals: entry 3 of each channel's 2 x 2 prefix table
    a.wcount = reinterpret_cast<const int32_t *>(static_cast<const char *>(tab) + f4_table_bytes(g)) + 3;
    a.out_c = g.out_c;
    a.hw = g.in_h * g.in_w;
    a.kbits = g.in_c * g.kh * g.kw;
    const int mblocks = (g.n + kF4Rows - 1) / kF4Rows;
    const long long tiles_per_xcd = (g.tiles + kF4Xcds - 1) / kF4Xcds;
    const long long blocks = (long long)kF4Xcds * tiles_per_xcd * mblocks;
    if (blocks == 0) return hipSuccess;
    const long long x_bytes = (long long)g.n * K * 4;
    if (blocks > 0x7fffffffLL || (K & 3) != 0 || x_bytes > 0x7fffffffLL) return hipErrorInvalidValue;
    const uint4 *x = reinterpret_cast<const uint4 *>(bits);
    const uint4 *w = static_cast<const uint4 *>(tab);
    auto go = [&](auto kernel) {
        return launch_kernel(L, kernel, dim3((unsigned)blocks), dim3(64 * kF4Waves), 0, x, (int)x_bytes, w, K / 4,
                             steps, g.n, mblocks, g.tiles, a);
    };
    return and_mode ? go(bgemm_f4_kernel<true>) : go(bgemm_f4_kernel<false>);
}

hipError_t launch_xconv_f4(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const void *tab,
                           const Epilogue &e, float *out, int32_t *acc_out)
{
    CF4Args a{};
    a.scale = e.scale;
    a.bias = e.bias;
    a.a_pad = e.a_pad;
    a.beta_out = e.beta_out;
    a.scale_value = e.scale_value;
    a.neuron = e.neuron;
    a.out = out;
    a.acc_out = acc_out;
    a.bits_out = e.bits_out;
    a.out_words = e.out_words;
    a.wrect = reinterpret_cast<const int32_t *>(static_cast<const char *>(tab) + f4_table_bytes(g));
    a.out_c = g.out_c;
    a.in_c = g.in_c;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.out_h = g.out_h;
    a.out_w = g.out_w;
    a.kh = g.kh;
    a.kw = g.kw;
    a.sh = g.sh;
    a.sw = g.sw;
    a.ph = g.ph;
    a.pw = g.pw;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    a.words = g.words;
    a.beta_valid = e.beta_valid_taps;
    a.div_ohw = make_fastdiv((uint32_t)(g.out_h * g.out_w));
    a.div_ow = make_fastdiv((uint32_t)g.out_w);
    const long long npix = (long long)g.n * g.out_h * g.out_w;
    const long long bits_bytes = ((long long)g.n * g.bits_rows * g.bits_cols * g.words + g.bits_slack_words) * 4;
    const long long mblocks = (npix + 16 * kCF4R * kCF4Waves - 1) / (16 * kCF4R * kCF4Waves);
    const long long blocks = mblocks * g.tiles;
    if (npix == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL || bits_bytes > 0x7fffffffLL || !f4_route(g)) return hipErrorInvalidValue;
    auto go = [&](auto kernel) {
        return launch_kernel(L, kernel, dim3((unsigned)blocks), dim3(64 * kCF4Waves), 0, bits, (int)bits_bytes,
                             static_cast<const uint4 *>(tab), f4_groups(g), f4_steps(g), (int)npix, g.tiles, a);
    };
    return and_mode ? go(xconv_f4_kernel<true>) : go(xconv_f4_kernel<false>);
}

}  // namespace

hipError_t launch_f4(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const void *tab,
                     const Epilogue &e, float *out, int32_t *acc_out)
{
    if (gemm_route(g)) return launch_gemm_f4(g, L, and_mode, bits, tab, e, out, acc_out);
    return launch_xconv_f4(g, L, and_mode, bits, tab, e, out, acc_out);
}

}  // namespace bconv
