// Binary matrix product of the fully connected layer on the fp4 matrix cores.
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
    const int32_t *wcount;  // S_w per channel [tiles * 64]
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

// One 16-word step: 4 matrix steps x (4 row x 4 channel fragments).
template <bool AND>
__device__ __forceinline__ void f4_step(const uint4 (&xa)[4], const uint4 (&wb)[4], v4f (&acc)[4][4],
                                        uint32_t (&rowcnt)[4])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v8i ex[4], ew[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
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
        for (int f = 0; f < 4; ++f)
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
            f4_step<AND>(x0, w0, acc, rowcnt);
            load(t + 2 < tend ? t + 2 : tend - 1, x0, w0);
            f4_step<AND>(x1, w1, acc, rowcnt);
        }
        if (t < tend) {
            f4_step<AND>(x0, w0, acc, rowcnt);
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
        f4_step<AND>(xa, wb, acc, rowcnt);
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
            const int sw = co_ok && !AND ? a.wcount[co] : 0;
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
                const float res = epilogue_value((float)v, sc, be[j], bi, a.neuron);
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

// S_w: set bits of each channel's valid weight bits (0 past out_c).
__global__ void weight_count_kernel(const uint32_t *__restrict__ user, int32_t *__restrict__ cnt, int out_c, int K,
                                    int words, int in_c, int channels)
{
    const int co = blockIdx.x * blockDim.x + threadIdx.x;
    if (co >= channels) return;
    int s = 0;
    if (co < out_c) {
        for (int k = 0; k < K; ++k) {
            uint32_t x = user[(long long)co * K + k];
            const int tail = in_c - 32 * (k % words);
            if (tail < 32) x &= (tail <= 0) ? 0u : ((1u << tail) - 1u);
            s += __builtin_popcount(x);
        }
    }
    cnt[co] = s;
}

int f4_steps(const Geom &g)
{
    const int K = g.kh * g.kw * g.words;
    return (K / 4 + 3) / 4;
}

}  // namespace

bool gemm_f4_route(const Geom &g)
{
    // rows of the bit buffer must be 16-byte aligned
    return gemm_route(g) && (g.kh * g.kw * g.words) % 4 == 0;
}

size_t gemm_f4_bytes(const Geom &g)
{
    return (size_t)g.tiles * f4_steps(g) * 256 * 16 + (size_t)g.tiles * kTile * 4;
}

hipError_t launch_prepack_f4(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *tab)
{
    const int K = g.kh * g.kw * g.words;
    const int steps = f4_steps(g);
    const long long total = (long long)g.tiles * steps * 256;
    uint4 *t = static_cast<uint4 *>(tab);
    int32_t *cnt = reinterpret_cast<int32_t *>(t + total);
    hipLaunchKernelGGL(prepack_f4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, user_bits, t,
                       g.out_c, K, g.words, g.in_c, g.tiles, steps);
    const int channels = g.tiles * kTile;
    hipLaunchKernelGGL(weight_count_kernel, dim3((unsigned)((channels + 63) / 64)), dim3(64), 0, s, user_bits, cnt,
                       g.out_c, K, g.words, g.in_c, channels);
    return hipGetLastError();
}

const char *gemm_f4_kernel_name(int and_mode)
{
    return and_mode ? "bgemm_f4_kernel<true>" : "bgemm_f4_kernel<false>";
}

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
    a.wcount = reinterpret_cast<const int32_t *>(static_cast<const uint4 *>(tab) + (long long)g.tiles * steps * 256);
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

}  // namespace bconv
