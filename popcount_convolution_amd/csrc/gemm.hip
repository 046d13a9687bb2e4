// Binary matrix product for the fully connected layer.
//
// Apple "MPSCNNFullyConnected" (Overview, conditions, matrix view): with the
// kernel the size of the source image, stride 1 and no padding, every output
// is the dot product of the NHWC-flattened image (K = H*W*Cin channels) with
// one row of a [No][K] weight matrix.  In the binary forms of
// "MPSCNNBinaryConvolution" (Overview, XNOR and AND bullets) that product is
// K - 2*popcount(x ^ w) summed over 32-bit words (XNOR) or popcount(x & w)
// (AND); the fused epilogue then applies scale*beta + bias and the neuron.
//
// Mapping on gfx950: M = batch rows, N = output channels, K = words.
//  * A workgroup owns a tile of 64 channels (one per lane) by MR = 8 rows; its
//    eight waves each take an eighth of K and the partial sums meet in LDS,
//    where each wave then finishes one of the rows (sum, epilogue, store).
//  * A row's activation words are the same for every lane: scalar loads
//    bring MR rows x 4 words into SGPRs per step and v_xor/v_and take them as
//    the scalar operand; the lane's 4 weight words come from a K-major table
//    with one 16-byte load per lane (256 contiguous bytes per wave).  Eight
//    rows keep a wave's registers small enough for eight waves per SIMD
//    (2048 workgroups for the 256 x 4096 layer), which hides the per-step
//    memory round trip far better than 16 rows at four waves per SIMD.
//  * Workgroups are numbered so that each of the eight XCDs (workgroups are
//    dealt to them round-robin) owns an eighth of the channel tiles, keeping
//    its share of the weight matrix in its own L2, and so that the workgroups
//    a compute unit receives together share one row group: their activation
//    words then hit in the scalar cache.
#include "internal.h"

namespace bconv {
namespace {

typedef const uint32_t __attribute__((address_space(4))) *scalar_u32_ptr;

constexpr int kMR = 8;    // batch rows per workgroup
constexpr int kWaves = 8; // waves per workgroup (K eighths)
constexpr int kXcds = 8;  // workgroup dealing period across XCDs

struct GArgs {
    const uint32_t *bits;   // activations [n][K] words (the unpadded bit buffer)
    const uint32_t *wflat;  // [tiles][k4][64][4], k4 = ceil(K/4)
    const float *scale, *bias;
    const float *a_pad;     // A map [n][H*W] or nullptr (beta = 1)
    float *beta_out;        // [n]
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;     // packed sign bits instead of out (see Epilogue)
    int out_words;
    int n, K, k4, out_c, tiles, mgroups, hw, in_c;
    int kbits;              // valid bits per row (H*W*Cin)
};

// The leading scalar arguments (a.bits, a.wflat, the divisor by a.mgroups,
// a.mgroups, a.tiles, a.k4, a.n, a.K) are what the main loop needs; they
// arrive preloaded in SGPRs, so the first loads go out before the argument
// struct (needed only by the epilogue) is fetched.
template <bool AND>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4))) void bgemm_kernel(
    const uint32_t *bits, const uint32_t *wflat, uint32_t mg_m, int mg_s, uint32_t mg_id, int mgroups, int tiles,
    int k4, int n, int K, GArgs a)
{
    constexpr int kRowsPerWave = kMR / kWaves;
    __shared__ int32_t part[kWaves][kMR][64];
    __shared__ float rbeta[kMR];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD-aware numbering: block b runs on XCD b % 8.  XCD x owns the channel
    // tiles x, x+8, x+16, ...; consecutive blocks of one XCD (which its
    // dispatcher spreads over its compute units) walk the row groups of one
    // tile, so the blocks a compute unit holds at once share their rows.
    const unsigned b = blockIdx.x;
    const unsigned xcd = b % kXcds, local = b / kXcds;
    const unsigned lq = fastdiv(local, FastDiv{mg_m, mg_s, mg_id});
    const unsigned mg = local - lq * (unsigned)mgroups;
    const unsigned tile = xcd + kXcds * lq;
    if (tile >= (unsigned)tiles) return;  // whole block uniform
    const int m0 = mg * kMR;

    // this wave's share of the K steps (4 words per step)
    const int steps = k4;
    const int q0 = (steps * wave) / kWaves, q1 = (steps * (wave + 1)) / kWaves;

    uint32_t acc[kMR];
#pragma unroll
    for (int r = 0; r < kMR; ++r) acc[r] = 0;
    const uint4 *wl = reinterpret_cast<const uint4 *>(wflat) + (long long)tile * steps * 64 + lane;
    // rows past the batch read the last row (their results are not stored)
    const int rows_valid = n - m0 < kMR ? n - m0 : kMR;
    const scalar_u32_ptr blk = (scalar_u32_ptr)bits + (long long)m0 * K;
    const int qfull = K / 4 < q1 ? K / 4 : q1;  // steps with 4 words inside K

    if (rows_valid == kMR) {
        for (int q = q0; q < qfull; ++q) {
            const uint4 wv = wl[(long long)q * 64];
            const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int r = 0; r < kMR; ++r) {
                const scalar_u32_ptr xr = blk + r * K + q * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[r] += __builtin_popcount(AND ? (xr[j] & w[j]) : (xr[j] ^ w[j]));
            }
        }
    } else {
        for (int q = q0; q < qfull; ++q) {
            const uint4 wv = wl[(long long)q * 64];
            const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int r = 0; r < kMR; ++r) {
                const int rr = r < rows_valid ? r : rows_valid - 1;
                const scalar_u32_ptr xr = blk + rr * K + q * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[r] += __builtin_popcount(AND ? (xr[j] & w[j]) : (xr[j] ^ w[j]));
            }
        }
    }
    // last, partial step (K not a multiple of 4): words past K are zero on both sides
    for (int q = qfull > q0 ? qfull : q0; q < q1; ++q) {
        const uint4 wv = wl[(long long)q * 64];
        const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int r = 0; r < kMR; ++r) {
            const int rr = r < rows_valid ? r : rows_valid - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t x = (q * 4 + j < K) ? blk[rr * K + q * 4 + j] : 0u;
                acc[r] += __builtin_popcount(AND ? (x & w[j]) : (x ^ w[j]));
            }
        }
    }

    // beta of the block's rows: mean of the A map over the whole image
    if (a.a_pad && wave == 0 && lane < kMR) {
        const int m = m0 + lane < a.n ? m0 + lane : a.n - 1;
        const float *ap = a.a_pad + (long long)m * a.hw;
        float sum = 0.0f;
        for (int i = 0; i < a.hw; ++i) sum += ap[i];
        const float be = sum / (float)a.hw;
        rbeta[lane] = be;
        if (tile == 0 && m0 + lane < a.n) a.beta_out[m0 + lane] = be;
    }
#pragma unroll
    for (int r = 0; r < kMR; ++r) part[wave][r][lane] = (int32_t)acc[r];
    __syncthreads();
    // wave w finishes rows w*kRowsPerWave ... (the sum over the K shares in a
    // fixed order, then the epilogue)
    const int co = tile * kTile + lane;
    const bool co_ok = co < a.out_c;
    if (!co_ok && !a.bits_out) return;  // the sign-bit path needs every lane
    const float sc = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
    const float bi = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        const int r = wave * kRowsPerWave + i;
        if (m0 + r >= a.n) break;
        int s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += part[w][r][lane];
        const int v = AND ? s : a.kbits - 2 * s;
        const long long o = (long long)(m0 + r) * a.out_c + co;
        if (a.acc_out) {
            __hip_atomic_store(&a.acc_out[o], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        const float be = a.a_pad ? rbeta[r] : 1.0f;
        const float res = epilogue_value((float)v, sc, be, bi, a.neuron);
        if (a.bits_out) {
            store_tile_bits(a.bits_out, m0 + r, a.out_words, (int)tile, co_ok && sign_bit(res));
            continue;
        }
        __hip_atomic_store(&a.out[o], res, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// [tiles][k4][64][4] K-major weight words (k = (ky*kw + kx)*words + w), bits
// >= in_c cleared, zero past K and for channels >= out_c.
__global__ void prepack_flat_kernel(const uint32_t *__restrict__ user, uint32_t *__restrict__ flat, int out_c,
                                    int K, int words, int in_c, int tiles, int k4)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)tiles * k4 * 256;
    if (t >= total) return;
    const int j = (int)(t % 4);
    const int lane = (int)((t / 4) % 64);
    const int q = (int)((t / 256) % k4);
    const int tile = (int)(t / (256LL * k4));
    const int k = q * 4 + j;
    const int co = tile * kTile + lane;
    uint32_t v = 0;
    if (co < out_c && k < K) {
        v = user[(long long)co * K + k];
        const int w = k % words;
        const int tail = in_c - 32 * w;
        if (tail < 32) v &= (tail <= 0) ? 0u : ((1u << tail) - 1u);
    }
    flat[t] = v;
}

}  // namespace

bool gemm_route(const Geom &g)
{
    return g.kh == g.in_h && g.kw == g.in_w && g.sh == 1 && g.sw == 1 && g.ph == 0 && g.pw == 0 &&
           g.bits_rows == g.in_h && g.bits_cols == g.in_w;  // no trailing padding either
}

size_t gemm_weight_words(const Geom &g)
{
    const long long K = (long long)g.kh * g.kw * g.words;
    return (size_t)g.tiles * ((K + 3) / 4) * 256;
}

hipError_t launch_prepack_flat(const Geom &g, hipStream_t s, const uint32_t *user_bits, uint32_t *flat)
{
    const int K = g.kh * g.kw * g.words;
    const int k4 = (K + 3) / 4;
    const long long total = (long long)g.tiles * k4 * 256;
    hipLaunchKernelGGL(prepack_flat_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, user_bits, flat,
                       g.out_c, K, g.words, g.in_c, g.tiles, k4);
    return hipGetLastError();
}

const char *gemm_kernel_name(const Geom &, int and_mode)
{
    return and_mode ? "bgemm_kernel<true>" : "bgemm_kernel<false>";
}

hipError_t launch_gemm(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits, const uint32_t *wflat,
                       const Epilogue &e, float *out, int32_t *acc_out)
{
    GArgs a{};
    a.bits = bits;
    a.wflat = wflat;
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
    a.n = g.n;
    a.K = g.kh * g.kw * g.words;
    a.k4 = (a.K + 3) / 4;
    a.out_c = g.out_c;
    a.tiles = g.tiles;
    a.mgroups = (g.n + kMR - 1) / kMR;
    a.hw = g.in_h * g.in_w;
    a.in_c = g.in_c;
    a.kbits = g.in_c * g.kh * g.kw;
    const long long tiles_per_xcd = (g.tiles + kXcds - 1) / kXcds;
    const long long blocks = (long long)kXcds * tiles_per_xcd * a.mgroups;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const FastDiv dm = make_fastdiv((uint32_t)a.mgroups);
    auto go = [&](auto kernel) {
        return launch_kernel(L, kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, a.bits, a.wflat, dm.m, dm.s,
                             dm.id, a.mgroups, a.tiles, a.k4, a.n, a.K, a);
    };
    return and_mode ? go(bgemm_kernel<true>) : go(bgemm_kernel<false>);
}

}  // namespace bconv
