// Create-time weight rearrangement.
//
// The binary weights B[c, ky, kx, f] of Apple "MPSCNNBinaryConvolution"
// (Overview, symbol definitions) arrive as uint32 words
// [out_c][kh][kw][words], channel f at bit f%32 of word f/32.  The kernels
// read them as:
//   * lane words [tiles][kh][kwc4][64][4] (word r = kx*words + w of row ky,
//     kwc4 = ceil(kw*words/4)): lane l of tile t owns output channel 64t + l,
//     so a wave loads 256 contiguous bytes per 4 words; bits >= in_c are
//     cleared, padding channels and r >= kw*words are 0;
//   * a per-lane 2-D prefix sum of the tap popcounts,
//     rect[tiles][64][(kh+1)*R] (R = kw+1 rounded up to 4, padding 0),
//     entry a*R + b = set bits of the cleared words of taps ky < a, kx < b;
//     lane-major so a lane reads a table row with whole 16-byte loads.  It serves the XNOR border correction: a
//     zero input word at a padded tap counts every set weight bit as a
//     disagreement, and those bits are total - (in-image rectangle);
//   * binaryWeights: +-1.0f [kh*kw*in_c][pm_cols] (zero for channels >=
//     out_c), the weight value the page assigns to bits 1 and 0.
#include "internal.h"

namespace bconv {
namespace {

__device__ __forceinline__ uint32_t cleared_word(const uint32_t *user, int co, int tap, int w,
                                                 int taps, int words, int in_c)
{
    uint32_t v = user[((long long)co * taps + tap) * words + w];
    const int tail = in_c - 32 * w;  // valid bits in this word
    if (tail < 32) v &= (tail <= 0) ? 0u : ((1u << tail) - 1u);
    return v;
}

__global__ void prepack_lane_kernel(const uint32_t *__restrict__ user, uint32_t *__restrict__ lane_words,
                                    int32_t *__restrict__ lane_rect, int out_c, int kh, int kw,
                                    int words, int in_c, int tiles, int kwc4)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int taps = kh * kw;
    const long long n_words = (long long)tiles * kh * kwc4 * 64 * 4;
    const int rrow = rect_row(kw);
    const int rect = (kh + 1) * rrow;
    const long long n_popc = (long long)tiles * rect * 64;
    if (t < n_words) {
        const int j = (int)(t % 4);
        const int lane = (int)((t / 4) % 64);
        const int q = (int)((t / 256) % kwc4);
        const int ky = (int)((t / (256LL * kwc4)) % kh);
        const int tile = (int)(t / (256LL * kwc4 * kh));
        const int r = q * 4 + j;
        const int co = tile * kTile + lane;
        uint32_t v = 0;
        if (co < out_c && r < kw * words)
            v = cleared_word(user, co, ky * kw + r / words, r % words, taps, words, in_c);
        lane_words[t] = v;
    } else if (t < n_words + n_popc) {
        const long long u = t - n_words;
        const int e = (int)(u % rect);
        const int lane = (int)((u / rect) % 64);
        const int tile = (int)(u / (64LL * rect));
        const int ra = e / rrow, rb = e % rrow;
        const int co = tile * kTile + lane;
        int pc = 0;
        if (co < out_c && rb <= kw)
            for (int ky = 0; ky < ra; ++ky)
                for (int kx = 0; kx < rb; ++kx)
                    for (int w = 0; w < words; ++w)
                        pc += __popc(cleared_word(user, co, ky * kw + kx, w, taps, words, in_c));
        lane_rect[u] = pc;
    }
}

__global__ void prepack_pm_kernel(const uint32_t *__restrict__ user, float *__restrict__ pm, int out_c,
                                  int taps, int words, int in_c, int pm_cols)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)taps * in_c * pm_cols;
    if (t >= total) return;
    const int co = (int)(t % pm_cols);
    const long long row = t / pm_cols;  // tap*in_c + f
    const int f = (int)(row % in_c);
    const int tap = (int)(row / in_c);
    float v = 0.0f;
    if (co < out_c) {
        const uint32_t word = user[((long long)co * taps + tap) * words + f / 32];
        v = ((word >> (f % 32)) & 1u) ? 1.0f : -1.0f;
    }
    pm[t] = v;
}

}  // namespace

hipError_t launch_prepack(const Geom &g, hipStream_t s, const uint32_t *user_bits, uint32_t *lane_words,
                          int32_t *lane_popc, float *pm_weights, int pm_cols, int type)
{
    const int taps = g.kh * g.kw;
    if (type != BCONV_BINARY_WEIGHTS) {
        const int kwc4 = (g.kw * g.words + 3) / 4;
        const long long total = (long long)g.tiles * g.kh * kwc4 * 256 +
                                (long long)g.tiles * (g.kh + 1) * rect_row(g.kw) * 64;
        hipLaunchKernelGGL(prepack_lane_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           user_bits, lane_words, lane_popc, g.out_c, g.kh, g.kw, g.words, g.in_c,
                           g.tiles, kwc4);
        return hipGetLastError();
    }
    const long long total = (long long)taps * g.in_c * pm_cols;
    hipLaunchKernelGGL(prepack_pm_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       user_bits, pm_weights, g.out_c, taps, g.words, g.in_c, pm_cols);
    return hipGetLastError();
}

}  // namespace bconv
