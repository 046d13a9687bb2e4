// XNOR / AND binary convolution: the window sum of Apple
// "MPSCNNBinaryConvolution" (Overview, output equation) with the XNOR and AND
// products of its type bullets, one 32-bit word pair at a time:
//   XNOR: 32 - 2*popcount(x ^ w) per word, so a window sums to
//         Cin*taps_in_image - 2*popcount-sum of the disagreements;
//   AND:  popcount(x & w) per word.
// followed by the fused epilogue  neuron(v*scale[c]*beta + bias[c]).
//
// Mapping on gfx950: a wave owns 64 output channels (one per lane).  The
// binarised input words under the window are the same for every lane, so they
// are fetched with scalar loads into SGPRs and fed to v_xor_b32 / v_and_b32 as
// the scalar operand; v_bcnt_u32_b32 then counts and accumulates in one
// instruction, two VALU instructions per word pair.  A lane's weight words come
// from the lane-major table (256 contiguous bytes per wave per 4 words): the
// specialised kernel reads them once per kernel row for a whole strip of output
// pixels, the generic kernel below once per tap for its single pixel.  No LDS.
//
// The specialised kernel (xconv_fast.h) is compiled per shape in
// xconv_k*.hip; this file holds the kernel for any geometry and the dispatch.
#include "xconv_fast.h"

namespace bconv {
namespace {

__device__ __forceinline__ void store_result(const XArgs &a, long long pix, int co, int v,
                                             float sc, float bi, float be)
{
    if (co >= a.out_c) return;
    const long long o = pix * a.out_c + co;
    // Agent-scope stores write through to memory while the kernel runs, so the
    // output does not sit dirty in L2 until the end-of-kernel write-back.
    if (a.acc_out) {
        __hip_atomic_store(&a.acc_out[o], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    __hip_atomic_store(&a.out[o], epilogue_value((float)v, sc, be, bi, a.neuron), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Any geometry: one wave = one output pixel and a 64-channel tile; taps
// outside the image are skipped, so no correction is needed.
__global__ __launch_bounds__(256) void xconv_generic(XArgs a, int and_mode)
{
    // Work indices fit 31 bits (the host checks pixels * tiles < 2^31).
    const int lane = threadIdx.x & 63;
    const unsigned gw = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned tile = gw % (unsigned)a.tiles;
    const unsigned upix = gw / (unsigned)a.tiles;
    if (upix >= (unsigned)a.n * (unsigned)a.out_h * (unsigned)a.out_w) return;
    const long long pix = upix;
    const int ox = (int)(upix % (unsigned)a.out_w);
    const int oy = (int)((upix / (unsigned)a.out_w) % (unsigned)a.out_h);
    const int img = (int)(upix / ((unsigned)a.out_w * (unsigned)a.out_h));
    const scalar_u32_ptr bits = (scalar_u32_ptr)a.bits;
    const uint32_t *wl = a.wlane + (long long)tile * a.kh * a.kwc4 * 256 + lane * 4;
    uint32_t acc = 0;
    int valid = 0;
    for (int ky = 0; ky < a.kh; ++ky) {
        const int iy = oy * a.sh - a.ph + ky;
        if (iy < 0 || iy >= a.in_h) continue;
        for (int kx = 0; kx < a.kw; ++kx) {
            const int ix = ox * a.sw - a.pw + kx;
            if (ix < 0 || ix >= a.in_w) continue;
            ++valid;
            const long long base =
                (((long long)img * a.rows + iy + a.ph) * a.cols + ix + a.pw) * a.words;
            const int r0 = kx * a.words;
            for (int j = 0; j < a.words; ++j) {
                const int r = r0 + j;
                const uint32_t xv = bits[base + j];
                const uint32_t wv = wl[(ky * a.kwc4 + (r >> 2)) * 256 + (r & 3)];
                acc += __builtin_popcount(and_mode ? (xv & wv) : (xv ^ wv));
            }
        }
    }
    const int co = tile * kTile + lane;
    const bool co_ok = co < a.out_c;
    const int v = and_mode ? (int)acc : a.in_c * valid - 2 * (int)acc;
    const float sc = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
    const float bi = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;
    float be = 1.0f;
    if (a.a_pad) {
        const float *ap = a.a_pad + ((long long)img * a.rows + oy * a.sh) * a.cols + ox * a.sw;
        float sum = 0.0f;
        for (int ky = 0; ky < a.kh; ++ky)
            for (int kx = 0; kx < a.kw; ++kx) sum += ap[ky * a.cols + kx];
        be = sum / (float)(a.beta_valid ? window_valid_taps(oy, ox, a.sh, a.sw, a.ph, a.pw, a.kh, a.kw, a.in_h, a.in_w) : a.kh * a.kw);
        if (tile == 0 && lane == 0) a.beta_out[pix] = be;
    }
    if (a.bits_out)
        store_tile_bits(a.bits_out, pix, a.out_words, (int)tile, co_ok && sign_bit(epilogue_value((float)v, sc, be, bi, a.neuron)));
    else
        store_result(a, pix, co, v, sc, bi, be);
}

// Every wave is one (strip, tile) task and all SIMDs run them at once, so
// the kernel lasts about ceil(tasks / SIMDs) strips of P pixels plus a fixed
// cost per strip (row loads, epilogue) of about 1.5 pixels' worth.  The strip
// width minimises that among the compiled widths.
double strip_cost(const Geom &g, int p)
{
    const long long tasks = (long long)g.n * g.out_h * ((g.out_w + p - 1) / p) * g.tiles;
    const long long simds = g.simds > 0 ? g.simds : 1024;
    return (double)((tasks + simds - 1) / simds) * (p + 1.5);
}

const FastEntry *find_fast(const Geom &g)
{
    const FastTable tables[] = {xconv_fast_k1(), xconv_fast_k3(), xconv_fast_k24(), xconv_fast_k5()};
    const FastEntry *best = nullptr;
    double best_cost = 0.0;
    for (const FastTable &t : tables) {
        for (int i = 0; i < t.count; ++i) {
            const FastEntry &e = t.entries[i];
            if (e.kh != g.kh || e.kw != g.kw || e.cw != g.words || e.sw != g.sw) continue;
            if (g.strip_p > 0 && e.p == g.strip_p) return &e;
            const double c = strip_cost(g, e.p);
            if (!best || c < best_cost || (c == best_cost && e.p > best->p)) {
                best = &e;
                best_cost = c;
            }
        }
    }
    return best;
}

XArgs make_args(const Geom &g, const uint32_t *bits, const LaneWeights &w, const Epilogue &e,
                float *out, int32_t *acc_out)
{
    XArgs a{};
    a.bits = bits;
    a.wlane = w.words;
    a.wrect = w.rect;
    a.scale = e.scale;
    a.bias = e.bias;
    a.a_pad = e.a_pad;
    a.beta_valid = e.beta_valid_taps;
    a.beta_out = e.beta_out;
    a.scale_value = e.scale_value;
    a.neuron = e.neuron;
    a.out = out;
    a.acc_out = acc_out;
    a.bits_out = e.bits_out;
    a.out_words = e.out_words;
    a.n = g.n;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.in_c = g.in_c;
    a.out_c = g.out_c;
    a.out_h = g.out_h;
    a.out_w = g.out_w;
    a.kh = g.kh;
    a.kw = g.kw;
    a.sh = g.sh;
    a.sw = g.sw;
    a.ph = g.ph;
    a.pw = g.pw;
    a.words = g.words;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    a.kwc4 = w.kwc4;
    a.tiles = g.tiles;
    a.out_bytes = (int)((long long)g.n * g.out_h * g.out_w * g.out_c * 4);
    a.wlane_bytes = (int)((long long)g.tiles * g.kh * w.kwc4 * 1024);
    a.wrect_bytes = (int)((long long)g.tiles * 64 * (g.kh + 1) * rect_row(g.kw) * 4);
    a.apad_bytes = (int)((long long)g.n * g.bits_rows * g.bits_cols * 4);
    a.beta_bytes = (int)((long long)g.n * g.out_h * g.out_w * 4);
    return a;
}

}  // namespace

bool xconv_fast_available(const Geom &g) { return find_fast(g) != nullptr; }

const char *xconv_kernel_name(const Geom &g)
{
    const FastEntry *e = find_fast(g);
    return e ? e->name : "xconv_generic";
}

hipError_t launch_xconv(const Geom &g, const Launch &L, int and_mode, const uint32_t *bits,
                        const LaneWeights &w, const Epilogue &e, float *out, int32_t *acc_out,
                        bool allow_fast)
{
    XArgs a = make_args(g, bits, w, e, out, acc_out);
    const FastEntry *f = allow_fast ? find_fast(g) : nullptr;
    if (f) return f->fn(a, L, and_mode);
    const long long waves = (long long)g.n * g.out_h * g.out_w * g.tiles;
    const long long blocks = (waves + 3) / 4;
    if (blocks == 0) return hipSuccess;
    if (waves * 4 >= 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_kernel(L, xconv_generic, dim3((unsigned)blocks), dim3(256), 0, a, and_mode);
}

}  // namespace bconv
