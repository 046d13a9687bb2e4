// binaryWeights convolution (Apple "MPSCNNBinaryConvolution", Overview,
// binaryWeights bullet): the input is not binarised; each weight bit is read
// as +1 (bit 1) or -1 (bit 0); fp32 accumulation; then the fused epilogue
// neuron(acc*scale[c]*beta + bias[c]).
//
// Mapping: a lane owns one output pixel and Q output channels (accumulators
// in VGPRs).  The +-1.0f weights of the Q channels are the same for every
// lane, so they come from scalar loads and enter v_fma_f32 as the scalar
// operand; each loaded input value (input affine applied once, 0 at padded
// taps) is reused Q times.  Sums are formed per tap and then added, which
// keeps the rounding error near (in_c + taps) ulps instead of in_c*taps.
#include "internal.h"

namespace bconv {
namespace {

typedef const float __attribute__((address_space(4))) *scalar_f32_ptr;

struct BwArgs {
    const float *x, *in_scale, *in_bias;
    const float *pm;  // [taps*in_c][pm_cols]
    int pm_cols;
    const float *scale, *bias;
    const float *a_pad;  // zero-halo A map or nullptr (beta = 1)
    float *beta_out;
    int beta_valid;      // beta divisor: in-image taps instead of kh*kw
    int rows, cols;
    float scale_value;
    Neuron neuron;
    float *out;
    float *acc_out;
    uint32_t *bits_out;  // packed sign bits instead of out (see Epilogue)
    int out_words;
    int n, in_h, in_w, in_c, out_c, out_h, out_w, kh, kw, sh, sw, ph, pw;
    int cblocks;
};

template <int Q, int VEC>
__global__ __launch_bounds__(256) void bwconv_kernel(BwArgs a)
{
    const int lane = threadIdx.x & 63;
    const long long gw = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cb = (int)(gw % a.cblocks);
    const long long mblock = gw / a.cblocks;
    const long long m_total = (long long)a.n * a.out_h * a.out_w;
    if (mblock * 64 >= m_total) return;
    const long long m = mblock * 64 + lane;
    const bool live = m < m_total;
    const int ox = (int)(m % a.out_w);
    const int oy = (int)((m / a.out_w) % a.out_h);
    const long long img = m / ((long long)a.out_w * a.out_h);
    const bool affine = a.in_scale != nullptr || a.in_bias != nullptr;
    const scalar_f32_ptr pm = (scalar_f32_ptr)a.pm;
    const scalar_f32_ptr isc = (scalar_f32_ptr)a.in_scale;
    const scalar_f32_ptr ibi = (scalar_f32_ptr)a.in_bias;

    float acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = 0.0f;

    for (int ky = 0; ky < a.kh; ++ky) {
        const int iy = oy * a.sh - a.ph + ky;
        for (int kx = 0; kx < a.kw; ++kx) {
            const int ix = ox * a.sw - a.pw + kx;
            const bool valid = live && iy >= 0 && iy < a.in_h && ix >= 0 && ix < a.in_w;
            const float *xp = a.x + (valid ? ((img * a.in_h + iy) * a.in_w + ix) * a.in_c : 0);
            const long long wrow = (long long)(ky * a.kw + kx) * a.in_c;
            float part[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) part[q] = 0.0f;
            for (int c = 0; c < a.in_c; c += VEC) {
                float v[VEC];
                if constexpr (VEC == 4) {
                    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (valid) t = *reinterpret_cast<const float4 *>(xp + c);
                    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
                } else {
                    v[0] = valid ? xp[c] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    float xv = v[j];
                    if (affine) {
                        const float s = a.in_scale ? isc[c + j] : 1.0f;
                        const float b = a.in_bias ? ibi[c + j] : 0.0f;
                        xv = valid ? __builtin_fmaf(xv, s, b) : 0.0f;
                    }
                    const long long wo = (wrow + c + j) * a.pm_cols + (long long)cb * Q;
#pragma unroll
                    for (int q = 0; q < Q; ++q) part[q] = __builtin_fmaf(xv, pm[wo + q], part[q]);
                }
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) acc[q] += part[q];
        }
    }

    if (!live) return;
    float be = 1.0f;
    if (a.a_pad) {
        // beta: window sum of the zero-halo A map / (kh*kw, or the in-image taps)
        const float *ap = a.a_pad + (img * a.rows + (long long)oy * a.sh) * a.cols + (long long)ox * a.sw;
        float sum = 0.0f;
        for (int ky = 0; ky < a.kh; ++ky)
            for (int kx = 0; kx < a.kw; ++kx) sum += ap[ky * a.cols + kx];
        be = sum / (float)(a.beta_valid ? window_valid_taps(oy, ox, a.sh, a.sw, a.ph, a.pw, a.kh, a.kw, a.in_h, a.in_w) : a.kh * a.kw);
        if (cb == 0) a.beta_out[m] = be;
    }
    if (a.bits_out) {
        // channels 32*cb + [0, 32) are word cb of the pixel
        static_assert(Q == 32, "one output word per lane");
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int co = cb * Q + q;
            if (co >= a.out_c) break;
            const float sc = a.scale ? a.scale[co] : a.scale_value;
            const float bi = a.bias ? a.bias[co] : 0.0f;
            if (sign_bit(epilogue_value(acc[q], sc, be, bi, a.neuron))) word |= 1u << q;
        }
        store_through(&a.bits_out[m * a.out_words + cb], word);
        return;
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int co = cb * Q + q;
        if (co >= a.out_c) break;
        const long long o = m * a.out_c + co;
        if (a.acc_out) {
            __hip_atomic_store(&a.acc_out[o], acc[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        const float sc = a.scale ? a.scale[co] : a.scale_value;
        const float bi = a.bias ? a.bias[co] : 0.0f;
        __hip_atomic_store(&a.out[o], epilogue_value(acc[q], sc, be, bi, a.neuron), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

constexpr int kQ = 32;

}  // namespace

int bwconv_pm_cols(int out_c) { return (out_c + kQ - 1) / kQ * kQ; }

const char *bwconv_kernel_name(const Geom &g)
{
    return (g.in_c % 4 == 0) ? "bwconv_kernel<32,4>" : "bwconv_kernel<32,1>";
}

hipError_t launch_bwconv(const Geom &g, const Launch &L, const float *x, const float *in_scale,
                         const float *in_bias, const float *pm_weights, int pm_cols,
                         const Epilogue &e, float *out, float *acc_out)
{
    BwArgs a{};
    a.x = x;
    a.in_scale = in_scale;
    a.in_bias = in_bias;
    a.pm = pm_weights;
    a.pm_cols = pm_cols;
    a.scale = e.scale;
    a.bias = e.bias;
    a.a_pad = e.a_pad;
    a.beta_valid = e.beta_valid_taps;
    a.beta_out = e.beta_out;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
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
    a.cblocks = (g.out_c + kQ - 1) / kQ;
    const long long m_total = (long long)g.n * g.out_h * g.out_w;
    const long long waves = (m_total + 63) / 64 * a.cblocks;
    const long long blocks = (waves + 3) / 4;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool vec4 = (g.in_c % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    if (vec4) return launch_kernel(L, bwconv_kernel<kQ, 4>, dim3((unsigned)blocks), dim3(256), 0, a);
    return launch_kernel(L, bwconv_kernel<kQ, 1>, dim3((unsigned)blocks), dim3(256), 0, a);
}

}  // namespace bconv
