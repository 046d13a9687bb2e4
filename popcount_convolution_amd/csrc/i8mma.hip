// XNOR / AND convolution on the int8 matrix cores: a measured comparison
// point for the popcount path, selected with BCONV_FLAG_INT8_MFMA.
//
// Apple "MPSCNNBinaryConvolution" (Overview, XNOR and AND bullets) defines
// the products on binarised values: XNOR reads both sides as +-1, AND as 0/1.
// Stored as int8, a window sum is an exact integer dot product, which
// v_mfma_i32_16x16x64_i8 computes with int32 accumulation.  Padded taps hold
// 0 in the zero-halo int8 buffer, so they contribute nothing to either form
// and no border correction is needed.
//
// Pipeline:
//  * pack_i8_kernel: input affine, sign, int8 value per channel (channels
//    padded with 0 to a multiple of 64) into a zero-halo NHWC buffer, plus the
//    zero-halo A map when beta is on; halo pixels are written as zeros by the
//    same pass;
//  * prepack_i8_kernel (create time): int8 weight fragments in the exact
//    A-operand order, [tiles][ksteps][4][64] x 16 bytes;
//  * i8mma_kernel: 8 waves = 64 output pixels x 64 output channels, K halves
//    summed in LDS, weight fragments staged in LDS, 16-byte activation loads.
#include "internal.h"

namespace bconv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPixTile = 64;
constexpr int kChanTile = 64;
constexpr int kStage = 18;    // K steps of weight fragments per LDS stage (72 KiB)
constexpr int kStepU4 = 256;  // 16-byte fragment entries per K step
constexpr int kXcds = 8;
constexpr int kThreads = 512;
constexpr int kRedBytes = 4 * 4 * 64 * 16;

// ------------------------------------------------------------------ pack

struct I8PackArgs {
    const float *x, *in_scale, *in_bias;  // scale and bias both set or both null
    int8_t *act;                          // [n][rows][cols][cpad]
    float *a_map;                         // [n][rows][cols] or nullptr
    int n, in_h, in_w, in_c, rows, cols, halo_h, halo_w, cpad, and_mode;
    int x_bytes, act_bytes, amap_bytes;
    FastDiv div_cols, div_rows;
    int pixels;  // n * rows * cols (padded)
};

// 16 lanes per padded pixel, 4 pixels per wave; lane sl of a pixel handles
// the 16-channel groups sl, sl+16, ...
template <bool VEC>
__global__ __launch_bounds__(256) void pack_i8_kernel(I8PackArgs a)
{
    const int lane = threadIdx.x & 63;
    const unsigned wave = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned pix = wave * 4u + (unsigned)(lane >> 4);
    const int sl = lane & 15;
    const bool live = pix < (unsigned)a.pixels;
    const unsigned pp = live ? pix : 0u;
    const unsigned rowi = fastdiv(pp, a.div_cols);
    const int c = (int)(pp - rowi * (unsigned)a.cols);
    const unsigned img = fastdiv(rowi, a.div_rows);
    const int r = (int)(rowi - img * (unsigned)a.rows);
    const int y = r - a.halo_h, x = c - a.halo_w;
    const bool inside = live && y >= 0 && y < a.in_h && x >= 0 && x < a.in_w;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.act, a.act_bytes);
    const uint32_t in_base = (uint32_t)(((img * (unsigned)a.in_h + (unsigned)y) * (unsigned)a.in_w + (unsigned)x) *
                                        (unsigned)a.in_c) * 4u;
    const uint32_t out_base = pp * (uint32_t)a.cpad;
    const bool affine = a.in_scale != nullptr;
    float asum = 0.0f;
    for (int g = sl; g < a.cpad / 16; g += 16) {
        uint32_t words[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c0 = g * 16 + q * 4;
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (inside && c0 < a.in_c) {
                if constexpr (VEC) {
                    const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, in_base + c0 * 4u, 0, 0));
                    v[0] = t[0];
                    v[1] = t[1];
                    v[2] = t[2];
                    v[3] = t[3];
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (c0 + k < a.in_c)
                            v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, in_base + (c0 + k) * 4u, 0, 0));
                }
            }
            uint32_t wv = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int ch = c0 + k;
                if (inside && ch < a.in_c) {
                    const float xv = affine ? __builtin_fmaf(v[k], a.in_scale[ch], a.in_bias[ch]) : v[k];
                    asum += __builtin_fabsf(xv);
                    // sign read as +1 unless x' < 0 (so -0 and NaN read +1)
                    const uint32_t b = (xv < 0.0f) ? (a.and_mode ? 0x00u : 0xffu) : 0x01u;
                    wv |= b << (8 * k);
                }
            }
            words[q] = wv;
        }
        if (live)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, u32x4{words[0], words[1], words[2], words[3]}),
                                                   orr, out_base + (uint32_t)g * 16u, 0, 0);
    }
    if (a.a_map) {
        // sum over the pixel's 16 lanes in a fixed order
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) asum += __shfl_xor(asum, m);
        if (live && sl == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, inside ? asum / (float)a.in_c : 0.0f),
                                                  make_rsrc(a.a_map, a.amap_bytes), pp * 4u, 0, 0);
    }
}

// ------------------------------------------------------------------ prepack

// int8 weight fragments [ntiles][ksteps][4][64] x 16: entry (tile, s, blk,
// lane) holds, for output channel 64*tile + 16*blk + lane%16, the weights of
// tap s / chunks at input channels 64*(s % chunks) + 16*(lane/16) + 0..15:
// +1/-1 (XNOR) or 1/0 (AND) from bit 1/0; 0 for channels past in_c or out_c.
__global__ void prepack_i8_kernel(const uint32_t *__restrict__ user, u32x4 *__restrict__ frag, int out_c, int taps,
                                  int words, int in_c, int chunks, int ksteps, int ntiles, int and_mode)
{
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)ntiles * ksteps * kStepU4;
    if (t >= total) return;
    const int lane = (int)(t % 64);
    const int blk = (int)((t / 64) % 4);
    const int s = (int)((t / kStepU4) % ksteps);
    const int tile = (int)(t / ((long long)kStepU4 * ksteps));
    const int co = tile * kChanTile + 16 * blk + (lane & 15);
    const int tap = s / chunks, q = s % chunks;
    u32x4 r = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16; ++j) {
        const int f = q * 64 + 16 * (lane >> 4) + j;
        uint32_t v = 0;
        if (co < out_c && f < in_c) {
            const uint32_t word = user[((long long)co * taps + tap) * words + f / 32];
            const bool bit = (word >> (f % 32)) & 1u;
            v = bit ? 0x01u : (and_mode ? 0x00u : 0xffu);
        }
        r[j / 4] |= v << (8 * (j % 4));
    }
    frag[t] = r;
}

// ------------------------------------------------------------------ conv

struct I8Args {
    const int8_t *act;  // [n][rows][cols][cpad]
    const u32x4 *frag;
    const float *scale, *bias;
    const float *a_pad;
    float *beta_out;
    int beta_valid;  // beta divisor: in-image taps instead of kh*kw
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;  // packed sign bits instead of out (see Epilogue)
    int out_words;
    int n, out_c, out_h, out_w, kh, kw, sh, sw, rows, cols, cpad;
    int in_h, in_w, ph, pw;
    int chunks, ksteps, ntiles, mtiles, m_total;
    int act_bytes, out_bytes, vec_out;
    int weights_major;  // consecutive tiles share a weight tile (weights outweigh activations)
};

__global__ __launch_bounds__(kThreads) void i8mma_kernel(I8Args a)
{
    extern __shared__ u32x4 stage[];  // [min(ksteps, kStage)][4][64], at least kRedBytes
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int group = wave & 3, khalf = wave >> 2;
    // XCD-aware numbering: block b runs on XCD b % 8; XCD x takes the
    // contiguous tile range [x*per, (x+1)*per).  Within it the larger operand
    // changes slowest, so the workgroups that share its tile run together
    // and read it through one L2.
    const int blocks = a.mtiles * a.ntiles;
    const int per = (blocks + kXcds - 1) / kXcds;
    const int idx = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (idx >= blocks) return;  // uniform over the workgroup
    int mtile, ntile;
    if (a.weights_major) {
        ntile = idx / a.mtiles;
        mtile = idx - ntile * a.mtiles;
    } else {
        mtile = idx / a.ntiles;
        ntile = idx - mtile * a.ntiles;
    }

    // this lane's output pixel (pixels past the batch reuse the last one and
    // are not stored)
    const int p_raw = mtile * kPixTile + group * 16 + (lane & 15);
    const bool live = p_raw < a.m_total;
    const int pix = live ? p_raw : a.m_total - 1;
    const int hw = a.out_h * a.out_w;
    const int img = pix / hw, rem = pix - (pix / hw) * hw;
    const int oy = rem / a.out_w, ox = rem - (rem / a.out_w) * a.out_w;
    // byte offset of the window's first tap in the zero-halo buffer, plus this
    // lane's 16-channel group; every tap stays inside the buffer
    const uint32_t lane_base =
        (uint32_t)(((img * a.rows + oy * a.sh) * a.cols + ox * a.sw) * a.cpad + 16 * (lane >> 4));
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.act, a.act_bytes);

    // epilogue operands, loaded now
    const int keep = khalf ? 2 : 0;
    float sc[2][4], bi[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int c = ntile * kChanTile + 16 * (keep + u) + 4 * (lane >> 4) + r;
            c = c < a.out_c ? c : a.out_c - 1;
            sc[u][r] = a.scale ? a.scale[c] : a.scale_value;
            bi[u][r] = a.bias ? a.bias[c] : 0.0f;
        }
    float be = 1.0f;
    if (a.a_pad) {
        const float *ap = a.a_pad + ((long long)img * a.rows + oy * a.sh) * a.cols + ox * a.sw;
        float sum = 0.0f;
        for (int ky = 0; ky < a.kh; ++ky)
            for (int kx = 0; kx < a.kw; ++kx) sum += ap[ky * a.cols + kx];
        be = sum / (float)(a.beta_valid ? window_valid_taps(oy, ox, a.sh, a.sw, a.ph, a.pw, a.kh, a.kw, a.in_h, a.in_w) : a.kh * a.kw);
    }

    i32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = i32x4{0, 0, 0, 0};

    const u32x4 *gfrag = a.frag + (long long)ntile * a.ksteps * kStepU4;
    for (int s0 = 0; s0 < a.ksteps; s0 += kStage) {
        const int cnt = a.ksteps - s0 < kStage ? a.ksteps - s0 : kStage;
        const int half = (cnt + 1) >> 1;
        const int sb = s0 + (khalf ? half : 0), se = s0 + (khalf ? cnt : half);
        __syncthreads();  // previous stage fully read
        for (int i = threadIdx.x; i < cnt * kStepU4; i += kThreads) stage[i] = gfrag[(long long)s0 * kStepU4 + i];
        __syncthreads();
        // (tap, chunk) of step sb, advanced without divisions
        int tap = sb / a.chunks, q = sb - (sb / a.chunks) * a.chunks;
        int ky = tap / a.kw, kx = tap - (tap / a.kw) * a.kw;
        for (int s = sb; s < se; ++s) {
            const uint32_t off = lane_base + (uint32_t)((ky * a.cols + kx) * a.cpad + q * 64);
            const i32x4 x = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0));
            const u32x4 *bs = stage + (s - s0) * kStepU4 + lane;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, bs[t * 64]), x, acc[t], 0, 0, 0);
            if (++q == a.chunks) {
                q = 0;
                if (++kx == a.kw) {
                    kx = 0;
                    ++ky;
                }
            }
        }
    }

    // Sum the two K halves through LDS (static register indices only).
    i32x4 *red = reinterpret_cast<i32x4 *>(stage) + group * 4 * 64 + lane;  // [4 groups][4 blocks][64]
    __syncthreads();  // stage fully read
    if (khalf == 0) {
        red[2 * 64] = acc[2];
        red[3 * 64] = acc[3];
    } else {
        red[0] = acc[0];
        red[64] = acc[1];
    }
    __syncthreads();
    i32x4 res[2];
    if (khalf == 0) {
        res[0] = acc[0] + red[0];
        res[1] = acc[1] + red[64];
    } else {
        res[0] = acc[2] + red[2 * 64];
        res[1] = acc[3] + red[3 * 64];
    }
    // Epilogue: element r of block keep+u is pixel p_raw, channel
    // ntile*64 + 16*(keep+u) + 4*(lane/16) + r.  The int8 dot product is the
    // window sum itself (+-1 sum for XNOR, 0/1 count for AND).
    if (live && ntile == 0 && khalf == 0 && lane < 16 && a.a_pad) a.beta_out[pix] = be;
    if (a.bits_out) {
        // The wave's two blocks are channels 64*ntile + 16*keep + [0, 32): word
        // 2*ntile + keep/2 of the pixel, element r of block keep+u at bit
        // 16u + 4*(lane/16) + r; the four 16-lane groups OR their parts.
        uint32_t part = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = ntile * kChanTile + 16 * (keep + u) + 4 * (lane >> 4) + r;
                const float y = epilogue_value((float)res[u][r], sc[u][r], be, bi[u][r], a.neuron);
                if (co < a.out_c && sign_bit(y)) part |= 1u << (16 * u + 4 * (lane >> 4) + r);
            }
        part |= __shfl_xor(part, 16);
        part |= __shfl_xor(part, 32);
        const int wi = 2 * ntile + keep / 2;
        if (live && lane < 16 && wi < a.out_words) store_through(&a.bits_out[(long long)pix * a.out_words + wi], part);
        return;
    }
    if (!live) return;
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.acc_out ? (void *)a.acc_out : (void *)a.out, a.out_bytes);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int co = ntile * kChanTile + 16 * (keep + u) + 4 * (lane >> 4);
        u32x4 w;
        if (a.acc_out) {
            w = __builtin_bit_cast(u32x4, res[u]);
        } else {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = epilogue_value((float)res[u][r], sc[u][r], be, bi[u][r], a.neuron);
            w = __builtin_bit_cast(u32x4, v);
        }
        const uint32_t off = (uint32_t)(pix * a.out_c + co) * 4u;
        if (a.vec_out && co + 3 < a.out_c) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, w), orr, off, 0, kStoreSc1);
        } else {
            if (co < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.x, orr, off, 0, kStoreSc1);
            if (co + 1 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.y, orr, off + 4u, 0, kStoreSc1);
            if (co + 2 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.z, orr, off + 8u, 0, kStoreSc1);
            if (co + 3 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.w, orr, off + 12u, 0, kStoreSc1);
        }
    }
}

}  // namespace

int i8_cpad(int in_c) { return (in_c + 63) / 64 * 64; }

size_t i8_act_bytes(const Geom &g) { return (size_t)g.n * g.bits_rows * g.bits_cols * i8_cpad(g.in_c); }

size_t i8_frag_bytes(const Geom &g)
{
    const long long chunks = i8_cpad(g.in_c) / 64;
    const long long ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    return (size_t)(ntiles * g.kh * g.kw * chunks * kStepU4 * 16);
}

hipError_t launch_prepack_i8(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *frag, int and_mode)
{
    const int chunks = i8_cpad(g.in_c) / 64;
    const int ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    const int ksteps = g.kh * g.kw * chunks;
    const long long total = (long long)ntiles * ksteps * kStepU4;
    hipLaunchKernelGGL(prepack_i8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, user_bits,
                       static_cast<u32x4 *>(frag), g.out_c, g.kh * g.kw, g.words, g.in_c, chunks, ksteps, ntiles,
                       and_mode);
    return hipGetLastError();
}

hipError_t launch_pack_i8(const Geom &g, const Launch &L, const float *x, const float *in_scale, const float *in_bias,
                          int and_mode, int8_t *act, float *a_map)
{
    I8PackArgs a{};
    a.x = x;
    a.in_scale = in_scale;
    a.in_bias = in_bias;
    a.act = act;
    a.a_map = a_map;
    a.n = g.n;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.in_c = g.in_c;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    a.halo_h = g.bits_halo_h;
    a.halo_w = g.bits_halo_w;
    a.cpad = i8_cpad(g.in_c);
    a.and_mode = and_mode;
    const long long xb = (long long)g.n * g.in_h * g.in_w * g.in_c * 4;
    const long long ab = (long long)i8_act_bytes(g);
    const long long mb = (long long)g.n * g.bits_rows * g.bits_cols * 4;
    const long long pixels = (long long)g.n * g.bits_rows * g.bits_cols;
    if (xb >= 0x7fffffffLL || ab >= 0x7fffffffLL || mb >= 0x7fffffffLL || pixels * 16 >= 0x7fffffffLL)
        return hipErrorInvalidValue;
    a.x_bytes = (int)xb;
    a.act_bytes = (int)ab;
    a.amap_bytes = (int)mb;
    a.pixels = (int)pixels;
    a.div_cols = make_fastdiv((uint32_t)g.bits_cols);
    a.div_rows = make_fastdiv((uint32_t)g.bits_rows);
    const long long waves = (pixels + 3) / 4;
    const long long blocks = (waves + 3) / 4;
    if (blocks == 0) return hipSuccess;
    const bool vec = g.in_c % 4 == 0 && (uintptr_t)x % 16 == 0;
    if (vec) return launch_kernel(L, pack_i8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, a);
    return launch_kernel(L, pack_i8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, a);
}

const char *i8mma_kernel_name() { return "i8mma_kernel"; }

hipError_t launch_i8mma(const Geom &g, const Launch &L, const int8_t *act, const void *frag, const Epilogue &e,
                        float *out, int32_t *acc_out)
{
    I8Args a{};
    a.act = act;
    a.frag = static_cast<const u32x4 *>(frag);
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
    a.out_c = g.out_c;
    a.out_h = g.out_h;
    a.out_w = g.out_w;
    a.kh = g.kh;
    a.kw = g.kw;
    a.sh = g.sh;
    a.sw = g.sw;
    a.in_h = g.in_h;
    a.in_w = g.in_w;
    a.ph = g.ph;
    a.pw = g.pw;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    a.cpad = i8_cpad(g.in_c);
    a.chunks = a.cpad / 64;
    a.ksteps = g.kh * g.kw * a.chunks;
    a.ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    const long long m_total = (long long)g.n * g.out_h * g.out_w;
    const long long mtiles = (m_total + kPixTile - 1) / kPixTile;
    const long long act_bytes = (long long)i8_act_bytes(g);
    const long long out_bytes = m_total * g.out_c * 4;
    if (m_total == 0) return hipSuccess;
    if (act_bytes >= 0x7fffffffLL || out_bytes >= 0x7fffffffLL || mtiles * a.ntiles >= 0x7fffffffLL - kXcds ||
        (long long)a.ksteps * kStepU4 * 16 >= 0x7fffffffLL)
        return hipErrorInvalidValue;
    a.m_total = (int)m_total;
    a.mtiles = (int)mtiles;
    a.act_bytes = (int)act_bytes;
    a.out_bytes = (int)out_bytes;
    const void *dst = acc_out ? (const void *)acc_out : (const void *)out;
    a.vec_out = g.out_c % 4 == 0 && (uintptr_t)dst % 16 == 0;
    a.weights_major = (long long)a.ntiles * a.ksteps * kStepU4 * 16 > act_bytes;
    const int blocks = a.mtiles * a.ntiles;
    const int grid = (blocks + kXcds - 1) / kXcds * kXcds;
    const uint32_t stage_bytes = (uint32_t)(a.ksteps < kStage ? a.ksteps : kStage) * kStepU4 * 16;
    const uint32_t lds = stage_bytes > kRedBytes ? stage_bytes : kRedBytes;
    return launch_kernel(L, i8mma_kernel, dim3(grid), dim3(kThreads), lds, a);
}

}  // namespace bconv
