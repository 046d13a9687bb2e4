// Specialised XNOR / AND binary convolution kernel, shared by the
// translation units that instantiate it (one per kernel-size family, so the
// instantiations compile in parallel).
//
// XNOR / AND binary convolution: the window sum of Apple
// "MPSCNNBinaryConvolution" (Overview, output equation) with the XNOR and AND
// products of its type bullets, one 32-bit word pair at a time:
//   XNOR: 32 - 2*popcount(x ^ w) per word, so a window sums to
//         Cin*taps_in_image - 2*popcount-sum of the disagreements;
//   AND:  popcount(x & w) per word.
// followed by the fused epilogue  neuron(v*scale[c]*beta + bias[c]).
//
// Mapping on gfx950: a wave owns 64 output channels (one per lane) of a
// strip of P neighbouring output pixels.  The kernel rows inside the image
// are walked in order (rows in the padding contribute nothing and are
// skipped); for each, every lane loads its channel's weight words of that row into
// VGPRs (16-byte loads from an L1/L2-resident table), and the binarised input
// words of the strip, the same for every lane, are fetched with scalar loads
// into SGPRs and fed to v_xor_b32 / v_and_b32 as the scalar operand;
// v_bcnt_u32_b32 then counts and accumulates in one instruction.  Two VALU
// instructions per word pair, issued in runs of P of each (see the row loop),
// no LDS.  Strips are numbered down image columns and dealt to the XCDs in
// contiguous ranges, so the waves running together share input rows in the
// caches.
#pragma once

#include "internal.h"

#include <type_traits>

namespace bconv {

typedef const uint32_t __attribute__((address_space(4))) *scalar_u32_ptr;
typedef const float __attribute__((address_space(4))) *scalar_f32_ptr;

struct XArgs {
    const uint32_t *bits;   // padded binarised input
    const uint32_t *wlane;  // [tiles][kh][kwc4][64][4]
    const int32_t *wrect;   // [tiles][64][(kh+1)*rect_row(kw)]
    const float *scale, *bias;
    const float *a_pad;  // zero-halo A map or nullptr (beta = 1)
    float *beta_out;
    int beta_valid;      // beta divisor: in-image taps instead of kh*kw
    float scale_value;
    Neuron neuron;
    float *out;
    int32_t *acc_out;
    uint32_t *bits_out;  // packed sign bits instead of out (see Epilogue)
    int out_words;
    int n, in_h, in_w, in_c, out_c, out_h, out_w;
    int kh, kw, sh, sw, ph, pw, words;
    int rows, cols;  // padded extent (halo = pad)
    int kwc4, tiles;
    int strips_per_row;
    long long strips;
    FastDiv div_tiles, div_oh, div_img;  // by tiles, out_h, strips_per_row * out_h
    // buffer sizes in bytes (each < 2^31, checked by the host)
    int out_bytes, wlane_bytes, wrect_bytes, apad_bytes, beta_bytes;
};

typedef hipError_t (*fast_launcher)(XArgs, const Launch &, int);

struct FastEntry {
    int kh, kw, cw, sw, p;
    fast_launcher fn;
    const char *name;
};

struct FastTable {
    const FastEntry *entries;
    int count;
};

// The compiled (KH, KW, CW, SW, P) instances, one table per kernel-size
// family: 1x1; 3x3; 2x2 and 4x4; 5x5.
FastTable xconv_fast_k1();
FastTable xconv_fast_k3();
FastTable xconv_fast_k24();
FastTable xconv_fast_k5();

namespace {

// v of lane i + N of the same 16-lane row (DPP row_shl:N; lanes past the row read 0).
template <int N>
__device__ __forceinline__ float row_shl(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x100 + N, 0xf,
                                                                 0xf, false));
}

// sum + v[i + K] + ... + v[i + KW - 1] within the 16-lane row, left to right.
template <int KW, int K = 1>
__device__ __forceinline__ float add_row_shifted(float sum, float v)
{
    if constexpr (K < KW)
        return add_row_shifted<KW, K + 1>(sum + row_shl<K>(v), v);
    else
        return sum;
}
// Specialised kernel: kernel KHxKW, CW words per pixel, horizontal stride SW,
// P output pixels per strip.  One wave = one (strip, 64-channel tile).
template <int KH, int KW, int CW, int SW, int P, bool AND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void xconv_fast(XArgs a)
{
    constexpr int RW = KW * CW;            // weight words per kernel row
    constexpr int RW4 = (RW + 3) / 4;
    constexpr int NCOL = (P - 1) * SW + KW;
    // words per scalar-load chunk: up to 4, fewer when a chunk of the strip
    // would take more than 64 SGPRs
    constexpr int CWC = (CW < 4 ? CW : 4) * NCOL <= 64 ? (CW < 4 ? CW : 4) : (CW % 2 == 0 && 2 * NCOL <= 64 ? 2 : 1);
    constexpr int NCH = CW / CWC;
    static_assert(CW % CWC == 0, "word chunking");

    // Work indices fit 31 bits (the host checks strips * tiles < 2^31).
    // Workgroups are dealt to the eight XCDs round-robin (block b to XCD
    // b % 8); renumbering gives XCD x a contiguous run of strips, so its L2
    // fetches only the input rows of its own part of the batch.  The grid is
    // a multiple of 8 blocks; blocks past the work exit below.  Strips are
    // numbered down the columns of an image: consecutive strips (a
    // workgroup's, and those dealt to neighbouring CUs at the same time) are
    // vertical neighbours that share KH - 1 of their input rows in the caches.
    const int lane = threadIdx.x & 63;
    const unsigned per_xcd = gridDim.x >> 3;
    const unsigned blk = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
    const unsigned gw = blk * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // (scalar multiply-high divisions by host-computed reciprocals)
    const unsigned strip = fastdiv(gw, a.div_tiles);
    const unsigned tile = gw - strip * (unsigned)a.tiles;
    if (strip >= (unsigned)a.strips) return;

    const unsigned imgu = fastdiv(strip, a.div_img);
    const unsigned in_img = strip - imgu * (unsigned)(a.strips_per_row * a.out_h);
    const unsigned col = fastdiv(in_img, a.div_oh);
    const int ow0 = (int)col * P;
    const int img = (int)imgu;
    const int oy = (int)(in_img - col * (unsigned)a.out_h);

    // beta of pixel `lane` (lanes < P): window sum of the zero-halo A map.
    // The A values are requested here, before the first kernel row's loads,
    // and summed only after the main loop: waiting for them here would put
    // one more memory round trip before the first popcount of every wave.
    constexpr int NA = (SW == 1 && NCOL <= 16) ? KH : (KH <= 4 && NCOL <= 16) ? 1 : KH * KW;
    float av[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) av[i] = 0.0f;
    if (a.a_pad) {
        const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.a_pad, a.apad_bytes);
        const uint32_t abase = (uint32_t)(((img * a.rows + oy * a.sh) * a.cols + ow0 * SW) * 4);
        if constexpr (SW == 1 && NCOL <= 16) {
            // Lane c < NCOL loads column c of the strip's KH x NCOL patch.
            // Past the last column of a ragged strip the patch reads zero
            // (buffer range) or a neighbouring pixel's value, which feed only
            // pixels not stored.
            const uint32_t coff = lane < NCOL ? (uint32_t)(lane * 4) : 0x80000000u;
#pragma unroll
            for (int r = 0; r < KH; ++r)
                av[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ar, coff, abase + r * a.cols * 4, 0));
        } else if constexpr (KH <= 4 && NCOL <= 16) {
            // One load brings the strip's KH x NCOL patch (row r in lanes
            // 16r..16r+15).  The patch stays inside the zero-halo map except
            // past the last column of a ragged strip: those read zero (buffer
            // range) or a neighbouring pixel's value, and feed only pixels
            // that are not stored.
            const int pr = lane >> 4, pc = lane & 15;
            const bool in_patch = pr < KH && pc < NCOL;
            av[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  ar, in_patch ? (uint32_t)((pr * a.cols + pc) * 4) : 0x80000000u, abase, 0));
        } else {
            if (lane < P && ow0 + lane < a.out_w) {
#pragma unroll
                for (int ky = 0; ky < KH; ++ky)
#pragma unroll
                    for (int kx = 0; kx < KW; ++kx)
                        av[ky * KW + kx] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                          ar, (uint32_t)(lane * SW * 4), abase + (ky * a.cols + kx) * 4, 0));
            }
        }
    }
    // beta from the loaded values: the window sum / (kh*kw), or / the
    // in-image taps of the lane's pixel.  Called after the main loop.
    auto finish_beta = [&]() -> float {
        if (!a.a_pad) return 1.0f;
        // (the empty asm keeps the compiler from forming the sum, and
        // waiting for the loads, before the main loop)
#pragma unroll
        for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(av[i]));
        float sum;
        if constexpr (SW == 1 && NCOL <= 16) {
            // lane c sums column c; pixel `lane` then adds columns lane ..
            // lane + KW - 1 with DPP row_shl (lane i reads lane i + kx of its
            // 16-lane row)
            float colsum = 0.0f;
#pragma unroll
            for (int r = 0; r < KH; ++r) colsum += av[r];
            sum = add_row_shifted<KW>(colsum, colsum);
        } else if constexpr (KH <= 4 && NCOL <= 16) {
            float colsum = av[0];
#pragma unroll
            for (int r = 1; r < KH; ++r) colsum += __shfl(av[0], (lane + 16 * r) & 63);
            sum = 0.0f;
#pragma unroll
            for (int kx = 0; kx < KW; ++kx) sum += __shfl(colsum, (lane * SW + kx) & 63);
        } else {
            sum = 0.0f;
#pragma unroll
            for (int i = 0; i < NA; ++i) sum += av[i];
        }
        if (a.beta_valid)
            return sum / (float)window_valid_taps(oy, ow0 + lane, a.sh, SW, a.ph, a.pw, KH, KW, a.in_h, a.in_w);
        return sum * (1.0f / (float)(KH * KW));
    };

    // Epilogue operands are loaded here, so their latency overlaps the first
    // kernel row's loads instead of sitting at the end of the wave.
    const int co = tile * kTile + lane;
    const bool co_ok = co < a.out_c;
    const float sc = a.scale ? (co_ok ? a.scale[co] : 0.0f) : a.scale_value;
    const float bi = a.bias ? (co_ok ? a.bias[co] : 0.0f) : 0.0f;
    // In-image tap rows [r0, r1) of this strip; every window holds at least
    // one in-image tap because pad < kernel.
    const int iy0 = oy * a.sh - a.ph;
    const int r0 = iy0 < 0 ? -iy0 : 0;
    const int r1 = a.in_h - iy0 < KH ? a.in_h - iy0 : KH;
    // Kernel rows outside the image are skipped.  XNOR border correction for
    // the padded columns of the rows that remain: a zero input word at a
    // padded tap counts every set weight bit as a disagreement; those bits
    // are (rows r0..r1, all columns) - (in-image rectangle), from the lane's
    // prefix sums rect[a][b] (taps ky < a, kx < b), rows r0 and r1 of the
    // table.  (read only on border strips, where they are loaded below)
    int rt0[KW + 1], rt1[KW + 1];
    const int ixa = ow0 * SW - a.pw;                 // first pixel's first tap column
    const int ixz = (ow0 + P - 1) * SW - a.pw + KW;  // one past the last pixel's last tap
    const bool border = r0 > 0 || r1 < KH || ixa < 0 || ixz > a.in_w;
    if (!AND && border) {
        // lane-major table: this lane's rows r0 and r1 are whole 16-byte loads
        constexpr int RR = (KW + 1 + 3) / 4 * 4;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.wrect, a.wrect_bytes);
        const uint32_t lbase = (uint32_t)((tile * 64 + lane) * (KH + 1) * RR) * 4u;
        int t0[RR], t1[RR];
#pragma unroll
        for (int q = 0; q < RR / 4; ++q) {
            const uint4 v0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, lbase, (r0 * RR + 4 * q) * 4, 0));
            const uint4 v1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, lbase, (r1 * RR + 4 * q) * 4, 0));
            t0[4 * q] = (int)v0.x; t0[4 * q + 1] = (int)v0.y; t0[4 * q + 2] = (int)v0.z; t0[4 * q + 3] = (int)v0.w;
            t1[4 * q] = (int)v1.x; t1[4 * q + 1] = (int)v1.y; t1[4 * q + 2] = (int)v1.z; t1[4 * q + 3] = (int)v1.w;
        }
#pragma unroll
        for (int c = 0; c <= KW; ++c) {
            rt0[c] = t0[c];
            rt1[c] = t1[c];
        }
    }

    uint32_t acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p] = 0;

    const scalar_u32_ptr bits = (scalar_u32_ptr)a.bits;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wlane, a.wlane_bytes);
    const uint32_t wbase = tile * (uint32_t)(KH * RW4 * 1024);
    // Kernel rows stay a rolled loop over the strip's in-image rows: the strip
    // words are invariant loads, and an unrolled row loop lets the compiler
    // hoist every row's scalar loads at once, which overflows the SGPR file.
    // The row's weights (RW words) are re-read from the L1/L2-resident table
    // each row.
#pragma unroll 1
    for (int ky = r0; ky < r1; ++ky) {
        uint32_t w[RW4 * 4];
#pragma unroll
        for (int q = 0; q < RW4; ++q) {
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   wr, (uint32_t)(lane * 16), wbase + (ky * RW4 + q) * 1024, 0));
            w[4 * q + 0] = v.x;
            w[4 * q + 1] = v.y;
            w[4 * q + 2] = v.z;
            w[4 * q + 3] = v.w;
        }
        const long long base = (((long long)img * a.rows + oy * a.sh + ky) * a.cols + (long long)ow0 * SW) * CW;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            uint32_t x[NCOL * CWC];
#pragma unroll
            for (int col = 0; col < NCOL; ++col)
#pragma unroll
                for (int j = 0; j < CWC; ++j) x[col * CWC + j] = bits[base + col * CW + ch * CWC + j];
            // Word pairs in runs of the strip's P pixels: P xor/and into
            // separate temporaries, then P counts into the P accumulators.
            // The VALU issues long runs of one instruction faster than
            // alternating dependent pairs (about 3.7 against 4.4 cycles per
            // wave64 instruction, measured); the scheduling barriers keep the
            // runs, and the count is written as the accumulating instruction
            // itself so the compiler cannot split it into a count and an add.
#pragma unroll
            for (int kx = 0; kx < KW; ++kx)
#pragma unroll
                for (int j = 0; j < CWC; ++j) {
                    const uint32_t wv = w[kx * CW + ch * CWC + j];
                    uint32_t t[P];
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        const uint32_t xv = x[(p * SW + kx) * CWC + j];
                        t[p] = AND ? (xv & wv) : (xv ^ wv);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int p = 0; p < P; ++p) asm("v_bcnt_u32_b32 %0, %1, %0" : "+v"(acc[p]) : "v"(t[p]));
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
    }

    const float be_lane = finish_beta();
    if (a.a_pad && tile == 0 && lane < P && ow0 + lane < a.out_w)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, be_lane), make_rsrc(a.beta_out, a.beta_bytes),
                                              (uint32_t)(lane * 4), (uint32_t)(((img * a.out_h + oy) * a.out_w + ow0) * 4), 0);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.acc_out ? (const void *)a.acc_out : (const void *)a.out, a.out_bytes);
    // byte offset of the strip's first output pixel, and the stride between pixels
    const uint32_t obase =
        __builtin_amdgcn_readfirstlane((uint32_t)(((img * a.out_h + oy) * a.out_w + ow0) * a.out_c) * 4u);
    const uint32_t ostep = (uint32_t)a.out_c * 4u;
    // the output value's integer part: window sum (XNOR with its border correction)
    const int full_taps = a.in_c * (KH * KW);  // XNOR value's constant when every tap is in the image
    // The output value's integer part: the window sum (XNOR with its border
    // correction).  FULL: every tap of every pixel of the strip is in the
    // image, so no border term (decided once per wave, not per pixel).
    auto window_value = [&](auto full, int p, int ox) -> int {
        if constexpr (AND) {
            return (int)acc[p];  // a zero word at a padded tap adds nothing
        } else if constexpr (decltype(full)::value) {
            return full_taps - 2 * (int)acc[p];
        } else {
            const int ix0 = ox * SW - a.pw;
            const int c0 = ix0 < 0 ? -ix0 : 0;
            const int c1 = a.in_w - ix0 < KW ? a.in_w - ix0 : KW;
            const int valid = (r1 - r0) * (c1 - c0);
            int corr = 0;
            if (valid != KH * KW) {
                // set weight bits at the padded taps of the rows taken =
                // row band - in-image rectangle (c0, c1 are wave-uniform: a
                // select chain, no register indexing)
                int a0 = 0, a1 = 0, b0 = 0, b1 = 0;
#pragma unroll
                for (int c = 0; c <= KW; ++c) {
                    if (c == c0) { a0 = rt0[c]; a1 = rt1[c]; }
                    if (c == c1) { b0 = rt0[c]; b1 = rt1[c]; }
                }
                corr = (rt1[KW] - rt0[KW]) - (b1 - b0 - a1 + a0);
            }
            return a.in_c * valid - 2 * ((int)acc[p] - corr);
        }
    };
    // The same value as a float, exactly (|value| < 2^24): the full-window
    // XNOR form is one fma on the converted count.
    auto window_value_f = [&](auto full, int p, int ox) -> float {
        if constexpr (!AND && decltype(full)::value)
            return __builtin_fmaf((float)acc[p], -2.0f, (float)full_taps);
        else
            return (float)window_value(full, p, ox);
    };
    // Lanes past out_c store at an out-of-range offset, which the buffer range
    // check discards.
    const uint32_t coff = co_ok ? (uint32_t)(co * 4) : 0x80000000u;
    auto emit = [&](auto full) {
        if (a.bits_out) {
            // one unrolled loop per activation class, as for the values below
            auto store_bits_all = [&](auto bit_of) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int ox = ow0 + p;
                    if (ox >= a.out_w) break;
                    const float be = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(be_lane), p));
                    store_tile_bits(a.bits_out, ((long long)img * a.out_h + oy) * a.out_w + ox, a.out_words,
                                    (int)tile, co_ok && bit_of(p, ox, be));
                }
            };
            if (a.neuron.type == kNeuronRelu)
                store_bits_all([](int, int, float) { return true; });  // a ReLU output is never below 0
            else if (a.neuron.type == kNeuronNone)
                store_bits_all([&](int p, int ox, float be) {
                    return sign_bit(__builtin_fmaf(window_value_f(full, p, ox) * sc, be, bi));
                });
            else
                store_bits_all([&](int p, int ox, float be) {
                    return sign_bit(epilogue_value(window_value_f(full, p, ox), sc, be, bi, a.neuron));
                });
            return;
        }
        // One unrolled loop per output form (window sums, values with and
        // without ReLU), so no per-pixel select between them.
        auto store_all = [&](auto value_bits) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int ox = ow0 + p;
                if (ox >= a.out_w) break;
                const float be = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(be_lane), p));
                __builtin_amdgcn_raw_buffer_store_b32(value_bits(p, ox, be), orr, coff,
                                                      __builtin_amdgcn_readfirstlane(obase + (uint32_t)p * ostep),
                                                      kStoreSc1);
            }
        };
        if (a.acc_out)
            store_all([&](int p, int ox, float) { return (uint32_t)window_value(full, p, ox); });
        else if (a.neuron.type == kNeuronRelu)
            store_all([&](int p, int ox, float be) {
                const float r = __builtin_fmaf(window_value_f(full, p, ox) * sc, be, bi);
                return __builtin_bit_cast(uint32_t, (r < 0.0f) ? 0.0f : r);
            });
        else if (a.neuron.type == kNeuronNone)
            store_all([&](int p, int ox, float be) {
                return __builtin_bit_cast(uint32_t, __builtin_fmaf(window_value_f(full, p, ox) * sc, be, bi));
            });
        else
            store_all([&](int p, int ox, float be) {
                return __builtin_bit_cast(uint32_t, epilogue_value(window_value_f(full, p, ox), sc, be, bi, a.neuron));
            });
    };
    if (!AND && border)
        emit(std::false_type{});
    else
        emit(std::true_type{});
}

template <int KH, int KW, int CW, int SW, int P>
hipError_t launch_fast(XArgs a, const Launch &L, int and_mode)
{
    a.strips_per_row = (a.out_w + P - 1) / P;
    a.strips = (long long)a.n * a.out_h * a.strips_per_row;
    a.div_tiles = make_fastdiv((uint32_t)a.tiles);
    a.div_oh = make_fastdiv((uint32_t)a.out_h);
    a.div_img = make_fastdiv((uint32_t)(a.strips_per_row * a.out_h));
    const long long waves = a.strips * a.tiles;
    const long long blocks = ((waves + 3) / 4 + 7) / 8 * 8;  // a multiple of the 8 XCDs
    if (blocks * 4 * 4 >= 0x7fffffffLL) return hipErrorInvalidValue;
    if (and_mode)
        return launch_kernel(L, xconv_fast<KH, KW, CW, SW, P, true>, dim3((unsigned)blocks), dim3(256), 0, a);
    return launch_kernel(L, xconv_fast<KH, KW, CW, SW, P, false>, dim3((unsigned)blocks), dim3(256), 0, a);
}

}  // namespace

#define BCONV_FAST(KH, KW, CW, SW, P)                                        \
    {KH, KW, CW, SW, P, &launch_fast<KH, KW, CW, SW, P>,                     \
     "xconv_fast<" #KH "," #KW "," #CW "," #SW "," #P ">"}
// the strip widths compiled for each shape
#define BCONV_FAST_P(KH, KW, CW, SW)                                                          \
    BCONV_FAST(KH, KW, CW, SW, 8), BCONV_FAST(KH, KW, CW, SW, 7), BCONV_FAST(KH, KW, CW, SW, 6), \
        BCONV_FAST(KH, KW, CW, SW, 4)

}  // namespace bconv
