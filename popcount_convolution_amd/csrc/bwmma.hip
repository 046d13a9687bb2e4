// binaryWeights convolution on the matrix cores.
//
// Apple "MPSCNNBinaryConvolution" (Overview, binaryWeights bullet): the input
// keeps full precision, each weight bit stands for +1 (bit 1) or -1 (bit 0),
// and the window sum is followed by the fused epilogue
// neuron(sum * scale[c] * beta + bias[c]).
//
// As a matrix product: rows = output pixels (N*Ho*Wo), columns = output
// channels, K = taps x input channels, A = the (affine-transformed, zero
// outside the image) input window, B = the +-1 weights.
//
// Exact products on bf16 matrix cores.  +-1 is exact in bf16.  Every fp32
// input value x splits exactly into three bf16 pieces by truncation:
// hi = x with the low 16 bits cleared, r = x - hi (exact, at most 16
// significant bits), mid = r truncated the same way, lo = r - mid (at most 8
// significant bits, exact in bf16).  So x*w = hi*w + mid*w + lo*w exactly,
// and three v_mfma_f32_16x16x32_bf16 per 32-deep K step accumulate the
// products in fp32, as the VALU path would (the matrix core keeps
// subnormal operands and results, checked on gfx950).  An infinite x has
// hi = x; its remainders are those of +-FLT_MAX (finite), so the sum stays
// infinite.
// Below |x| = 2^-110 the last piece can hold bits finer than bf16's
// smallest subnormal (2^-133); those bits show up as nonzero low halves of
// the final remainder.  When any lane of a step has them, the lost part
// (below 2^-133, at most 16 significant bits) is scaled by 2^32, split into
// two more bf16 pieces and multiplied by the weights scaled by 2^-32 (+-2^-32
// is exact in bf16, and the product is an exact fp32 value), so every finite
// fp32 input enters exactly.
//
// Mapping on gfx950:
//  * the weights are the A operand (rows = 16 output channels) and the
//    input the B operand (columns = 16 output pixels), so each lane ends
//    with 4 consecutive channels of one pixel (one 16-byte store) and that
//    pixel is the one whose input it loaded;
//  * a workgroup = 8 waves = 64 output pixels x 64 output channels: wave w
//    owns pixels 16*(w%4)..+15, all four 16-channel blocks, and half of the
//    K steps (w/4); the two halves are summed through LDS at the end;
//  * K is walked in steps of 32: (tap, 32-channel chunk), advanced without
//    divisions; lane l loads the 8 channels 8*(l/16)..+7 of its pixel l%16
//    (two 16-byte loads), exactly the B operand of the 16x16x32
//    instruction; taps outside the image read zero through the buffer range
//    check; two input buffers keep the loads of step s+2 in flight while
//    step s runs;
//  * the bf16 weight fragments of the workgroup's 64 channels are staged in
//    LDS (up to 18 K steps = 72 KiB per stage), read with one ds_read_b128
//    per channel block;
//  * workgroups are dealt to the eight XCDs so that each XCD works on a
//    contiguous range of output pixels (its L2 then holds the input rows its
//    windows share).
#include "internal.h"

namespace bconv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPixTile = 64;    // output pixels per workgroup (4 pixel groups x 16)
constexpr int kChanTile = 64;   // output channels per workgroup (4 x 16)
constexpr int kStage = 18;      // K steps of weight fragments per LDS stage
constexpr int kStepU4 = 256;    // 16-byte fragment entries per K step (4 blocks x 64 lanes)
constexpr int kXcds = 8;
constexpr int kThreads = 512;   // 8 waves: 4 pixel groups x 2 K halves
#ifndef BWMMA_PREFETCH
#define BWMMA_PREFETCH 2
#endif
constexpr int kPrefetch = BWMMA_PREFETCH;  // K steps of input loads in flight per wave
constexpr int kRedBytes = 4 * 4 * 64 * 16;  // LDS for summing the K halves
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: loads return 0

struct MmaArgs {
    const float *x, *in_scale, *in_bias;
    const u32x4 *frag;  // [ntiles][ksteps][4][64] 16-byte bf16 fragments
    const float *scale, *bias;
    const float *a_pad;  // zero-halo A map or nullptr (beta = 1)
    float *beta_out;
    int beta_valid;      // beta divisor: in-image taps instead of kh*kw
    float scale_value;
    Neuron neuron;
    float *out;
    float *acc_out;
    uint32_t *bits_out;  // packed sign bits instead of out (see Epilogue)
    int out_words;
    int n, in_h, in_w, in_c, out_c, out_h, out_w, kh, kw, sh, sw, ph, pw;
    int chunks, ksteps, ntiles, mtiles, rows, cols, m_total;
    int x_bytes, out_bytes;
    int vec_out;  // out_c % 4 == 0 and a 16-byte aligned destination: 16-byte stores
};

// Exact three-way bf16 split of 8 floats (see the file comment); element j
// of each result is bits 16*(j%2).. of dword j/2, the bf16x8 operand order.
__device__ __forceinline__ float trunc16(float x)
{
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & 0xffff0000u);
}

// Upper halves of (even, odd) floats -> one dword of two bf16.
__device__ __forceinline__ uint32_t pack_hi(float even, float odd)
{
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, odd), __builtin_bit_cast(uint32_t, even), 0x07060302u);
}

// Also returns the final remainders r2 (lo is their upper half).
__device__ __forceinline__ void split3(const float v[8], u32x4 &hi, u32x4 &mid, u32x4 &lo, float r2[8])
{
    float r1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // The remainders come from x clamped to +-FLT_MAX: the same for finite
        // x, finite for +-inf (whose hi piece is the infinity itself), NaN or
        // garbage next to a NaN hi piece for NaN x.
        const float xc = __builtin_amdgcn_fmed3f(v[j], -3.40282347e38f, 3.40282347e38f);
        r1[j] = xc - trunc16(xc);
        r2[j] = r1[j] - trunc16(r1[j]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        hi[p] = pack_hi(v[2 * p], v[2 * p + 1]);
        mid[p] = pack_hi(r1[2 * p], r1[2 * p + 1]);
        lo[p] = pack_hi(r2[2 * p], r2[2 * p + 1]);
    }
}

// The bits of r2 below bf16's reach, scaled by 2^32 and split in two.
__device__ __forceinline__ void split_lost(const float r2[8], u32x4 &th, u32x4 &tl)
{
    float t[8], u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        t[j] = (r2[j] - trunc16(r2[j])) * 4294967296.0f;  // exact: below 2^-133 before scaling
        u[j] = t[j] - trunc16(t[j]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        th[p] = pack_hi(t[2 * p], t[2 * p + 1]);
        tl[p] = pack_hi(u[2 * p], u[2 * p + 1]);
    }
}

__device__ __forceinline__ f32x4 mma(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Tap (ky, kx) and 32-channel chunk q of a K step (s = (ky*kw + kx)*chunks + q).
struct StepPos {
    int ky, kx, q;
};

__device__ __forceinline__ StepPos step_pos(const MmaArgs &a, int s)
{
    const int tap = s / a.chunks;
    return StepPos{tap / a.kw, tap % a.kw, s % a.chunks};
}

__device__ __forceinline__ void advance(const MmaArgs &a, StepPos &p)
{
    if (++p.q == a.chunks) {
        p.q = 0;
        if (++p.kx == a.kw) {
            p.kx = 0;
            ++p.ky;
        }
    }
}

// One lane's 8 input values of the K step at p (zero outside the image or
// past in_c).  lane_base = element index of channel cg of input pixel
// (iy0, ix0) (negative or past the image for padded windows: then unused).
// With AFFINE both in_scale and in_bias are set.
template <bool VEC8, bool AFFINE>
__device__ __forceinline__ void load_step(const MmaArgs &a, const __amdgpu_buffer_rsrc_t &xr, const StepPos &p,
                                          int lane_base, int iy0, int ix0, int cg, bool live, float v[8])
{
    const int iy = iy0 + p.ky, ix = ix0 + p.kx;
    // bitwise & keeps this branch-free
    const bool inside = live & ((unsigned)iy < (unsigned)a.in_h) & ((unsigned)ix < (unsigned)a.in_w);
    const int c = p.q * 32 + cg;
    const int tap_off = (p.ky * a.in_w + p.kx) * a.in_c + p.q * 32;  // uniform
    const uint32_t pix_off = (uint32_t)(lane_base + tap_off) * 4u;
    if constexpr (VEC8) {
        const uint32_t off = (inside & (c < a.in_c)) ? pix_off : kOob;
        const f32x4 p0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        const f32x4 p1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u, 0, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = p0[j];
            v[4 + j] = p1[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = (inside & (c + j < a.in_c)) ? pix_off + 4u * j : kOob;
            v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0));
        }
    }
    if constexpr (AFFINE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = inside & (c + j < a.in_c);
            const int cj = ok ? c + j : 0;
            v[j] = ok ? __builtin_fmaf(v[j], a.in_scale[cj], a.in_bias[cj]) : 0.0f;
        }
    }
}

// One K step: split the lane's 8 inputs, multiply by the four 16-channel
// weight blocks at bs (this lane's entry of the step in LDS).
__device__ __forceinline__ void mma_step(f32x4 acc[4], const float x[8], const u32x4 *bs)
{
    u32x4 ph, pm, pl;
    float r2[8];
    split3(x, ph, pm, pl, r2);
    uint32_t low = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) low |= __builtin_bit_cast(uint32_t, r2[j]);
    u32x4 b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = bs[t * 64];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mma(b[t], ph, acc[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mma(b[t], pm, acc[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mma(b[t], pl, acc[t]);
    if (__builtin_amdgcn_ballot_w64((low & 0xffffu) != 0u)) {  // rare: inputs below 2^-110
        // the lost bits, scaled by 2^32, times the weights scaled by 2^-32
        // (bf16 +-1 -> +-2^-32 flips exponent bit 12; zero stays zero)
        u32x4 th, tl;
        split_lost(r2, th, tl);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4 bt;
#pragma unroll
            for (int k = 0; k < 4; ++k) bt[k] = b[t][k] ^ ((b[t][k] >> 1) & 0x10001000u);
            acc[t] = mma(bt, th, acc[t]);
            acc[t] = mma(bt, tl, acc[t]);
        }
    }
}

template <bool VEC8, bool AFFINE>
__global__ __launch_bounds__(kThreads) void bwmma_kernel(MmaArgs a)
{
    extern __shared__ u32x4 stage[];  // [min(ksteps, kStage)][4][64], at least kRedBytes
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int group = wave & 3, khalf = wave >> 2;
    // XCD-aware numbering: block b runs on XCD b % 8; XCD x takes the
    // contiguous tile range [x*per, (x+1)*per).
    const int blocks = a.mtiles * a.ntiles;
    const int per = (blocks + kXcds - 1) / kXcds;
    const int idx = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (idx >= blocks) return;  // uniform over the workgroup
    const int mtile = idx / a.ntiles, ntile = idx - (idx / a.ntiles) * a.ntiles;

    // this lane's output pixel (pixels past the batch reuse the last one and
    // are not stored)
    const int p_raw = mtile * kPixTile + group * 16 + (lane & 15);
    const bool live = p_raw < a.m_total;
    const int pix = live ? p_raw : a.m_total - 1;
    const int hw = a.out_h * a.out_w;
    const int img = pix / hw, rem = pix - (pix / hw) * hw;
    const int oy = rem / a.out_w, ox = rem - (rem / a.out_w) * a.out_w;
    const int iy0 = oy * a.sh - a.ph, ix0 = ox * a.sw - a.pw;
    const int cg = (lane >> 4) * 8;
    const int lane_base = ((img * a.in_h + iy0) * a.in_w + ix0) * a.in_c + cg;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);

    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // epilogue operands, loaded now so their latency hides behind the loop:
    // channels ntile*64 + 16*(keep+u) + 4*(lane/16) + r
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
    // beta of this lane's pixel: window sum of the zero-halo A map / (kh*kw,
    // or the in-image taps)
    float be = 1.0f;
    if (a.a_pad) {
        const float *ap = a.a_pad + ((long long)img * a.rows + oy * a.sh) * a.cols + ox * a.sw;
        float sum = 0.0f;
        for (int ky = 0; ky < a.kh; ++ky)
            for (int kx = 0; kx < a.kw; ++kx) sum += ap[ky * a.cols + kx];
        be = sum / (float)(a.beta_valid ? window_valid_taps(oy, ox, a.sh, a.sw, a.ph, a.pw, a.kh, a.kw, a.in_h, a.in_w) : a.kh * a.kw);
    }

    const u32x4 *gfrag = a.frag + (long long)ntile * a.ksteps * kStepU4;
    for (int s0 = 0; s0 < a.ksteps; s0 += kStage) {
        const int cnt = a.ksteps - s0 < kStage ? a.ksteps - s0 : kStage;
        const int half = (cnt + 1) >> 1;
        const int sb = s0 + (khalf ? half : 0), se = s0 + (khalf ? cnt : half);
        // A ring of kPrefetch input buffers, each refilled right after its
        // step is split: a load has kPrefetch steps of work to arrive, and
        // the matrix-core work of one step overlaps the split of the next.
        // Loads past this wave's last step read in-bounds data (or zero) that
        // is never used.
        StepPos lpos = step_pos(a, sb);
        float xbuf[kPrefetch][8];
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) {
            load_step<VEC8, AFFINE>(a, xr, lpos, lane_base, iy0, ix0, cg, live, xbuf[i]);
            advance(a, lpos);
        }
        __syncthreads();  // previous stage fully read
        for (int i = threadIdx.x; i < cnt * kStepU4; i += kThreads) stage[i] = gfrag[(long long)s0 * kStepU4 + i];
        __syncthreads();
        int s = sb;
        for (; s + kPrefetch <= se; s += kPrefetch) {
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) {
                mma_step(acc, xbuf[i], stage + (s + i - s0) * kStepU4 + lane);
                load_step<VEC8, AFFINE>(a, xr, lpos, lane_base, iy0, ix0, cg, live, xbuf[i]);
                advance(a, lpos);
            }
        }
#pragma unroll
        for (int i = 0; i < kPrefetch - 1; ++i)
            if (s + i < se) mma_step(acc, xbuf[i], stage + (s + i - s0) * kStepU4 + lane);
    }

    // Sum the two K halves: the first half keeps channel blocks 0,1, the
    // second 2,3; each sends the other pair through LDS (khalf selects a
    // branch, so every register index stays static).
    f32x4 *red = reinterpret_cast<f32x4 *>(stage) + group * 4 * 64 + lane;  // [4 groups][4 blocks][64]
    __syncthreads();  // stage fully read
    if (khalf == 0) {
        red[2 * 64] = acc[2];
        red[3 * 64] = acc[3];
    } else {
        red[0] = acc[0];
        red[64] = acc[1];
    }
    __syncthreads();
    f32x4 res[2];
    if (khalf == 0) {
        res[0] = acc[0] + red[0];
        res[1] = acc[1] + red[64];
    } else {
        res[0] = acc[2] + red[2 * 64];
        res[1] = acc[3] + red[3 * 64];
    }
    // Epilogue: element r of block keep+u is pixel p_raw, channel
    // ntile*64 + 16*(keep+u) + 4*(lane/16) + r.
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
                const float y = epilogue_value(res[u][r], sc[u][r], be, bi[u][r], a.neuron);
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
        f32x4 v = res[u];
        // one loop per output form, so no per-element select among activations
        if (a.acc_out) {
        } else if (a.neuron.type == kNeuronNone) {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(v[r] * sc[u][r], be, bi[u][r]);
        } else if (a.neuron.type == kNeuronRelu) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float y = __builtin_fmaf(v[r] * sc[u][r], be, bi[u][r]);
                v[r] = (y < 0.0f) ? 0.0f : y;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = epilogue_value(v[r], sc[u][r], be, bi[u][r], a.neuron);
        }
        const uint32_t off = (uint32_t)(pix * a.out_c + co) * 4u;
        if (a.vec_out && co + 3 < a.out_c) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), orr, off, 0, kStoreSc1);
        } else {
            // Cast the whole vector, then take elements: this compiler reads
            // element x for a bit-cast of a single float-vector element.
            const u32x4 w = __builtin_bit_cast(u32x4, v);
            if (co < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.x, orr, off, 0, kStoreSc1);
            if (co + 1 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.y, orr, off + 4u, 0, kStoreSc1);
            if (co + 2 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.z, orr, off + 8u, 0, kStoreSc1);
            if (co + 3 < a.out_c) __builtin_amdgcn_raw_buffer_store_b32(w.w, orr, off + 12u, 0, kStoreSc1);
        }
    }
}

// bf16 +-1 fragments [ntiles][ksteps][4][64] x 8: entry (tile, s, t, lane),
// element j is the weight of output channel 64*tile + 16t + lane%16 at tap
// s / chunks, input channel 32*(s % chunks) + 8*(lane/16) + j; 0 for channels
// past out_c or in_c.
__global__ void prepack_bwmma_kernel(const uint32_t *__restrict__ user, u32x4 *__restrict__ frag, int out_c,
                                     int taps, int words, int in_c, int chunks, int ksteps, int ntiles)
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
    for (int j = 0; j < 8; ++j) {
        const int f = q * 32 + 8 * (lane >> 4) + j;
        uint32_t h = 0;  // bf16 +0
        if (co < out_c && f < in_c) {
            const uint32_t word = user[((long long)co * taps + tap) * words + f / 32];
            h = ((word >> (f % 32)) & 1u) ? 0x3f80u : 0xbf80u;  // +1 / -1
        }
        r[j / 2] |= h << (16 * (j % 2));
    }
    frag[t] = r;
}

}  // namespace

size_t bwmma_frag_bytes(const Geom &g)
{
    const long long chunks = (g.in_c + 31) / 32;
    const long long ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    return (size_t)(ntiles * g.kh * g.kw * chunks * kStepU4 * 16);
}

hipError_t launch_prepack_bwmma(const Geom &g, hipStream_t s, const uint32_t *user_bits, void *frag)
{
    const int chunks = (g.in_c + 31) / 32;
    const int ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    const int ksteps = g.kh * g.kw * chunks;
    const long long total = (long long)ntiles * ksteps * kStepU4;
    hipLaunchKernelGGL(prepack_bwmma_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, user_bits,
                       static_cast<u32x4 *>(frag), g.out_c, g.kh * g.kw, g.words, g.in_c, chunks, ksteps, ntiles);
    return hipGetLastError();
}

static bool vec8(const Geom &g) { return g.in_c % 8 == 0; }

const char *bwmma_kernel_name(const Geom &g, bool affine)
{
    static const char *const names[4] = {"bwmma_kernel<false,false>", "bwmma_kernel<false,true>",
                                         "bwmma_kernel<true,false>", "bwmma_kernel<true,true>"};
    return names[(vec8(g) ? 2 : 0) + (affine ? 1 : 0)];
}

hipError_t launch_bwmma(const Geom &g, const Launch &L, const float *x, const float *in_scale, const float *in_bias,
                        const void *frag, const Epilogue &e, float *out, float *acc_out)
{
    MmaArgs a{};
    a.x = x;
    a.in_scale = in_scale;
    a.in_bias = in_bias;
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
    a.chunks = (g.in_c + 31) / 32;
    a.ksteps = g.kh * g.kw * a.chunks;
    a.ntiles = (g.out_c + kChanTile - 1) / kChanTile;
    const long long m_total = (long long)g.n * g.out_h * g.out_w;
    const long long mtiles = (m_total + kPixTile - 1) / kPixTile;
    a.rows = g.bits_rows;
    a.cols = g.bits_cols;
    const long long x_bytes = (long long)g.n * g.in_h * g.in_w * g.in_c * 4;
    const long long out_bytes = m_total * g.out_c * 4;
    if (m_total == 0) return hipSuccess;
    // every buffer offset and work index stays below 2^31
    // (the fragment table itself may exceed 2 GiB: it is indexed with 64-bit offsets)
    if (x_bytes >= 0x7fffffffLL || out_bytes >= 0x7fffffffLL || mtiles * a.ntiles >= 0x7fffffffLL - kXcds ||
        (long long)a.ksteps * kStepU4 >= 0x7fffffffLL)
        return hipErrorInvalidValue;
    a.m_total = (int)m_total;
    a.mtiles = (int)mtiles;
    a.x_bytes = (int)x_bytes;
    a.out_bytes = (int)out_bytes;
    const void *dst = acc_out ? (const void *)acc_out : (const void *)out;
    a.vec_out = g.out_c % 4 == 0 && (uintptr_t)dst % 16 == 0;
    const int blocks = a.mtiles * a.ntiles;
    const int grid = (blocks + kXcds - 1) / kXcds * kXcds;
    const uint32_t stage_bytes = (uint32_t)(a.ksteps < kStage ? a.ksteps : kStage) * kStepU4 * 16;
    const uint32_t lds = stage_bytes > kRedBytes ? stage_bytes : kRedBytes;
    // input affine: both arrays or neither (the handle fills in a missing one)
    const bool affine = in_scale != nullptr;
    if ((in_scale != nullptr) != (in_bias != nullptr)) return hipErrorInvalidValue;
    const dim3 gr(grid), bl(kThreads);
    if (vec8(g))
        return affine ? launch_kernel(L, bwmma_kernel<true, true>, gr, bl, lds, a)
                      : launch_kernel(L, bwmma_kernel<true, false>, gr, bl, lds, a);
    return affine ? launch_kernel(L, bwmma_kernel<false, true>, gr, bl, lds, a)
                  : launch_kernel(L, bwmma_kernel<false, false>, gr, bl, lds, a);
}

}  // namespace bconv
