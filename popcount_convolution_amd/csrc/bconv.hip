// Host side of libbconv.so: argument checks, handle lifecycle, workspace
// layout and the forward dispatch.  Every step of the forward pass runs in the
// kernels of this library; this file only checks, sizes and launches.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bconv.h"
#include "internal.h"

struct bconv_handle {
    bconv_desc_t desc;
    int32_t type;
    uint32_t flags;
    int device;
    int out_h, out_w, words, tiles;
    int simds;                // SIMD units of the device
    bool force_generic;
    bool small_fused;         // small layers take the single-launch kernel (BCONV_SMALL_FUSED)
    int strip_width;          // forced strip width of the specialised convolution (0: by cost)
    bconv::LaneWeights lane;  // XNOR / AND
    uint32_t *d_lane_words;
    int32_t *d_lane_popc;
    uint32_t *d_flat;         // K-major weights of the fully connected route
    bool gemm;
    void *d_f4;               // fp4 matrix-core comparison path: weight table and set-bit counts
    bool i8;                  // int8 matrix-core comparison path (XNOR / AND)
    void *d_i8frag;           // its int8 weight fragments
    float *d_pm;              // binaryWeights, VALU kernel (+-1.0f table)
    int pm_cols;
    void *d_mma;              // binaryWeights, matrix-core kernel (bf16 fragments)
    float *d_out_scale, *d_out_bias, *d_in_scale, *d_in_bias;
};

namespace {

thread_local std::string g_last_error;

bconv_status_t fail(bconv_status_t s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bconv_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(BCONV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int32_t kMaxExtent = 1 << 16;
constexpr int32_t kMaxChannels = 1 << 20;
constexpr long long kMaxWindowBits = 1LL << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Output extent for leading padding p and trailing padding pe.
int out_dim(int in, int k, int s, int p, int pe) { return (in + p + pe - k) / s + 1; }

bconv_status_t check_desc(const bconv_desc_t *d, int32_t type, uint32_t flags)
{
    if (!d) return fail(BCONV_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (type != BCONV_BINARY_WEIGHTS && type != BCONV_XNOR && type != BCONV_AND)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "unknown type %d", type);
    if (flags & ~(uint32_t)(BCONV_FLAG_USE_BETA_SCALING | BCONV_FLAG_INT8_MFMA | BCONV_FLAG_BETA_VALID_TAPS |
                            BCONV_FLAG_FP4_MFMA))
        return fail(BCONV_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
    if ((flags & BCONV_FLAG_BETA_VALID_TAPS) && !(flags & BCONV_FLAG_USE_BETA_SCALING))
        return fail(BCONV_ERR_INVALID_ARGUMENT, "BCONV_FLAG_BETA_VALID_TAPS requires BCONV_FLAG_USE_BETA_SCALING");
    if ((flags & BCONV_FLAG_INT8_MFMA) && type == BCONV_BINARY_WEIGHTS)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "BCONV_FLAG_INT8_MFMA applies to XNOR and AND only");
    if ((flags & BCONV_FLAG_FP4_MFMA) && type == BCONV_BINARY_WEIGHTS)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "BCONV_FLAG_FP4_MFMA applies to XNOR and AND only");
    if ((flags & BCONV_FLAG_FP4_MFMA) && (flags & BCONV_FLAG_INT8_MFMA))
        return fail(BCONV_ERR_INVALID_ARGUMENT, "BCONV_FLAG_FP4_MFMA and BCONV_FLAG_INT8_MFMA exclude each other");
    if (d->neuron < 0 || d->neuron >= BCONV_NEURON_COUNT)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "unknown neuron %d", d->neuron);
    if (d->groups <= 0) return fail(BCONV_ERR_INVALID_ARGUMENT, "groups must be >= 1");
    if (d->groups != 1) return fail(BCONV_ERR_UNSUPPORTED, "groups > 1 is not supported");
    if (d->in_h < 1 || d->in_w < 1 || d->in_h > kMaxExtent || d->in_w > kMaxExtent)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "in_h/in_w must be in [1, %d]", kMaxExtent);
    if (d->in_c < 1 || d->out_c < 1 || d->in_c > kMaxChannels || d->out_c > kMaxChannels)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "in_c/out_c must be in [1, %d]", kMaxChannels);
    if (d->kernel_h < 1 || d->kernel_w < 1 || d->kernel_h > kMaxExtent || d->kernel_w > kMaxExtent)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "kernel extents must be >= 1");
    if (d->stride_h < 1 || d->stride_w < 1 || d->stride_h > kMaxExtent || d->stride_w > kMaxExtent)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "strides must be >= 1");
    if (d->pad_h < 0 || d->pad_w < 0 || d->pad_h >= d->kernel_h || d->pad_w >= d->kernel_w ||
        d->pad_h_end < 0 || d->pad_w_end < 0 || d->pad_h_end >= d->kernel_h || d->pad_w_end >= d->kernel_w)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "padding must satisfy 0 <= pad < kernel");
    if (d->in_h + d->pad_h + d->pad_h_end < d->kernel_h || d->in_w + d->pad_w + d->pad_w_end < d->kernel_w)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "kernel larger than the padded input");
    if ((long long)d->in_c * d->kernel_h * d->kernel_w > kMaxWindowBits)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "in_c*kernel_h*kernel_w exceeds 2^24");
    return BCONV_OK;
}

bconv::Geom make_geom(const bconv_handle *h, int n)
{
    const bconv_desc_t &d = h->desc;
    bconv::Geom g{};
    g.n = n;
    g.in_h = d.in_h;
    g.in_w = d.in_w;
    g.in_c = d.in_c;
    g.out_c = d.out_c;
    g.kh = d.kernel_h;
    g.kw = d.kernel_w;
    g.sh = d.stride_h;
    g.sw = d.stride_w;
    g.ph = d.pad_h;
    g.pw = d.pad_w;
    g.out_h = h->out_h;
    g.out_w = h->out_w;
    g.words = h->words;
    g.tiles = h->tiles;
    g.simds = h->simds;
    g.strip_p = h->strip_width;
    g.bits_halo_h = d.pad_h;
    g.bits_halo_w = d.pad_w;
    g.bits_rows = d.in_h + d.pad_h + d.pad_h_end;
    g.bits_cols = d.in_w + d.pad_w + d.pad_w_end;
    // A strip of the specialised kernel may read past the last column of the
    // last row; those words exist and are zero.
    g.bits_slack_words = (long long)(8 * g.sw + g.kw) * g.words + 64;
    return g;
}

bool uses_bits(const bconv_handle *h) { return h->type != BCONV_BINARY_WEIGHTS; }
bool uses_beta(const bconv_handle *h) { return (h->flags & BCONV_FLAG_USE_BETA_SCALING) != 0; }

bconv_workspace_layout_t layout_for(const bconv_handle *h, int n)
{
    bconv_workspace_layout_t L{};
    L.bits_offset = L.a_map_offset = L.beta_offset = SIZE_MAX;
    const bconv::Geom g = make_geom(h, n);
    size_t off = 0;
    if (uses_bits(h) && n > 0) {
        L.bits_offset = off;
        L.bits_rows = g.bits_rows;
        L.bits_cols = g.bits_cols;
        L.bits_words = h->i8 ? bconv::i8_cpad(g.in_c) / 4 : g.words;
        L.bits_pad_h = g.bits_halo_h;
        L.bits_pad_w = g.bits_halo_w;
        if (h->i8) {
            off = align_up(off + bconv::i8_act_bytes(g));
        } else {
            const size_t words = (size_t)n * g.bits_rows * g.bits_cols * g.words + (size_t)g.bits_slack_words;
            off = align_up(off + words * 4);
        }
    }
    if (uses_beta(h) && n > 0) {
        // A map with the same zero halo as the bit buffer; beta as written by
        // the convolution kernels.
        L.a_map_offset = off;
        L.bits_rows = g.bits_rows;
        L.bits_cols = g.bits_cols;
        L.bits_pad_h = g.bits_halo_h;
        L.bits_pad_w = g.bits_halo_w;
        off = align_up(off + (size_t)n * g.bits_rows * g.bits_cols * 4);
        L.beta_offset = off;
        off = align_up(off + (size_t)n * g.out_h * g.out_w * 4);
    }
    L.total_bytes = off;
    return L;
}

// Runs `fn` with the handle's device current, restoring the caller's device.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
        else if (err == hipSuccess) prev = -1;
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

template <typename T>
bconv_status_t upload(const T *host, size_t count, T **dev)
{
    *dev = nullptr;
    if (!host || count == 0) return BCONV_OK;
    hipError_t e = hipMalloc(reinterpret_cast<void **>(dev), count * sizeof(T));
    if (e != hipSuccess) {
        *dev = nullptr;
        return fail(BCONV_ERR_ALLOC, "hipMalloc(%zu): %s", count * sizeof(T), hipGetErrorString(e));
    }
    e = hipMemcpy(*dev, host, count * sizeof(T), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
    return BCONV_OK;
}

void release(bconv_handle *h)
{
    if (!h) return;
    void *ptrs[] = {h->d_lane_words, h->d_lane_popc, h->d_flat, h->d_f4, h->d_pm, h->d_mma, h->d_i8frag, h->d_out_scale,
                    h->d_out_bias, h->d_in_scale, h->d_in_bias};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    delete h;
}

bool ranges_overlap(const void *a, size_t an, const void *b, size_t bn)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Whether a call with fp32 input takes the single-launch small-layer kernel.
bool takes_small(const bconv_handle *h, const bconv::Geom &g)
{
    return h->small_fused && !h->force_generic && !h->i8 && !h->d_f4 && h->type != BCONV_BINARY_WEIGHTS &&
           !uses_beta(h) &&
           bconv::small_route(g);
}

// Output forms: fp32 values, raw window sums, or packed sign bits of the
// fp32 values ([n][out_h][out_w][ceil(out_c/32)] words).
enum class Sink { Output, Accum, Bits };

// Input forms: fp32 NHWC values, or sign bits already packed in the layout
// of the bit buffer without its halo ([n][in_h][in_w][ceil(in_c/32)] words).
enum class Source { Values, Bits };

bconv_status_t forward_impl(bconv_t h, void *stream, int32_t n, const void *src, Source source, void *dst,
                            Sink sink, void *workspace, size_t workspace_bytes, void *ev_begin, void *ev_end,
                            void *ev_pack_begin = nullptr, void *ev_pack_end = nullptr)
{
    if (!h) return fail(BCONV_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (n < 0) return fail(BCONV_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (source == Source::Bits) {
        // Packed bits carry only the signs: every step that reads the
        // full-precision input is out of reach.
        if (h->type == BCONV_BINARY_WEIGHTS)
            return fail(BCONV_ERR_UNSUPPORTED, "binaryWeights multiplies the full-precision input, not its sign");
        if (uses_beta(h))
            return fail(BCONV_ERR_UNSUPPORTED, "beta needs |input|, which packed sign bits do not carry");
        if (h->d_in_scale || h->d_in_bias)
            return fail(BCONV_ERR_UNSUPPORTED, "the input scale and bias apply before the sign");
        if (h->i8) return fail(BCONV_ERR_UNSUPPORTED, "the int8 matrix-core path takes fp32 input only");
    }
    if (n == 0) return BCONV_OK;
    if (!src || !dst) return fail(BCONV_ERR_INVALID_ARGUMENT, "in/out must not be NULL");
    const bconv_desc_t &d = h->desc;
    const float *in = source == Source::Values ? static_cast<const float *>(src) : nullptr;
    const size_t in_bytes =
        (size_t)n * d.in_h * d.in_w * (source == Source::Bits ? (size_t)((d.in_c + 31) / 32) : (size_t)d.in_c) * 4;
    const int out_words = (d.out_c + 31) / 32;
    const size_t out_bytes =
        (size_t)n * h->out_h * h->out_w * (sink == Sink::Bits ? (size_t)out_words : (size_t)d.out_c) * 4;
    if (ranges_overlap(src, in_bytes, dst, out_bytes))
        return fail(BCONV_ERR_INVALID_ARGUMENT, "input and output overlap");
    if ((long long)n * d.in_h * d.in_w >= (1LL << 31) || (long long)n * h->out_h * h->out_w * h->tiles >= (1LL << 29) ||
        in_bytes >= (size_t)0x7fffffff || out_bytes >= (size_t)0x7fffffff)
        return fail(BCONV_ERR_INVALID_ARGUMENT,
                    "batch too large for one call: input and output must each stay below 2 GiB");
    const bconv_workspace_layout_t L = layout_for(h, n);
    if (L.bits_offset != SIZE_MAX && (long long)n * L.bits_rows * L.bits_cols * L.bits_words +
                                             make_geom(h, n).bits_slack_words >= 0x7fffffffLL)
        return fail(BCONV_ERR_INVALID_ARGUMENT,
                    "batch too large for one call: the padded bit buffer must stay below 2^31 words");
    if (L.total_bytes > 0 && (!workspace || workspace_bytes < L.total_bytes))
        return fail(BCONV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    if (L.total_bytes > 0 && (ranges_overlap(workspace, L.total_bytes, src, in_bytes) ||
                              ranges_overlap(workspace, L.total_bytes, dst, out_bytes)))
        return fail(BCONV_ERR_INVALID_ARGUMENT, "workspace overlaps input or output");

    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bconv::Geom g = make_geom(h, n);
    char *ws = static_cast<char *>(workspace);
    uint32_t *bits = L.bits_offset == SIZE_MAX ? nullptr : reinterpret_cast<uint32_t *>(ws + L.bits_offset);
    float *a_map = L.a_map_offset == SIZE_MAX ? nullptr : reinterpret_cast<float *>(ws + L.a_map_offset);
    float *beta = L.beta_offset == SIZE_MAX ? nullptr : reinterpret_cast<float *>(ws + L.beta_offset);

    hipError_t e;
    const bconv::Launch first{s, static_cast<hipEvent_t>(ev_pack_begin), static_cast<hipEvent_t>(ev_pack_end)};
    const bool small = source == Source::Values && takes_small(h, g);
    if (small) {
        // one kernel binarises and convolves; nothing is written to the workspace
    } else if (source == Source::Bits) {
        e = bconv::launch_repad(g, first, static_cast<const uint32_t *>(src), bits);
        if (e != hipSuccess) return hip_fail(e, "repad kernel");
    } else if (h->i8) {
        e = bconv::launch_pack_i8(g, first, in, h->d_in_scale, h->d_in_bias, h->type == BCONV_AND,
                                  reinterpret_cast<int8_t *>(bits), a_map);
        if (e != hipSuccess) return hip_fail(e, "int8 pack kernel");
    } else if (bits || a_map) {
        e = bconv::launch_pack(g, first, in, h->d_in_scale, h->d_in_bias, bits, a_map);
        if (e != hipSuccess) return hip_fail(e, "pack kernel");
    }
    bconv::Epilogue ep{};
    ep.scale = h->d_out_scale;
    ep.bias = h->d_out_bias;
    ep.scale_value = d.scale_value;
    ep.a_pad = a_map;
    ep.beta_out = beta;
    ep.neuron = bconv::Neuron{d.neuron, d.neuron_a, d.neuron_b};
    ep.beta_valid_taps = (h->flags & BCONV_FLAG_BETA_VALID_TAPS) ? 1 : 0;
    if (sink == Sink::Bits) {
        ep.bits_out = static_cast<uint32_t *>(dst);
        ep.out_words = out_words;
    }
    const bconv::Launch main{s, static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)};
    if (small) {
        e = bconv::launch_xconv_small(g, main, h->type == BCONV_AND, in, h->d_in_scale, h->d_in_bias, h->lane, ep,
                                      sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                                      sink == Sink::Accum ? static_cast<int32_t *>(dst) : nullptr);
    } else if (h->i8) {
        e = bconv::launch_i8mma(g, main, reinterpret_cast<const int8_t *>(bits), h->d_i8frag, ep,
                                sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                                sink == Sink::Accum ? static_cast<int32_t *>(dst) : nullptr);
    } else if (h->type == BCONV_BINARY_WEIGHTS && !h->force_generic) {
        e = bconv::launch_bwmma(g, main, in, h->d_in_scale, h->d_in_bias, h->d_mma, ep,
                                sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                                sink == Sink::Accum ? static_cast<float *>(dst) : nullptr);
    } else if (h->type == BCONV_BINARY_WEIGHTS) {
        e = bconv::launch_bwconv(g, main, in, h->d_in_scale, h->d_in_bias, h->d_pm, h->pm_cols, ep,
                                 sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                                 sink == Sink::Accum ? static_cast<float *>(dst) : nullptr);
    } else if (h->d_f4 && !h->force_generic) {
        e = bconv::launch_f4(g, main, h->type == BCONV_AND, bits, h->d_f4, ep,
                             sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                             sink == Sink::Accum ? static_cast<int32_t *>(dst) : nullptr);
    } else if (h->gemm && !h->force_generic) {
        e = bconv::launch_gemm(g, main, h->type == BCONV_AND, bits, h->d_flat, ep,
                               sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                               sink == Sink::Accum ? static_cast<int32_t *>(dst) : nullptr);
    } else {
        e = bconv::launch_xconv(g, main, h->type == BCONV_AND, bits, h->lane, ep,
                                sink == Sink::Output ? static_cast<float *>(dst) : nullptr,
                                sink == Sink::Accum ? static_cast<int32_t *>(dst) : nullptr,
                                !h->force_generic);
    }
    if (e != hipSuccess) return hip_fail(e, "convolution kernel");
    return BCONV_OK;
}

// Workspace of bconv_forward_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes `scratch` itself
// (on the host that name is a stand-in, not a device address): each device's
// address is taken once with hipGetSymbolAddress, with that device current,
// and kept in scratch_ptr[].
__device__ __align__(256) unsigned char scratch[BCONV_SCRATCH_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// Address of this device's scratch array; `dev` must be the current device.
// Resolved on the first call per device (bconv_create calls it at set-up).
bconv_status_t scratch_for_device(int dev, void **ptr)
{
    *ptr = nullptr;
    if (dev < 0 || dev >= kMaxDevices) return fail(BCONV_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return BCONV_OK;
}

}  // namespace

extern "C" {

bconv_status_t bconv_validate_desc(const bconv_desc_t *desc, int32_t type, uint32_t flags)
{
    return check_desc(desc, type, flags);
}

bconv_status_t bconv_create(const bconv_desc_t *desc, const uint32_t *weight_bits,
                            const float *output_scale, const float *output_bias,
                            const float *input_scale, const float *input_bias, int32_t type,
                            uint32_t flags, bconv_t *out)
{
    if (!out) return fail(BCONV_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    bconv_status_t st = check_desc(desc, type, flags);
    if (st != BCONV_OK) return st;
    if (!weight_bits) return fail(BCONV_ERR_INVALID_ARGUMENT, "weight_bits is NULL");

    bconv_handle *h = new (std::nothrow) bconv_handle();
    if (!h) return fail(BCONV_ERR_ALLOC, "host allocation failed");
    h->desc = *desc;
    h->type = type;
    h->flags = flags;
    h->out_h = out_dim(desc->in_h, desc->kernel_h, desc->stride_h, desc->pad_h, desc->pad_h_end);
    h->out_w = out_dim(desc->in_w, desc->kernel_w, desc->stride_w, desc->pad_w, desc->pad_w_end);
    h->words = (desc->in_c + 31) / 32;
    h->tiles = (desc->out_c + bconv::kTile - 1) / bconv::kTile;
    const char *fg = getenv("BCONV_FORCE_GENERIC");
    h->force_generic = fg && fg[0] == '1';
    const char *sp = getenv("BCONV_STRIP_WIDTH");
    h->strip_width = sp ? atoi(sp) : 0;
    const char *sf = getenv("BCONV_SMALL_FUSED");
    h->small_fused = !(sf && sf[0] == '0');
    hipError_t e = hipGetDevice(&h->device);
    int cus = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) {
        release(h);
        return hip_fail(e, "hipGetDevice");
    }
    h->simds = 4 * cus;
    {
        // set-up of the scratch-free entry point on this device
        void *sp = nullptr;
        if ((st = scratch_for_device(h->device, &sp)) != BCONV_OK) {
            release(h);
            return st;
        }
    }

    const int taps = desc->kernel_h * desc->kernel_w;
    const size_t user_words = (size_t)desc->out_c * taps * h->words;
    uint32_t *d_user = nullptr;
    if ((st = upload(weight_bits, user_words, &d_user)) != BCONV_OK ||
        (st = upload(output_scale, (size_t)desc->out_c, &h->d_out_scale)) != BCONV_OK ||
        (st = upload(output_bias, (size_t)desc->out_c, &h->d_out_bias)) != BCONV_OK ||
        (st = upload(input_scale, (size_t)desc->in_c, &h->d_in_scale)) != BCONV_OK ||
        (st = upload(input_bias, (size_t)desc->in_c, &h->d_in_bias)) != BCONV_OK) {
        if (d_user) (void)hipFree(d_user);
        release(h);
        return st;
    }
    // An input affine is held as both arrays: a missing scale is 1, a missing bias 0.
    if ((h->d_in_scale == nullptr) != (h->d_in_bias == nullptr)) {
        const std::vector<float> identity((size_t)desc->in_c, h->d_in_scale ? 0.0f : 1.0f);
        st = upload(identity.data(), identity.size(), h->d_in_scale ? &h->d_in_bias : &h->d_in_scale);
        if (st != BCONV_OK) {
            (void)hipFree(d_user);
            release(h);
            return st;
        }
    }

    const bconv::Geom g = make_geom(h, 1);
    if ((flags & BCONV_FLAG_FP4_MFMA) && !bconv::f4_route(g)) {
        (void)hipFree(d_user);
        release(h);
        return fail(BCONV_ERR_UNSUPPORTED,
                    "BCONV_FLAG_FP4_MFMA needs a fully connected window of a multiple of 4 words, or a convolution "
                    "with ceil(in_c/32) a multiple of 4 and at most 4096 words per window");
    }
    if (type != BCONV_BINARY_WEIGHTS) {
        h->lane.kwc4 = (desc->kernel_w * h->words + 3) / 4;
        const size_t nw = (size_t)h->tiles * desc->kernel_h * h->lane.kwc4 * 256;
        const size_t np = (size_t)h->tiles * (desc->kernel_h + 1) * bconv::rect_row(desc->kernel_w) * 64;
        e = hipMalloc(reinterpret_cast<void **>(&h->d_lane_words), nw * 4);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&h->d_lane_popc), np * 4);
        if (e != hipSuccess) {
            (void)hipFree(d_user);
            release(h);
            return fail(BCONV_ERR_ALLOC, "hipMalloc: %s", hipGetErrorString(e));
        }
        h->lane.words = h->d_lane_words;
        h->lane.rect = h->d_lane_popc;
    } else {
        h->pm_cols = bconv::bwconv_pm_cols(desc->out_c);
        e = hipMalloc(reinterpret_cast<void **>(&h->d_pm), (size_t)taps * desc->in_c * h->pm_cols * 4);
        if (e == hipSuccess) e = hipMalloc(&h->d_mma, bconv::bwmma_frag_bytes(g));
        if (e != hipSuccess) {
            (void)hipFree(d_user);
            release(h);
            return fail(BCONV_ERR_ALLOC, "hipMalloc: %s", hipGetErrorString(e));
        }
    }
    e = bconv::launch_prepack(g, nullptr, d_user, h->d_lane_words, h->d_lane_popc, h->d_pm, h->pm_cols, type);
    if (e == hipSuccess && type == BCONV_BINARY_WEIGHTS) e = bconv::launch_prepack_bwmma(g, nullptr, d_user, h->d_mma);
    h->i8 = (flags & BCONV_FLAG_INT8_MFMA) != 0;
    if (e == hipSuccess && h->i8) {
        e = hipMalloc(&h->d_i8frag, bconv::i8_frag_bytes(g));
        if (e == hipSuccess) e = bconv::launch_prepack_i8(g, nullptr, d_user, h->d_i8frag, type == BCONV_AND);
    }
    h->gemm = type != BCONV_BINARY_WEIGHTS && bconv::gemm_route(g);
    if (e == hipSuccess && h->gemm) {
        e = hipMalloc(reinterpret_cast<void **>(&h->d_flat), bconv::gemm_weight_words(g) * 4);
        if (e == hipSuccess) e = bconv::launch_prepack_flat(g, nullptr, d_user, h->d_flat);
    }
    if (e == hipSuccess && (flags & BCONV_FLAG_FP4_MFMA)) {
        e = hipMalloc(&h->d_f4, bconv::f4_bytes(g));
        if (e == hipSuccess) e = bconv::launch_prepack_f4(g, nullptr, d_user, h->d_f4);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    (void)hipFree(d_user);
    if (e != hipSuccess) {
        release(h);
        return hip_fail(e, "weight prepack");
    }
    *out = h;
    return BCONV_OK;
}

bconv_status_t bconv_create_fc(int32_t in_h, int32_t in_w, int32_t in_c, int32_t out_c,
                               int32_t neuron, float scale_value, const uint32_t *weight_bits,
                               const float *output_scale, const float *output_bias,
                               const float *input_scale, const float *input_bias, int32_t type,
                               uint32_t flags, bconv_t *out)
{
    bconv_desc_t d{};
    d.in_h = in_h;
    d.in_w = in_w;
    d.in_c = in_c;
    d.out_c = out_c;
    d.kernel_h = in_h;
    d.kernel_w = in_w;
    d.stride_h = d.stride_w = 1;
    d.pad_h = d.pad_w = d.pad_h_end = d.pad_w_end = 0;
    d.groups = 1;
    d.neuron = neuron;
    d.scale_value = scale_value;
    return bconv_create(&d, weight_bits, output_scale, output_bias, input_scale, input_bias, type,
                        flags, out);
}

bconv_status_t bconv_get_info(bconv_t h, int32_t *in_c, int32_t *out_c, int32_t *out_h, int32_t *out_w)
{
    if (!h) return fail(BCONV_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (in_c) *in_c = h->desc.in_c;
    if (out_c) *out_c = h->desc.out_c;
    if (out_h) *out_h = h->out_h;
    if (out_w) *out_w = h->out_w;
    return BCONV_OK;
}

bconv_status_t bconv_workspace_size(bconv_t h, int32_t n, size_t *bytes)
{
    if (!h || !bytes) return fail(BCONV_ERR_INVALID_ARGUMENT, "handle or bytes is NULL");
    if (n < 0) return fail(BCONV_ERR_INVALID_ARGUMENT, "n must be >= 0");
    *bytes = layout_for(h, n).total_bytes;
    return BCONV_OK;
}

bconv_status_t bconv_workspace_layout(bconv_t h, int32_t n, bconv_workspace_layout_t *layout)
{
    if (!h || !layout) return fail(BCONV_ERR_INVALID_ARGUMENT, "handle or layout is NULL");
    if (n < 0) return fail(BCONV_ERR_INVALID_ARGUMENT, "n must be >= 0");
    *layout = layout_for(h, n);
    return BCONV_OK;
}

bconv_status_t bconv_forward(bconv_t h, void *stream, int32_t n, const float *in, float *out,
                             void *workspace, size_t workspace_bytes)
{
    return forward_impl(h, stream, n, in, Source::Values, out, Sink::Output, workspace, workspace_bytes, nullptr,
                        nullptr);
}

bconv_status_t bconv_forward_noalloc(bconv_t h, void *stream, int32_t n, const float *in, float *out)
{
    if (!h) return fail(BCONV_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (n < 0) return fail(BCONV_ERR_INVALID_ARGUMENT, "n must be >= 0");
    const size_t need = layout_for(h, n).total_bytes;
    if (need > (size_t)BCONV_SCRATCH_MAX_BYTES)
        return fail(BCONV_ERR_WORKSPACE, "batch %d needs %zu workspace bytes, beyond the %zu of the built-in scratch",
                    n, need, (size_t)BCONV_SCRATCH_MAX_BYTES);
    void *ptr = nullptr;
    {
        DeviceGuard guard(h->device);
        if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
        const bconv_status_t st = scratch_for_device(h->device, &ptr);
        if (st != BCONV_OK) return st;
    }
    // Every byte the kernels read from the workspace is written earlier in
    // the same call (the pack writes the halo and slack zeros, the convolution
    // writes beta), so nothing needs clearing between calls.
    return forward_impl(h, stream, n, in, Source::Values, out, Sink::Output, ptr, BCONV_SCRATCH_MAX_BYTES, nullptr,
                        nullptr);
}

bconv_status_t bconv_forward_accum(bconv_t h, void *stream, int32_t n, const float *in, void *acc,
                                   void *workspace, size_t workspace_bytes)
{
    return forward_impl(h, stream, n, in, Source::Values, acc, Sink::Accum, workspace, workspace_bytes, nullptr,
                        nullptr);
}

bconv_status_t bconv_forward_profiled(bconv_t h, void *stream, int32_t n, const float *in, float *out,
                                      void *workspace, size_t workspace_bytes, void *main_begin,
                                      void *main_end, void *input_begin, void *input_end)
{
    return forward_impl(h, stream, n, in, Source::Values, out, Sink::Output, workspace, workspace_bytes, main_begin,
                        main_end, input_begin, input_end);
}

bconv_status_t bconv_forward_bits(bconv_t h, void *stream, int32_t n, const float *in, uint32_t *out_bits,
                                  void *workspace, size_t workspace_bytes)
{
    return forward_impl(h, stream, n, in, Source::Values, out_bits, Sink::Bits, workspace, workspace_bytes,
                        nullptr, nullptr);
}

bconv_status_t bconv_forward_bits_profiled(bconv_t h, void *stream, int32_t n, const float *in,
                                           uint32_t *out_bits, void *workspace, size_t workspace_bytes,
                                           void *main_begin, void *main_end, void *input_begin, void *input_end)
{
    return forward_impl(h, stream, n, in, Source::Values, out_bits, Sink::Bits, workspace, workspace_bytes, main_begin,
                        main_end, input_begin, input_end);
}

bconv_status_t bconv_forward_packed(bconv_t h, void *stream, int32_t n, const uint32_t *in_bits, float *out,
                                    void *workspace, size_t workspace_bytes)
{
    return forward_impl(h, stream, n, in_bits, Source::Bits, out, Sink::Output, workspace, workspace_bytes, nullptr,
                        nullptr);
}

bconv_status_t bconv_forward_packed_bits(bconv_t h, void *stream, int32_t n, const uint32_t *in_bits,
                                         uint32_t *out_bits, void *workspace, size_t workspace_bytes)
{
    return forward_impl(h, stream, n, in_bits, Source::Bits, out_bits, Sink::Bits, workspace, workspace_bytes,
                        nullptr, nullptr);
}

bconv_status_t bconv_calibrate_popcount(void *stream, int32_t blocks, int32_t iters, uint32_t seed, uint32_t *sink)
{
    if (blocks < 1 || blocks > (1 << 22) || iters < 0)
        return fail(BCONV_ERR_INVALID_ARGUMENT, "blocks must be in [1, 2^22] and iters >= 0");
    if (!sink) return fail(BCONV_ERR_INVALID_ARGUMENT, "sink is NULL");
    const hipError_t e = bconv::launch_popc_peak(static_cast<hipStream_t>(stream), blocks, iters, seed, sink);
    if (e != hipSuccess) return hip_fail(e, "calibration kernel");
    return BCONV_OK;
}

const char *bconv_main_kernel(bconv_t h, int32_t n)
{
    if (!h || n < 0) return "";
    const bconv::Geom g = make_geom(h, n);
    if (h->i8) return bconv::i8mma_kernel_name();
    if (h->type == BCONV_BINARY_WEIGHTS)
        return h->force_generic ? bconv::bwconv_kernel_name(g) : bconv::bwmma_kernel_name(g, h->d_in_scale != nullptr);
    if (h->force_generic) return "xconv_generic";
    if (takes_small(h, g)) return bconv::small_kernel_name(g, h->type == BCONV_AND);
    if (h->d_f4) return bconv::f4_kernel_name(g, h->type == BCONV_AND);
    if (h->gemm) return bconv::gemm_kernel_name(g, h->type == BCONV_AND);
    return bconv::xconv_kernel_name(g);
}

bconv_status_t bconv_destroy(bconv_t h)
{
    if (!h) return BCONV_OK;
    DeviceGuard guard(h->device);
    release(h);
    return BCONV_OK;
}

const char *bconv_status_string(bconv_status_t s)
{
    switch (s) {
    case BCONV_OK: return "BCONV_OK";
    case BCONV_ERR_INVALID_ARGUMENT: return "BCONV_ERR_INVALID_ARGUMENT";
    case BCONV_ERR_UNSUPPORTED: return "BCONV_ERR_UNSUPPORTED";
    case BCONV_ERR_WORKSPACE: return "BCONV_ERR_WORKSPACE";
    case BCONV_ERR_ALLOC: return "BCONV_ERR_ALLOC";
    case BCONV_ERR_HIP: return "BCONV_ERR_HIP";
    }
    return "BCONV_ERR_UNKNOWN";
}

const char *bconv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
