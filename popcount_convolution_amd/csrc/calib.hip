// Calibration of the popcount path's own instruction pair on this chip: the
// sustained rate of v_xor_b32 + v_bcnt_u32_b32 (two VALU instructions per
// 32-bit word pair, the count accumulating in the second) with register
// operands, no memory traffic in the loop.  Timing it gives the measured VALU
// popcount peak that the convolution and GEMM kernels are compared with, beside
// the published-clock figure.
#include "internal.h"

namespace bconv {
namespace {

constexpr int kChains = 8;  // independent accumulators per lane

__global__ __launch_bounds__(256) void popc_peak_kernel(uint32_t seed, int iters, uint32_t *sink)
{
    const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
    // scalar (wave-uniform) words, as the convolution's input words are
    const uint32_t x0 = seed * 0x9E3779B1u, x1 = x0 ^ 0x85EBCA77u, x2 = x0 + 0xC2B2AE3Du, x3 = x0 ^ 0x27D4EB2Fu;
    uint32_t w[kChains], acc[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        w[k] = (tid * 2654435761u) ^ ((uint32_t)k * 0x9E3779B9u);
        acc[k] = 0;
    }
    for (int i = 0; i < iters; ++i) {
        uint32_t t0, t1, t2, t3, t4, t5, t6, t7;
        // chain k: t = x[k % 4] ^ w[k]; acc[k] += popcount(t)
        asm volatile(
            "v_xor_b32 %0, %16, %20\n\t"
            "v_xor_b32 %1, %17, %21\n\t"
            "v_xor_b32 %2, %18, %22\n\t"
            "v_xor_b32 %3, %19, %23\n\t"
            "v_xor_b32 %4, %16, %24\n\t"
            "v_xor_b32 %5, %17, %25\n\t"
            "v_xor_b32 %6, %18, %26\n\t"
            "v_xor_b32 %7, %19, %27\n\t"
            "v_bcnt_u32_b32 %8, %0, %8\n\t"
            "v_bcnt_u32_b32 %9, %1, %9\n\t"
            "v_bcnt_u32_b32 %10, %2, %10\n\t"
            "v_bcnt_u32_b32 %11, %3, %11\n\t"
            "v_bcnt_u32_b32 %12, %4, %12\n\t"
            "v_bcnt_u32_b32 %13, %5, %13\n\t"
            "v_bcnt_u32_b32 %14, %6, %14\n\t"
            "v_bcnt_u32_b32 %15, %7, %15"
            : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7),
              "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
              "+v"(acc[7])
            : "s"(x0), "s"(x1), "s"(x2), "s"(x3), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]),
              "v"(w[6]), "v"(w[7]));
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += acc[k];
    sink[tid] = s;
}

}  // namespace

hipError_t launch_popc_peak(hipStream_t stream, int blocks, int iters, uint32_t seed, uint32_t *sink)
{
    hipLaunchKernelGGL(popc_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, seed, iters, sink);
    return hipGetLastError();
}

}  // namespace bconv
