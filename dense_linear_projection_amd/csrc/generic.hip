// generic.hip -- any-shape, any-alignment projection kernel.
//
// One thread per output cell: the weighted sum over k of X[m, k] * W[n, k]
// in fp32 (worklog "How I made Muse's GPU projections 1.32x faster in the
// Open Kernel Challenge", section "The full equation, now with the letters
// explained"), then the epilogue.  Loads are 2-byte scalar reads, so any
// pointer alignment and any K work.  It is the fallback for inputs the
// vector kernels cannot take (K % 8 != 0 or X/W not 16-byte aligned), not a
// fast path.
#include "common.hpp"
#include "kernels.hpp"

namespace proj {

__global__ __launch_bounds__(256) void generic_kernel(Args a) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= a.M * a.N) return;
    const int64_t m = idx / a.N, n = idx % a.N;
    const uint16_t *x = a.X + m * a.K;
    const uint16_t *w = a.W + n * a.K;
    float s = 0.f;
    for (int64_t k = 0; k < a.K; ++k) s = __builtin_fmaf(bf16_bits_to_f32(x[k]), bf16_bits_to_f32(w[k]), s);
    const float b = (a.epi & 1) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
    store_out(a.Y, a.out, idx, apply_epilogue(s, a.epi, b));
}

#ifndef __HIP_DEVICE_COMPILE__
hipError_t launch_generic(const Args &a, hipStream_t st) {
    const int64_t cells = a.M * a.N;
    const int64_t blocks = (cells + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(generic_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
    return hipGetLastError();
}
#endif

}  // namespace proj
