// common.hpp -- shared device types and the fused epilogue for libproj
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace proj {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

enum Epi { EPI_NONE = 0, EPI_BIAS = 1, EPI_GELU = 2, EPI_BIAS_GELU = 3 };
enum Out { OUT_F32 = 0, OUT_BF16 = 1 };

// Everything a kernel needs to know about one call.  The fields a kernel
// reads before its first copy come first, so that they share the first
// 64 bytes of the argument block (one scalar load at kernel entry); the
// output side follows.
struct Args {
    const uint16_t *X;     // bf16 [M, K]
    const uint16_t *W;     // bf16 [N, K]
    int64_t M, N, K;
    int64_t kx;            // X row length: K, or K/2 for a hi/lo weight pair (X column k' reads k' mod kx)
    int epi, out;
    int16_t wpack = 0;     // 0: W row-major [N][K]; t > 0: W packed in tiles of 16t rows (see proj_pack_weights)
    int16_t walk = 0;      // streaming kernel: tile t starts its K walk at stage (walk x t) mod T (0: stride 7)
    int atomic = 0;        // split K (S > 1), fp32 Y: partials are added into Y (zeroed first) with fp32 atomics
    const uint16_t *bias;  // bf16 [N] or nullptr
    void *Y;               // fp32 / bf16 [M, N]
    float *ws;             // split-K partials [S][M][N] (library-owned)
    const uint16_t *zeros; // >= 64 zero bytes in device memory, for masked loads
};
static_assert(offsetof(Args, atomic) + sizeof(int) == 64, "the prologue's fields fill the first 64 bytes");

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// GELU, tanh form: 0.5 v (1 + tanh(u)) with u = sqrt(2/pi) (v + 0.044715 v^3),
// evaluated as v / (1 + exp(-2u)) -- the same function, one exponential.
// The exponential overflows to +inf for very negative v, giving -0; it goes to
// 0 for large v, giving v.  NaN propagates.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float c2 = 2.0f * 0.7978845608028654f;  // 2 * sqrt(2/pi)
    float u2 = c2 * (v + 0.044715f * v * v * v);
    return v / (1.0f + __expf(-u2));
}

// The same GELU for the large-M epilogues, where the per-element cost
// matters: the exponent -2u log2(e) = v (A + B v^2) with the constants
// folded, the hardware base-2 exponential, and a hardware reciprocal (about
// 1 ulp) in place of the IEEE division.  The result differs from gelu_tanh
// by a few fp32 ulps; the limits (v for large v, -0 for very negative v) and
// NaN propagation are the same.
__device__ __forceinline__ float gelu_tanh_fast(float v) {
    const float A = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
    const float B = A * 0.044715f;
    const float z = v * __builtin_fmaf(v * v, B, A);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// bias (fp32-widened bf16) is added to the finished fp32 sum, then GELU.
__device__ __forceinline__ float apply_epilogue(float acc, int epi, float bias) {
    float v = acc;
    if (epi & 1) v += bias;
    if (epi & 2) v = gelu_tanh(v);
    return v;
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950;
// NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    __bf16 h = static_cast<__bf16>(v);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ void store_out(void *Y, int out, int64_t idx, float v) {
    if (out == OUT_F32)
        static_cast<float *>(Y)[idx] = v;
    else
        static_cast<uint16_t *>(Y)[idx] = f32_to_bf16_bits(v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 matrix op.  Lane l supplies row (A) / column (B) l % 32 and
// k elements 8 (l / 32) .. +7; element v of the result is row
// 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load16(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// 16-byte global -> LDS copy without a register round trip
// (global_load_lds_dwordx4): lane i of the wave writes lds_wave_base + 16*i.
// lds_wave_base must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// The same copy with the non-temporal (streaming) cache hint: for data read
// exactly once, so that it does not push reused data out of L2.
__device__ __forceinline__ void dma16_nt(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 2);
}

// Raw buffer resource over [base, base + bytes): loads at offsets at or past
// `bytes` return zero instead of touching memory.  Word 3 is the gfx9 raw
// (untyped, unswizzled) buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane i reads
// rsrc + voff + soff and writes lds_wave_base + 16*i.  soff and lds_wave_base
// are wave-uniform, so a loop that only moves soff needs no vector arithmetic.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16,
                                             voff, soff, 0, 0);
}

// The same copy with the non-temporal (streaming) cache hint.
__device__ __forceinline__ void dma16_buf_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                             void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16,
                                             voff, soff, 0, 2);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima), emitted as a
// real waitcnt instruction so the compiler's own wait insertion sees it.
__device__ __forceinline__ void lds_wait_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt lgkmcnt(N): all but the N most recent LDS operations are done.
template <int N>
__device__ __forceinline__ void lds_wait_keep() {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// s_waitcnt vmcnt(N): all but the N most recent vector memory operations are done.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ bf16x8 load16_nt(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
}

}  // namespace proj
