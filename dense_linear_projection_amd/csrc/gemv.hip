// gemv.hip -- projection for at most 8 token rows, with W read straight into
// registers.
//
// At one token the projection is a matrix-vector product: every weight is
// used once, and the whole cost is reading W (worklog "How I made Muse's GPU
// projections 1.32x faster in the Open Kernel Challenge", section "A rough
// way to ask how much room was left"; its one-token vector path in "The
// change that finally took me over 1.30x": a block owns a few output rows and
// the weight stream and the reused input vector are treated differently in
// cache). Two things decide the time at these sizes:
// how many workgroups share the weight rows, and how many bytes each CU
// keeps in flight.  A 16-row MFMA tile answers neither well for narrow
// outputs (N = 2304 has 144 such tiles for 256 CUs), and an LDS ring caps
// the bytes in flight at what fits in LDS.  Here:
//   * a workgroup owns R output features (W rows) and one of S contiguous
//     ranges of K, cut at 8-element (16-byte) chunks; with S > 1 it writes an
//     fp32 partial and the split-K pass adds the partials and applies the
//     epilogue;
//   * lane t of the workgroup takes chunks t, t + T, t + 2T, ... of its range
//     (T threads), U of them per iteration for each of the R rows: every
//     load is one 16-byte buffer load straight into registers, the R*U loads
//     of an iteration are independent, and nothing passes through LDS, so
//     several workgroups share a CU and all of their loads are in flight;
//   * the matching 16-byte chunks of the M <= MR token rows are loaded once
//     per iteration and reused for all R rows;
//   * products accumulate in fp32 with v_dot2_f32_bf16 (two bf16 products
//     and an fp32 add per instruction);
//   * W loads carry the non-temporal hint (W is read once);
//   * chunks past the range, rows past N and token rows past M read zero
//     through the buffer resources' bounds.
// After the loop each lane holds MR*R partial sums.  They are summed over the
// wave by halving exchanges (each step a lane keeps half of its values and
// adds its partner's copy of that half, so 64 values need 63 exchanges),
// then over the waves through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace proj {

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

// offset past every resource used here: a load there returns zero
constexpr uint32_t kOutside = 0x80000000u;

// 16-byte buffer load into registers; AUX 2 is the non-temporal hint
template <int AUX>
__device__ __forceinline__ u32x4_v load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
}

// acc + <w, x> over 8 bf16 pairs
__device__ __forceinline__ float dot8(u32x4_v w, u32x4_v x, float acc) {
    const bf16x8_v wb = __builtin_bit_cast(bf16x8_v, w), xb = __builtin_bit_cast(bf16x8_v, x);
    acc = __builtin_amdgcn_fdot2_f32_bf16(wb.s01, xb.s01, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(wb.s23, xb.s23, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(wb.s45, xb.s45, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(wb.s67, xb.s67, acc, false);
    return acc;
}

// One halving exchange per step, N values left of the wave's V: partners
// are lanes 32*N/V apart; a lane keeps the upper or lower half of its values
// (by that lane bit) and adds the partner's copy of the same half.
template <int N, int V>
__device__ __forceinline__ void halve_values(float (&v)[V], int lane) {
    if constexpr (N > 1) {
        constexpr int half = N / 2, h = 32 * N / V;
        const bool upper = (lane & h) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? v[i] : v[i + half];
            const float keep = upper ? v[i + half] : v[i];
            v[i] = keep + __shfl_xor(send, h, 64);
        }
        halve_values<half, V>(v, lane);
    }
}

// Sum V = 2^LV values over the 64 lanes of a wave.  Returns, in lane l, the
// total of value number l >> (6 - LV).
template <int V>
__device__ __forceinline__ float wave_sum_values(float (&v)[V], int lane) {
    constexpr int LV = __builtin_ctz(V);
    static_assert((1 << LV) == V && V <= 64, "a power of two, at most 64 values");
    halve_values<V, V>(v, lane);
    float x = v[0];
#pragma unroll
    for (int h = 32 / V; h >= 1; h >>= 1) x += __shfl_xor(x, h, 64);
    return x;
}

template <int MR, int R, int WAVES, int U, int WNT>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(Args a, int S) {
    constexpr int T = WAVES * 64, V = MR * R;
    __shared__ float red[WAVES * V];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 32-bit arithmetic and no division at all for S = 1: this runs before
    // the first load is issued (the launcher keeps the chunk count times S
    // below 2^32 for S > 1)
    const uint32_t us = static_cast<uint32_t>(S);
    uint32_t tile_u = blockIdx.x, split_u = 0;
    if (us > 1) {
        tile_u = blockIdx.x / us;
        split_u = blockIdx.x - tile_u * us;
    }
    const int split = static_cast<int>(split_u);
    const int64_t N = a.N, K = a.K, M = a.M;
    const int64_t n0 = static_cast<int64_t>(tile_u) * R;
    const int64_t rows_w = (N - n0) < R ? (N - n0) : R;

    // chunk range of this split
    const int64_t C = K / 8;
    int64_t cb = 0, ce = C;
    if (us > 1) {
        const uint32_t c32 = static_cast<uint32_t>(C);
        cb = (c32 * split_u) / us;
        ce = (c32 * (split_u + 1)) / us;
    }

    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.W + n0 * K, static_cast<uint32_t>(rows_w * K * 2));
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.X, static_cast<uint32_t>(M * a.kx * 2));
    const int64_t cx = a.kx / 8;  // chunks per X row (X columns wrap at kx)

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    for (int64_t base = cb; base < ce; base += static_cast<int64_t>(T) * U) {
        u32x4_v w[U][R], x[U][MR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = base + tid + static_cast<int64_t>(u) * T;
            const bool live = c < ce;
            const int64_t cxw = c < cx ? c : c - cx;
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[u][r] = load_b128<WNT ? 2 : 0>(rw, live ? static_cast<uint32_t>((r * K + c * 8) * 2) : kOutside);
#pragma unroll
            for (int m = 0; m < MR; ++m)
                x[u][m] = load_b128<0>(rx, live ? static_cast<uint32_t>((m * a.kx + cxw * 8) * 2) : kOutside);
        }
        // keep every load of the iteration ahead of the first product, so all
        // of them are in flight together
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m * R + r] = dot8(w[u][r], x[u][m], acc[m * R + r]);
    }

    const float s = wave_sum_values<V>(acc, lane);
    constexpr int LV = __builtin_ctz(V);
    if ((lane & ((64 >> LV) - 1)) == 0) red[wave * V + (lane >> (6 - LV))] = s;
    __syncthreads();
    if (tid < V) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) t += red[w * V + tid];
        const int m = tid / R, r = tid % R;
        const int64_t n = n0 + r;
        if (m < M && n < N) {
            if (S == 1) {
                const float b = (a.epi & 1) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
                store_out(a.Y, a.out, m * N + n, apply_epilogue(t, a.epi, b));
            } else {
                a.ws[(static_cast<int64_t>(split) * M + m) * N + n] = t;
            }
        }
    }
}

// ---------------------------------------------------------------- registry
// (MR token rows, R features per workgroup, waves, chunks per row per
// iteration, non-temporal W)
#define PROJ_GEMV_VARIANTS(X)                                                                   \
    X(1, 2, 4, 4, 1) X(1, 4, 4, 4, 1) X(1, 4, 4, 2, 1) X(1, 8, 4, 2, 1) X(1, 16, 4, 1, 1)        \
    X(1, 8, 8, 1, 1) X(1, 4, 8, 2, 1) X(1, 1, 4, 8, 1) X(1, 2, 4, 8, 1) X(1, 2, 8, 2, 1)          \
    X(1, 2, 4, 4, 0)                                                                            \
    X(2, 4, 4, 2, 1) X(2, 8, 4, 2, 1) X(2, 4, 4, 4, 1) X(2, 2, 4, 4, 1)                          \
    X(4, 4, 4, 2, 1) X(4, 8, 4, 2, 1) X(4, 8, 4, 1, 1) X(4, 2, 4, 2, 1)                          \
    X(8, 4, 4, 2, 1) X(8, 8, 4, 1, 1) X(8, 8, 4, 2, 1) X(8, 2, 4, 2, 1)

#define PROJ_GEMV_INST(MR, R, WV, U, WNT) template __global__ void gemv_kernel<MR, R, WV, U, WNT>(Args, int);
PROJ_GEMV_VARIANTS(PROJ_GEMV_INST)

#ifndef __HIP_DEVICE_COMPILE__
template <int MR, int R, int WV, int U, int WNT>
static hipError_t launch_gemv(const Args &a, int S, hipStream_t st) {
    // whole 16-byte chunks, X rows within the variant, offsets within the
    // resources' 31-bit range
    if (a.K % 8 != 0 || a.kx % 8 != 0 || a.M > MR || S < 1 || a.wpack) return hipErrorInvalidValue;
    if (static_cast<int64_t>(R) * a.K * 2 > 0x7fffffff || a.M * a.kx * 2 > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t grid = ((a.N + R - 1) / R) * S;
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    // the kernel cuts the chunk range of a split in 32-bit arithmetic
    if (S > 1 && (a.K / 8) * S >= (int64_t{1} << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemv_kernel<MR, R, WV, U, WNT>), dim3(static_cast<unsigned>(grid)), dim3(WV * 64), 0, st, a,
                       S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_splitk_reduce(a, S, st);
}

#define PROJ_GEMV_ENTRY(MR, R, WV, U, WNT) {"gemv", MR, R, WV, U, WNT, &launch_gemv<MR, R, WV, U, WNT>},
const GemvVariant kGemvVariants[] = {PROJ_GEMV_VARIANTS(PROJ_GEMV_ENTRY)};
const int kNumGemvVariants = sizeof(kGemvVariants) / sizeof(kGemvVariants[0]);
#endif

}  // namespace proj
