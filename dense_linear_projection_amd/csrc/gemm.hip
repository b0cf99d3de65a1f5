// gemm.hip -- LDS-pipelined MFMA GEMM for many token rows (large M).
//
// With many token rows each weight is reused M times and the projection is
// bound by matrix-core throughput, so the kernel tiles the output and
// reuses every loaded operand across a whole tile (worklog "How I made
// Muse's GPU projections 1.32x faster in the Open Kernel Challenge", section
// "Tiling: load a small piece and use it more than once": a BM x BN tile
// does 2*BM*BN*BK flops per (BM+BN)*BK operands), stages the next K slice
// while the current one is multiplied (same page, section "How a pipeline
// hides waiting"), and lays LDS out so a wave's fragment reads hit distinct
// banks (same page, section "Shared memory has a layout problem too").
//
// Tile schedule: a workgroup of WM x WN wave64s computes a BM x BN output
// tile; each wave owns a (BM/WM) x (BN/WN) sub-tile held as 16x16 fp32
// MFMA accumulators (v_mfma_f32_16x16x32_bf16).  Both operands are K-major
// in memory (X[m, k], W[n, k]), so both are staged the same way:
//   * global -> LDS with global_load_lds_dwordx4 (no VGPR round trip), one
//     instruction moving 64 lanes x 16 bytes = 8 rows x 64 k of one operand;
//   * LDS row r holds 8 chunks of 8 k; chunk c is stored at position
//     c ^ (r & 7), so the 16 rows one MFMA fragment read touches fall on
//     distinct bank groups; the XOR is applied when choosing each lane's
//     global address, because the DMA writes lane i to position i;
//   * two LDS stages: stage k+1 is in flight while stage k is consumed.
// Workgroups are numbered so that those sharing an XCD (dispatch goes round
// robin over the 8 XCDs) get neighbouring tiles, grouped GM tile-rows at a
// time, so the operands they share stay in that XCD's L2.
//
// Epilogue (bias, GELU, output rounding) runs on the accumulators and writes
// Y once (page "blackroom" on Devpost, section "How we built it", the
// GEMM + GELU epilogue row).  Rows beyond M or N read a clamped valid row and
// are not stored.  The planner only picks this kernel when K % BK == 0 and X,
// W are 16-byte aligned.
#include "common.hpp"
#include "kernels.hpp"

namespace proj {

template <int BM, int BN, int BK, int WM, int WN, int GM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(Args a) {
    static_assert(BK == 64, "LDS swizzle assumes 128-byte rows");
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;   // wave sub-tile
    constexpr int FM = TM / 16, FN = TN / 16;   // 16x16 blocks per wave
    constexpr int ROWB = BK * 2;                // bytes per LDS row
    constexpr int STAGE = (BM + BN) * ROWB;     // bytes per stage
    constexpr int A_INSTR = BM / 8, B_INSTR = BN / 8;  // 1 KB DMA blocks
    static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0, "blocks per wave");

    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t M = a.M, N = a.N, K = a.K;

    // ---- tile id: XCD-contiguous renumbering, then grouped order
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t G = tiles_m * tiles_n;
    int64_t L = blockIdx.x;
    if (G % 8 == 0) L = (L % 8) * (G / 8) + L / 8;
    const int64_t per_group = GM * tiles_n;
    const int64_t group = L / per_group;
    const int64_t first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int64_t tm = first_m + (L % per_group) % gsz;
    const int64_t tn = (L % per_group) / gsz;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    // ---- per-lane DMA source rows for this wave's share of the blocks
    // block j covers rows 8j..8j+7; lane l fills row 8j + l/8, position l%8,
    // which holds chunk (l%8) ^ (l/8).
    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;
    const uint16_t *asrc[A_INSTR / NW];
    const uint16_t *bsrc[B_INSTR / NW];
#pragma unroll
    for (int j = 0; j < A_INSTR / NW; ++j) {
        int64_t row = m0 + (wave + j * NW) * 8 + drow;
        if (row >= M) row = M - 1;
        asrc[j] = a.X + row * K + dchunk * 8;
    }
#pragma unroll
    for (int j = 0; j < B_INSTR / NW; ++j) {
        int64_t row = n0 + (wave + j * NW) * 8 + drow;
        if (row >= N) row = N - 1;
        bsrc[j] = a.W + row * K + dchunk * 8;
    }

    auto issue = [&](int stage, int64_t kt) {
        char *sbase = lds + stage * STAGE;
#pragma unroll
        for (int j = 0; j < A_INSTR / NW; ++j)
            dma16(asrc[j] + kt * BK, sbase + (wave + j * NW) * 1024);
#pragma unroll
        for (int j = 0; j < B_INSTR / NW; ++j)
            dma16(bsrc[j] + kt * BK, sbase + BM * ROWB + (wave + j * NW) * 1024);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t KT = K / BK;
    const int fr = lane & 15, fg = lane >> 4;
    if (KT > 0) issue(0, 0);
    wait_vmem();
    __syncthreads();

    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        if (kt + 1 < KT) issue(cur ^ 1, kt + 1);
        const char *sa = lds + cur * STAGE;
        const char *sb = sa + BM * ROWB;
        // all fragments of the stage first, so the LDS reads of the second
        // k-step overlap the matrix ops of the first
        bf16x8 af[BK / 32][FM], bfr[BK / 32][FN];
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int c = ks * 4 + fg;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 16 + fr;
                af[ks][i] = *reinterpret_cast<const bf16x8 *>(sa + row * ROWB + ((c ^ (row & 7)) << 4));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 16 + fr;
                bfr[ks][j] = *reinterpret_cast<const bf16x8 *>(sb + row * ROWB + ((c ^ (row & 7)) << 4));
            }
        }
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[ks][i], bfr[ks][j], acc[i][j]);
        wait_vmem();
        __syncthreads();
    }

    // ---- epilogue: lane holds column lane%16, rows 4*(lane/16) + r
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 16 + fr;
        if (n >= N) continue;
        const float b = (a.epi & 1) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * TM + i * 16 + fg * 4 + r;
                if (m < M) store_out(a.Y, a.out, m * N + n, apply_epilogue(acc[i][j][r], a.epi, b));
            }
        }
    }
}

// Four-wave variant with an explicit in-wave software pipeline.  Each wave
// owns a 128 x (BN/2) sub-tile (8 x FN accumulators of 16x16, up to all 256
// AGPRs), so it is the only wave on its SIMD and must hide its own LDS
// latency.  A stage (BK = 64) is 2*8 groups of FN matrix ops, one group per
// A fragment row; the A fragment for group g is read PD groups earlier, the
// B fragments of the second k-step during the first, and the DMA copies of
// the next stage either all at the start of the stage (EARLY) or one per
// group.  Each group begins with an explicit wait that only covers reads
// issued at least one group ago, then issues its own reads, then its matrix
// ops; scheduling fences keep that order (the compiler would otherwise sink
// each read to just before its first use and wait on it there).
template <int FM, int FN, int PD, int G>
struct PipeReads {
    static constexpr int ks = G / FM, i = G % FM;
    static constexpr int a = (G + PD < 2 * FM) ? 1 : 0;              // A fragment for group G+PD
    static constexpr int b = (ks == 0 && i < FN) ? 1 : 0;            // B fragment of k-step 1
    static constexpr int n = a + b;
};

template <int FM, int FN, int PD, int G>
__device__ __forceinline__ void pipe_wait() {
    // reads issued in the previous group may still be in flight
    if constexpr (G == 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
    } else {
        constexpr int keep = PD > 1 ? PipeReads<FM, FN, PD, G - 1>::n : 0;
        __builtin_amdgcn_s_waitcnt(0xC07F | (keep << 8));  // lgkmcnt(keep)
    }
}

template <int BN, int GM, bool EARLY, int PD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_pipe_kernel(Args a) {
    constexpr int BM = 256, BK = 64, WN = 2, NW = 4;
    constexpr int TM = 128, TN = BN / 2;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int A_BLK = BM / 8, B_BLK = BN / 8;
    constexpr int A_PW = A_BLK / NW, B_PW = B_BLK / NW;  // DMA copies per wave per stage
    constexpr int NG = 2 * FM;                           // matrix-op groups per stage
    static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "copies divide over the waves");
    static_assert(A_PW + B_PW <= NG, "one copy per group at most");
    static_assert(FN <= FM, "B fragments of the next k-step fit one per group");
    static_assert(PD == 1 || PD == 2, "prefetch distance");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t M = a.M, N = a.N, K = a.K;

    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t G = tiles_m * tiles_n;
    int64_t L = blockIdx.x;
    if (G % 8 == 0) L = (L % 8) * (G / 8) + L / 8;
    const int64_t per_group = GM * tiles_n;
    const int64_t group = L / per_group;
    const int64_t first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int64_t tm = first_m + (L % per_group) % gsz;
    const int64_t tn = (L % per_group) / gsz;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;
    const uint16_t *src[A_PW + B_PW];
    int dst[A_PW + B_PW];
#pragma unroll
    for (int j = 0; j < A_PW; ++j) {
        int64_t row = m0 + (wave + j * NW) * 8 + drow;
        if (row >= M) row = M - 1;
        src[j] = a.X + row * K + dchunk * 8;
        dst[j] = (wave + j * NW) * 1024;
    }
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
        int64_t row = n0 + (wave + j * NW) * 8 + drow;
        if (row >= N) row = N - 1;
        src[A_PW + j] = a.W + row * K + dchunk * 8;
        dst[A_PW + j] = BM * ROWB + (wave + j * NW) * 1024;
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t KT = K / BK;
    const int fr = lane & 15, fg = lane >> 4;
    auto frag = [&](const char *base, int row, int ks) -> bf16x8 {
        const int c = ks * 4 + fg;
        return *reinterpret_cast<const bf16x8 *>(base + row * ROWB + ((c ^ (row & 7)) << 4));
    };

    if (KT > 0) {
#pragma unroll
        for (int j = 0; j < A_PW + B_PW; ++j) dma16(src[j], lds + dst[j]);
    }
    wait_vmem();
    __syncthreads();

    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const char *sa = lds + cur * STAGE;
        const char *sb = sa + BM * ROWB;
        char *nxt = lds + (cur ^ 1) * STAGE;
        // the last stage re-reads itself into the idle buffer: no branch
        const int64_t koff = (kt + 1 < KT ? kt + 1 : kt) * BK;

        if (EARLY) {
#pragma unroll
            for (int c = 0; c < A_PW + B_PW; ++c) dma16(src[c] + koff, nxt + dst[c]);
        }
        bf16x8 bf[2][FN], af[NG];
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[0][j] = frag(sb, wn * TN + j * 16 + fr, 0);
#pragma unroll
        for (int p = 0; p < PD; ++p) af[p] = frag(sa, wm * TM + (p % FM) * 16 + fr, p / FM);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int ks = g / FM, i = g % FM;
            if (g == 0) pipe_wait<FM, FN, PD, 0>();
            if (g == 1) pipe_wait<FM, FN, PD, 1>();
            if (g == 2) pipe_wait<FM, FN, PD, 2>();
            if (g == 3) pipe_wait<FM, FN, PD, 3>();
            if (g == 4) pipe_wait<FM, FN, PD, 4>();
            if (g == 5) pipe_wait<FM, FN, PD, 5>();
            if (g == 6) pipe_wait<FM, FN, PD, 6>();
            if (g == 7) pipe_wait<FM, FN, PD, 7>();
            if (g == 8) pipe_wait<FM, FN, PD, 8>();
            if (g == 9) pipe_wait<FM, FN, PD, 9>();
            if (g == 10) pipe_wait<FM, FN, PD, 10>();
            if (g == 11) pipe_wait<FM, FN, PD, 11>();
            if (g == 12) pipe_wait<FM, FN, PD, 12>();
            if (g == 13) pipe_wait<FM, FN, PD, 13>();
            if (g == 14) pipe_wait<FM, FN, PD, 14>();
            if (g == 15) pipe_wait<FM, FN, PD, 15>();
            if (g + PD < NG) {
                const int gp = g + PD;
                af[gp] = frag(sa, wm * TM + (gp % FM) * 16 + fr, gp / FM);
            }
            if (ks == 0 && i < FN) bf[1][i] = frag(sb, wn * TN + i * 16 + fr, 1);
            if (!EARLY && g < A_PW + B_PW) dma16(src[g] + koff, nxt + dst[g]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[g], bf[ks][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmem();
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 16 + fr;
        if (n >= N) continue;
        const float b = (a.epi & 1) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * TM + i * 16 + fg * 4 + r;
                if (m < M) store_out(a.Y, a.out, m * N + n, apply_epilogue(acc[i][j][r], a.epi, b));
            }
        }
    }
}

// One list drives both compilation passes (device: kernel instantiation,
// host: launch table).
#define PROJ_GEMM_VARIANTS(X)                                                                    \
    X(128, 128, 2, 2, 4) X(256, 128, 2, 2, 4) X(128, 256, 2, 2, 4) X(256, 256, 2, 2, 4)          \
    X(256, 192, 2, 2, 4) X(192, 256, 2, 2, 4) X(256, 256, 2, 4, 4) X(256, 256, 4, 2, 4)          \
    X(256, 128, 4, 2, 4) X(256, 256, 2, 2, 8) X(256, 256, 2, 2, 2)

#define PROJ_GEMM_INST(BM, BN, WM, WN, GM) template __global__ void gemm_kernel<BM, BN, 64, WM, WN, GM>(Args);
PROJ_GEMM_VARIANTS(PROJ_GEMM_INST)

#define PROJ_GEMM_PIPE_VARIANTS(X) X(256, 4, false, 1) X(256, 4, true, 1) X(256, 4, true, 2) X(256, 4, false, 2)
#define PROJ_GEMM_PIPE_INST(BN, GM, E, PD) template __global__ void gemm_pipe_kernel<BN, GM, E, PD>(Args);
PROJ_GEMM_PIPE_VARIANTS(PROJ_GEMM_PIPE_INST)

#ifndef __HIP_DEVICE_COMPILE__
template <int BM, int BN, int BK, int WM, int WN, int GM>
static hipError_t prepare_gemm() {
    constexpr int lds_bytes = 2 * (BM + BN) * BK * 2;
    auto fn = gemm_kernel<BM, BN, BK, WM, WN, GM>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               lds_bytes);
}

// prepare_gemm must have run once in the process (the library does it when a
// context is created), so launching is capture-safe.
template <int BM, int BN, int BK, int WM, int WN, int GM>
static hipError_t launch_gemm(const Args &a, hipStream_t st) {
    const int64_t G = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = 2 * (BM + BN) * BK * 2;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, GM>), dim3(static_cast<unsigned>(G)),
                       dim3(WM * WN * 64), lds_bytes, st, a);
    return hipGetLastError();
}

template <int BN, int GM, bool E, int PD>
static hipError_t prepare_gemm_pipe() {
    auto fn = gemm_pipe_kernel<BN, GM, E, PD>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               2 * (256 + BN) * 128);
}

template <int BN, int GM, bool E, int PD>
static hipError_t launch_gemm_pipe(const Args &a, hipStream_t st) {
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = 2 * (256 + BN) * 128;
    hipLaunchKernelGGL((gemm_pipe_kernel<BN, GM, E, PD>), dim3(static_cast<unsigned>(G)), dim3(256), lds_bytes, st, a);
    return hipGetLastError();
}

#define PROJ_GEMM_ENTRY(BM, BN, WM, WN, GM) \
    {"gemm", BM, BN, 64, WM, WN, GM, &launch_gemm<BM, BN, 64, WM, WN, GM>, &prepare_gemm<BM, BN, 64, WM, WN, GM>},
#define PROJ_GEMM_PIPE_ENTRY(BN, GM, E, PD)                                                                    \
    {E ? (PD == 2 ? "gemmpipe_e_p2" : "gemmpipe_e") : (PD == 2 ? "gemmpipe_p2" : "gemmpipe"), 256, BN, 64, 2, 2, GM, \
     &launch_gemm_pipe<BN, GM, E, PD>, &prepare_gemm_pipe<BN, GM, E, PD>},
const GemmVariant kGemmVariants[] = {PROJ_GEMM_VARIANTS(PROJ_GEMM_ENTRY) PROJ_GEMM_PIPE_VARIANTS(PROJ_GEMM_PIPE_ENTRY)};
const int kNumGemmVariants = sizeof(kGemmVariants) / sizeof(kGemmVariants[0]);
#endif

}  // namespace proj
