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
#include <atomic>
#include <utility>

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

// Four-wave GEMM on a 4-deep ring of BK = 32 stages.  Each wave owns a
// 128 x (BN/2) sub-tile (8 x FN accumulators of 16x16) and is the only wave
// on its SIMD, so it must hide its own latencies:
//   * a stage (256 rows of X and BN rows of W, 32 k each) is one k-step: 8
//     groups of FN matrix ops, one group per 16-row fragment of A;
//   * the A fragment for group g is read two groups ahead, and in the second
//     half of stage t the B fragments and first two A fragments of stage t+1
//     are read, so a stage starts with its operands already in registers;
//   * one barrier per stage, in its middle (before group 4): each wave first
//     waits for its own DMA copies of stage t+1 (vmcnt), the barrier then
//     makes stage t+1 visible to all waves and proves that stage t-1's slot
//     is no longer read, so the copies of stage t+3 go into that slot right
//     after it (two stages of lead for the DMA);
//   * rows of 64 bytes hold 16-byte chunks at position chunk ^ ((row >> 1) & 3):
//     a 16-byte LDS read is served eight lanes at a time over 128 bytes of
//     banks, and eight consecutive rows then cover all eight 16-byte bank
//     groups; the DMA writes lane i to position i, so the XOR picks each
//     lane's source.
// Scheduling fences keep each group's reads ahead of its matrix ops (the
// compiler would otherwise sink each read to just before its first use).
// Epilogue: bias, GELU and rounding to bf16 in registers, then the whole
// tile is staged through LDS (XOR-swizzled by row group) and written with
// 16-byte row-contiguous stores; partial tiles, fp32 output or an unaligned
// Y store element by element.
// Per-group counts of the ring pipeline: in the second half of a stage
// (groups MID..FM-1) the next stage's FN B fragments and the PERW DMA copies
// are spread evenly; every group also reads one A fragment.
template <int FM, int FN, int PERW, int MID>
struct RingPlan {
    static constexpr int H = FM - MID;
    static constexpr int NB = (FN + H - 1) / H;      // next-stage B fragments per group
    static constexpr int NC = (PERW + H - 1) / H;    // DMA copies per group
    static constexpr int b_lo(int g) { return g < MID ? 0 : ((g - MID) * NB < FN ? (g - MID) * NB : FN); }
    static constexpr int b_hi(int g) { return g < MID ? 0 : ((g - MID + 1) * NB < FN ? (g - MID + 1) * NB : FN); }
    static constexpr int c_lo(int g) { return g < MID ? 0 : ((g - MID) * NC < PERW ? (g - MID) * NC : PERW); }
    static constexpr int c_hi(int g) { return g < MID ? 0 : ((g - MID + 1) * NC < PERW ? (g - MID + 1) * NC : PERW); }
    // LDS reads issued in group g
    static constexpr int reads(int g) { return 1 + b_hi(g) - b_lo(g); }
    // before group g's own reads: every read but the previous group's has
    // landed (group 0 follows the previous stage's last group; MID follows a
    // full wait)
    static constexpr int keep(int g) { return g == MID ? 0 : reads(g == 0 ? FM - 1 : g - 1); }
};

// lgkmcnt wait for group g of the ring pipeline (g folds to a constant once
// the group loop is unrolled)
template <class P, int... Gs>
__device__ __forceinline__ void ring_wait(int g, std::integer_sequence<int, Gs...>) {
    ((g == Gs ? lds_wait_keep<P::keep(Gs)>() : void()), ...);
}

template <int BN, int GM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_ring_kernel(Args a) {
    constexpr int BM = 256, BK = 32, D = 4, WN = 2, NW = 4;
    constexpr int TM = 128, TN = BN / 2;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ROWB = BK * 2;                     // 64 bytes per row per stage
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int A_BLK = BM / 16, B_BLK = BN / 16;  // 1 KB DMA blocks (16 rows)
    constexpr int PERW = (A_BLK + B_BLK) / NW;       // DMA copies per wave per stage
    constexpr int MID = FM / 2;                      // group before which the barrier sits
    static_assert((A_BLK + B_BLK) % NW == 0, "copies divide over the waves");
    using P = RingPlan<FM, FN, PERW, MID>;
    static_assert(P::reads(FM - 1) <= 15 && P::reads(MID) <= 15, "lgkmcnt range");
    static_assert(D * STAGE <= 160 * 1024 && BM * BN * 2 <= D * STAGE, "LDS budget");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
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

    // DMA: block b (16 rows) of a stage is one 1 KB copy; lane l fills row
    // 16b + l/4, position l%4, which holds chunk (l%4) ^ ((l/8)%4).  The
    // first A_BLK/NW copies of each wave are X blocks, the rest W blocks.
    // Each operand is read through a buffer resource over the tile's valid
    // rows: rows past M or N read as zero, the per-lane offset is fixed for
    // the whole loop and the k offset is a scalar.
    const int drow = lane >> 2;
    const int dchunk = (lane & 3) ^ ((lane >> 3) & 3);
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(a.X + m0 * K, static_cast<uint32_t>(rows_a * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(a.W + n0 * K, static_cast<uint32_t>(rows_b * K * 2));
    constexpr int PA = A_BLK / NW;
    uint32_t voff[PERW];
#pragma unroll
    for (int j = 0; j < PERW; ++j) {
        const int r = (j < PA ? (wave + j * NW) : (wave + (j - PA) * NW)) * 16 + drow;
        voff[j] = static_cast<uint32_t>(r * K * 2 + dchunk * 16);
    }
    const int64_t KT = K / BK;
    auto copy = [&](int j, int64_t t) {
        // stages past the end re-read the last one into an idle slot
        const uint32_t soff = static_cast<uint32_t>((t < KT ? t : KT - 1) * (BK * 2));
        const int blk = j < PA ? wave + j * NW : A_BLK + wave + (j - PA) * NW;
        char *dst = lds + static_cast<int>(t % D) * STAGE + blk * 1024;
        dma16_buf(j < PA ? rsrc_a : rsrc_b, voff[j], soff, dst);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fg = lane >> 4;
    auto frag = [&](const char *base, int row) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(base + row * ROWB + ((fg ^ ((row >> 1) & 3)) << 4));
    };
    auto stage_a = [&](int64_t t) -> const char * { return lds + static_cast<int>(t % D) * STAGE; };

    if (KT > 0) {
        // stages 0..2 in flight; stage 0 (and 1) landed and visible
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 0);
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 1);
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 2);
        wait_vm<PERW>();
        __syncthreads();
    }

    // Two fragment sets alternate between even and odd stages, so the next
    // stage's fragments are prefetched into the idle set without copies.
    bf16x8 b0[FN], b1[FN], a0[FM + 2], a1[FM + 2];
    {
        const char *sa = stage_a(0), *sb = sa + BM * ROWB;
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = frag(sb, wn * TN + j * 16 + fr);
        a0[0] = frag(sa, wm * TM + fr);
        a0[1] = frag(sa, wm * TM + 16 + fr);
        lds_wait_all();
    }

    auto stage = [&](int64_t kt, bf16x8(&bc)[FN], bf16x8(&bn)[FN], bf16x8(&ac)[FM + 2], bf16x8(&an)[FM + 2]) {
        const char *sa = stage_a(kt), *sb = sa + BM * ROWB;
        const char *na = stage_a(kt + 1), *nb = na + BM * ROWB;
#pragma unroll
        for (int g = 0; g < FM; ++g) {
            if (g == MID) {
                // stage kt+1 landed for this wave (stage kt+2 may still fly),
                // then for all waves; stage kt-1's slot is free
                wait_vm<PERW>();
                lds_wait_all();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            // reads issued at least one group ago have landed (the previous
            // group's own reads may still fly)
            ring_wait<P>(g, std::make_integer_sequence<int, FM>{});
            if (g + 2 < FM)
                ac[g + 2] = frag(sa, wm * TM + (g + 2) * 16 + fr);
            else
                an[g + 2 - FM] = frag(na, wm * TM + (g + 2 - FM) * 16 + fr);
#pragma unroll
            for (int q = P::b_lo(g); q < P::b_hi(g); ++q) bn[q] = frag(nb, wn * TN + q * 16 + fr);
#pragma unroll
            for (int q = P::c_lo(g); q < P::c_hi(g); ++q) copy(q, kt + 3);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[g][j] = mfma16x16x32(ac[g], bc[j], acc[g][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // KT is even: the planner offers this kernel only for K % 64 == 0
    for (int64_t kt = 0; kt < KT; kt += 2) {
        stage(kt, b0, b1, a0, a1);
        stage(kt + 1, b1, b0, a1, a0);
    }
    wait_vm<0>();
    lds_wait_all();
    __syncthreads();

    // ---- epilogue
    const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (N % 8 == 0) && a.out == OUT_BF16 &&
                      (reinterpret_cast<uintptr_t>(a.Y) % 16 == 0);
    float bias[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 16 + fr;
        bias[j] = ((a.epi & 1) && n < N) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
    }
    if (full) {
        // The tile goes to LDS as bf16 [BM][BN] with 16-column chunks XOR'd by
        // the row's group of four ((row >> 2) & 3, which is this lane's fg for
        // every value it holds), so one write's four row groups hit different
        // banks; every address is then a per-lane base plus a constant.
        uint16_t *t16 = reinterpret_cast<uint16_t *>(lds);
        uint16_t *lbase = t16 + (wm * TM + fg * 4) * BN + fr;
        const int epi = a.epi;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            uint16_t *cb = lbase + ((wn * TN + j * 16) ^ (fg << 4));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    cb[(i * 16 + r) * BN] = f32_to_bf16_bits(apply_epilogue_fast(acc[i][j][r], epi, bias[j]));
        }
        __syncthreads();
        constexpr int CPR = BN / 8;  // 16-byte chunks per row
        if constexpr (256 % CPR == 0) {
            constexpr int RPP = 256 / CPR;  // rows per pass of the workgroup
            const int prow = tid / CPR, ch = tid % CPR;
            const uint16_t *lsrc = t16 + prow * BN;
            uint16_t *gdst = static_cast<uint16_t *>(a.Y) + (m0 + prow) * N + n0 + ch * 8;
#pragma unroll 8
            for (int p = 0; p < BM / RPP; ++p) {
                const int row = prow + p * RPP;
                const int pcol = (ch * 8) ^ (((row >> 2) & 3) << 4);
                const u32x4 v = *reinterpret_cast<const u32x4 *>(lsrc + p * RPP * BN + pcol);
                *reinterpret_cast<u32x4 *>(gdst + static_cast<int64_t>(p) * RPP * N) = v;
            }
        } else {
#pragma unroll 4
            for (int c = tid; c < BM * CPR; c += 256) {
                const int row = c / CPR, ch = c % CPR;
                const u32x4 v =
                    *reinterpret_cast<const u32x4 *>(t16 + row * BN + ((ch * 8) ^ (((row >> 2) & 3) << 4)));
                *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.Y) + (m0 + row) * N + n0 + ch * 8) = v;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * TN + j * 16 + fr;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm * TM + i * 16 + fg * 4 + r;
                    if (m < M) store_out(a.Y, a.out, m * N + n, apply_epilogue(acc[i][j][r], a.epi, bias[j]));
                }
        }
    }
}

// The same four-wave ring with 32x32x16 matrix ops: a wave's 128 x (BN/2)
// sub-tile is 4 x FN blocks of 32x32 (16 accumulators of 16 floats for
// BN = 256), and a BK = 32 stage is two k-halves.  Half the matrix-op
// instructions of the 16x16 form for the same work, and every group reads
// exactly one A and at most ceil(FN/4) B fragments:
//   * group g = 4h + i runs the FN matrix ops of A block i, k-half h;
//   * the A fragment of group g is read two groups ahead (the last two
//     groups read the next stage's first two);
//   * k-half 1 B fragments of the current stage are read in groups 0..3,
//     k-half 0 B fragments of the next stage in groups 4..7, so a stage
//     starts with its first operands in registers;
//   * barrier, DMA ring, LDS layout and swizzle as in the 16x16 ring.
// Epilogue: the tile is staged through LDS as bf16, 64-column halves XOR'd
// by bit 2 of the row so that the two half-waves' rows (4 apart) write
// different banks, then written with 16-byte row-contiguous stores.
template <int BN, int GM, int D, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_ring32_kernel(Args a) {
    constexpr int BM = 256, BK = 32, WN = 2, NW = 4;
    static_assert(D == 4 || D == 5, "ring depth");
    constexpr int TM = 128, TN = BN / 2;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int NG = 2 * FM;                       // groups per stage
    constexpr int MID = NG / 2;                      // group before which the barrier sits
    constexpr int ROWB = BK * 2;                     // 64 bytes per row per stage
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int A_BLK = BM / 16, B_BLK = BN / 16;  // 1 KB DMA blocks (16 rows)
    constexpr int PERW = (A_BLK + B_BLK) / NW;       // DMA copies per wave per stage
    constexpr int PA = A_BLK / NW;
    constexpr int NBG = (FN + MID - 1) / MID;        // B fragments read per group
    // DMA schedule.  D = 4: the copies of stage t+3 are issued in the second
    // half of stage t (after the barrier frees the slot of stage t-1).
    // D = 5: one copy per group -- the first PH copies of stage t+4 in the
    // second half of stage t, the rest of stage t+3 in the first half of
    // stage t; a slot is then refilled three stages before it is read.
    constexpr int PH = D == 4 ? PERW : (PERW + 1) / 2;
    constexpr int NC1 = (PH + MID - 1) / MID;               // per group, second half
    constexpr int NC2 = (PERW - PH + MID - 1) / MID;        // per group, first half (D = 5)
    constexpr int LEAD = D == 4 ? PERW : 2 * PERW;          // copies still in flight at the barrier
    static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "copies divide over the waves");
    static_assert(1 + NBG <= 15, "lgkmcnt range");
    static_assert(D * STAGE <= 160 * 1024 && BM * BN * 2 <= D * STAGE, "LDS budget");
    static_assert(LEAD + PH <= 63, "vmcnt range");
    static_assert(BN % 64 == 0, "epilogue swizzle works on 64-column halves");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t M = a.M, N = a.N, K = a.K;

    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t G = tiles_m * tiles_n;
    // Persistent form: the grid is at most one workgroup per CU and each
    // workgroup walks tiles blockIdx.x, + gridDim.x, ...  With a grid that is
    // a multiple of 8 those tiles stay on the workgroup's XCD, whose tile
    // range the renumbering below makes contiguous.
    for (int64_t tile = blockIdx.x; tile < G; tile += (PERSIST ? gridDim.x : G)) {
    int64_t L = tile;
    if (G % 8 == 0) L = (L % 8) * (G / 8) + L / 8;
    const int64_t per_group = GM * tiles_n;
    const int64_t group = L / per_group;
    const int64_t first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int64_t tm = first_m + (L % per_group) % gsz;
    const int64_t tn = (L % per_group) / gsz;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    // DMA (as in the 16x16 ring): lane l fills row 16b + l/4, position l%4,
    // which holds chunk (l%4) ^ ((l/8)%4); rows past M or N read as zero.
    const int drow = lane >> 2;
    const int dchunk = (lane & 3) ^ ((lane >> 3) & 3);
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(a.X + m0 * K, static_cast<uint32_t>(rows_a * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(a.W + n0 * K, static_cast<uint32_t>(rows_b * K * 2));
    uint32_t voff[PERW];
#pragma unroll
    for (int j = 0; j < PERW; ++j) {
        const int r = (j < PA ? (wave + j * NW) : (wave + (j - PA) * NW)) * 16 + drow;
        voff[j] = static_cast<uint32_t>(r * K * 2 + dchunk * 16);
    }
    const int KT = static_cast<int>(K / BK);  // K < 2^22 (planner limit)
    // stages past the end go through an empty resource: no memory traffic,
    // but the copy still counts for the vmcnt waits
    const __amdgpu_buffer_rsrc_t rsrc_none = buffer_rsrc(a.X, 0);
    // copy j of stage t into ring slot `slot` (= t % D, kept by the caller)
    auto copy = [&](int j, int t, int slot) {
        const uint32_t soff = static_cast<uint32_t>((t < KT ? t : KT - 1) * (BK * 2));
        const int blk = j < PA ? wave + j * NW : A_BLK + wave + (j - PA) * NW;
        dma16_buf(t < KT ? (j < PA ? rsrc_a : rsrc_b) : rsrc_none, voff[j], soff, lds + slot * STAGE + blk * 1024);
    };
    // slot of stage t + d given the slot of stage t
    auto slot_add = [](int slot, int d) { return slot + d >= D ? slot + d - D : slot + d; };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // fragment of 32 rows starting at row0 (a multiple of 32), k-half h:
    // lane l reads row row0 + l%32, chunk 2h + l/32
    const int fr = lane & 31, fq = lane >> 5;
    const int sw = (fr >> 1) & 3;
    auto frag = [&](const char *base, int row0, int h) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(base + (row0 + fr) * ROWB + (((2 * h + fq) ^ sw) << 4));
    };


    if (KT > 0) {
        // stages 0..2 (and the first part of stage 3 for D = 5) in flight;
        // stage 0 landed and visible
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 0, 0);
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 1, 1);
#pragma unroll
        for (int j = 0; j < PERW; ++j) copy(j, 2, 2);
        if constexpr (D == 5) {
#pragma unroll
            for (int j = 0; j < PH; ++j) copy(j, 3, 3);
            wait_vm<2 * PERW + PH>();
        } else {
            wait_vm<2 * PERW>();
        }
        __syncthreads();
    }

    // b0x: k-half 0 fragments of the current stage (x alternates between
    // stages), b1: k-half 1 of the current stage, a0x: A fragments by group
    // (entries NG, NG+1 are the next stage's groups 0 and 1)
    bf16x8 b0e[FN], b0o[FN], b1[FN], a0e[NG + 2], a0o[NG + 2];
    {
        const char *sa = lds, *sb = sa + BM * ROWB;
#pragma unroll
        for (int j = 0; j < FN; ++j) b0e[j] = frag(sb, wn * TN + j * 32, 0);
        a0e[0] = frag(sa, wm * TM, 0);
        a0e[1] = frag(sa, wm * TM + 32, 0);
        lds_wait_all();
    }

    auto stage = [&](int kt, int slot, bf16x8(&bc)[FN], bf16x8(&bn)[FN], bf16x8(&ac)[NG + 2],
                     bf16x8(&an)[NG + 2]) {
        const char *sa = lds + slot * STAGE, *sb = sa + BM * ROWB;
        const char *na = lds + slot_add(slot, 1) * STAGE, *nb = na + BM * ROWB;
        const int slot3 = slot_add(slot, 3), slot_last = slot_add(slot, D - 1);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int h = g / FM, i = g % FM;
            if (g == MID) {
                // stage kt+1 landed for this wave, then for all waves; the
                // slot of stage kt-1 is no longer read
                wait_vm<LEAD>();
                lds_wait_all();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            // every LDS read but the previous group's has landed
            if (g == MID)
                lds_wait_keep<0>();
            else
                lds_wait_keep<1 + NBG>();
            const int gn = g + 2;
            if (gn < NG)
                ac[gn] = frag(sa, wm * TM + (gn % FM) * 32, gn / FM);
            else
                an[gn - NG] = frag(na, wm * TM + (gn - NG) * 32, 0);
            const int q0 = (g % MID) * NBG;
#pragma unroll
            for (int q = q0; q < q0 + NBG && q < FN; ++q) {
                if (g < MID)
                    b1[q] = frag(sb, wn * TN + q * 32, 1);
                else
                    bn[q] = frag(nb, wn * TN + q * 32, 0);
            }
            if (g >= MID) {
                const int c0 = (g - MID) * NC1;
#pragma unroll
                for (int c = c0; c < c0 + NC1 && c < PH; ++c) copy(c, kt + D - 1, slot_last);
            } else if (D == 5) {
                const int c0 = PH + g * NC2;
#pragma unroll
                for (int c = c0; c < c0 + NC2 && c < PERW; ++c) copy(c, kt + 3, slot3);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(ac[g], h == 0 ? bc[j] : b1[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // KT is even: the planner offers this kernel only for K % 64 == 0
    for (int kt = 0, slot = 0; kt < KT; kt += 2) {
        stage(kt, slot, b0e, b0o, a0e, a0o);
        slot = slot_add(slot, 1);
        stage(kt + 1, slot, b0o, b0e, a0o, a0e);
        slot = slot_add(slot, 1);
    }
    wait_vm<0>();
    lds_wait_all();
    __syncthreads();

    // ---- epilogue
    const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (N % 8 == 0) && a.out == OUT_BF16 &&
                      (reinterpret_cast<uintptr_t>(a.Y) % 16 == 0);
    float bias[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 32 + fr;
        bias[j] = ((a.epi & 1) && n < N) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
    }
    if (full) {
        // bf16 tile [BM][BN] in LDS; a value of row r, column c sits at column
        // c ^ (32 * ((r >> 2) & 1)).  Row bit 2 is this lane's fq for every
        // value it holds, so the XOR is one per-lane constant.
        uint16_t *t16 = reinterpret_cast<uint16_t *>(lds);
        uint16_t *lbase = t16 + (wm * TM + 4 * fq) * BN;
        const int epi = a.epi;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            // the XOR applies to the whole column (j * 32 toggles bit 5)
            uint16_t *cb = lbase + ((wn * TN + j * 32 + fr) ^ (fq << 5));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    cb[(i * 32 + 8 * (v / 4) + (v % 4)) * BN] =
                        f32_to_bf16_bits(apply_epilogue_fast(acc[i][j][v], epi, bias[j]));
        }
        __syncthreads();
        constexpr int CPR = BN / 8;  // 16-byte chunks per row
        for (int c = tid; c < BM * CPR; c += 256) {
            const int row = c / CPR, ch = c % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(t16 + row * BN + ((ch * 8) ^ (((row >> 2) & 1) << 5)));
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.Y) + (m0 + row) * N + n0 + ch * 8) = v;
        }
    } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * TN + j * 32 + fr;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = m0 + wm * TM + i * 32 + 8 * (v / 4) + 4 * fq + (v % 4);
                    if (m < M) store_out(a.Y, a.out, m * N + n, apply_epilogue(acc[i][j][v], a.epi, bias[j]));
                }
        }
    }
    // the next tile's copies overwrite LDS that other waves may still read
    if (PERSIST) __syncthreads();
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

#define PROJ_GEMM_RING_VARIANTS(X) X(256, 4) X(256, 8) X(192, 4) X(128, 4)
#define PROJ_GEMM_RING_INST(BN, GM) template __global__ void gemm_ring_kernel<BN, GM>(Args);
PROJ_GEMM_RING_VARIANTS(PROJ_GEMM_RING_INST)

#define PROJ_GEMM_RING32_VARIANTS(X) \
    X(256, 4, 4, false) X(256, 4, 5, false) X(192, 4, 5, false) X(256, 4, 5, true) X(192, 4, 5, true) X(128, 4, 5, true)
#define PROJ_GEMM_RING32_INST(BN, GM, D, P) template __global__ void gemm_ring32_kernel<BN, GM, D, P>(Args);
PROJ_GEMM_RING32_VARIANTS(PROJ_GEMM_RING32_INST)

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

// The ring kernel addresses a 256-row tile through 32-bit buffer offsets.
constexpr int64_t kRingMaxK = (int64_t{1} << 31) / (256 * 2);

template <int BN, int GM>
static hipError_t prepare_gemm_ring() {
    auto fn = gemm_ring_kernel<BN, GM>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               4 * (256 + BN) * 64);
}

template <int BN, int GM>
static hipError_t launch_gemm_ring(const Args &a, hipStream_t st) {
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = 4 * (256 + BN) * 64;
    hipLaunchKernelGGL((gemm_ring_kernel<BN, GM>), dim3(static_cast<unsigned>(G)), dim3(256), lds_bytes, st, a);
    return hipGetLastError();
}

// Number of CUs of the current device (all devices a process drives here are
// the same part), read once.
static int device_cus() {
    static std::atomic<int> cus{0};
    int n = cus.load(std::memory_order_relaxed);
    if (n == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus.store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int BN, int GM, int D, bool P>
static hipError_t prepare_gemm_ring32() {
    device_cus();
    auto fn = gemm_ring32_kernel<BN, GM, D, P>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               D * (256 + BN) * 64);
}

template <int BN, int GM, int D, bool P>
static hipError_t launch_gemm_ring32(const Args &a, hipStream_t st) {
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t grid = P ? (G < device_cus() ? G : device_cus()) : G;
    constexpr int lds_bytes = D * (256 + BN) * 64;
    hipLaunchKernelGGL((gemm_ring32_kernel<BN, GM, D, P>), dim3(static_cast<unsigned>(grid)), dim3(256), lds_bytes, st,
                       a);
    return hipGetLastError();
}

#define PROJ_GEMM_ENTRY(BM, BN, WM, WN, GM) \
    {"gemm", BM, BN, 64, 64, WM, WN, GM, 0, &launch_gemm<BM, BN, 64, WM, WN, GM>, &prepare_gemm<BM, BN, 64, WM, WN, GM>},
#define PROJ_GEMM_PIPE_ENTRY(BN, GM, E, PD)                                                                    \
    {E ? (PD == 2 ? "gemmpipe_e_p2" : "gemmpipe_e") : (PD == 2 ? "gemmpipe_p2" : "gemmpipe"), 256, BN, 64, 64, 2, 2, GM, 0, \
     &launch_gemm_pipe<BN, GM, E, PD>, &prepare_gemm_pipe<BN, GM, E, PD>},
#define PROJ_GEMM_RING_ENTRY(BN, GM) \
    {"gemmring", 256, BN, 32, 64, 2, 2, GM, kRingMaxK, &launch_gemm_ring<BN, GM>, &prepare_gemm_ring<BN, GM>},
#define PROJ_GEMM_RING32_ENTRY(BN, GM, D, P)                                                         \
    {P ? "gemmring32p" : (D == 5 ? "gemmring32d5" : "gemmring32"), 256, BN, 32, 64, 2, 2, GM, kRingMaxK, \
     &launch_gemm_ring32<BN, GM, D, P>, &prepare_gemm_ring32<BN, GM, D, P>},
const GemmVariant kGemmVariants[] = {PROJ_GEMM_VARIANTS(PROJ_GEMM_ENTRY) PROJ_GEMM_PIPE_VARIANTS(PROJ_GEMM_PIPE_ENTRY)
                                         PROJ_GEMM_RING_VARIANTS(PROJ_GEMM_RING_ENTRY)
                                             PROJ_GEMM_RING32_VARIANTS(PROJ_GEMM_RING32_ENTRY)};
const int kNumGemmVariants = sizeof(kGemmVariants) / sizeof(kGemmVariants[0]);
#endif

}  // namespace proj
