// gemm.hip -- LDS-pipelined MFMA GEMM for many token rows (large M).
//
// With many token rows each weight is reused M times and the projection is
// bound by matrix-core throughput, so the kernels tile the output and reuse
// every loaded operand across a whole tile (worklog "How I made Muse's GPU
// projections 1.32x faster in the Open Kernel Challenge", section "Tiling:
// load a small piece and use it more than once": a BM x BN tile does
// 2*BM*BN*BK flops per (BM+BN)*BK operands), stage the next K slices while
// the current one is multiplied (same page, section "How a pipeline hides
// waiting"), and lay LDS out so a wave's fragment reads hit distinct banks
// (same page, section "Shared memory has a layout problem too").
//
// Four kernel families, all candidates of the measured planner:
//   * gemm_kernel: WM x WN waves, 16x16x32 matrix ops, two LDS stages of
//     BK = 64 (any tile from 128 x 128 up);
//   * gemm_pp_kernel: eight waves in two groups that alternate between a
//     phase of matrix ops and a phase of LDS reads and DMA ("ping-pong"),
//     32x32x16 matrix ops on 64-byte LDS rows (K a multiple of 32);
//   * gemm_pp64_kernel: the same with 128-byte LDS rows (k copied 64 at a
//     time) in a ring of operand halves (K a multiple of 64);
//   * gemm_pp64p_kernel: its persistent form, one workgroup per CU walking
//     tiles with the ring running on across them, on 16x16x32 matrix ops.
// Both operands are K-major in memory (X[m, k], W[n, k]) and are staged the
// same way: global -> LDS copies without a register round trip (one
// instruction moves 64 lanes x 16 bytes), with 16-byte chunks XOR-swizzled by
// row so a fragment read hits distinct banks; the XOR is applied when choosing
// each lane's global address, because the copy writes lane i to position i.
// Workgroups are numbered so that those sharing an XCD (dispatch goes round
// robin over the 8 XCDs) get neighbouring tiles, grouped GM tile-rows at a
// time, so the operands they share stay in that XCD's L2.
//
// Epilogue (bias, GELU, output rounding) runs on the accumulators and writes
// Y once (page "blackroom" on Devpost, section "How we built it", the
// GEMM + GELU epilogue row).  Rows beyond M or N are read as a clamped valid
// row (gemm_kernel) or as zeros (buffer resources of the other two) and are
// not stored.  The planner only picks a kernel when K is a multiple of its
// stage depth and X, W are 16-byte aligned.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace proj {

// Chunk position on 128-byte LDS rows.  A 16-byte LDS read is served 16
// lanes at a time over a 256-byte window of banks (the model that fits the
// conflict counts measured on 64-byte rows), and a fragment read gives 16
// consecutive lanes 16 consecutive rows at one chunk.  A row's chunk lands
// at byte (row & 1) * 128 + 16 * position of that window, so the 8 rows of
// each parity need 8 distinct positions: the XOR takes row bits 1..3.
// chunk ^ (row & 7) gives rows r and r + 8 the same bytes (2-way conflicts
// in SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }

// Origin of the L-th tile of a BM x BN tiling walked in groups of GM tile
// rows (tiles_m x tiles_n tiles), so the workgroups that run together share
// operand blocks.  32-bit arithmetic (the launchers keep the tile count
// below 2^31) with one division by a runtime value: this runs before a
// workgroup's first copy, and a 64-bit division by a runtime value is a
// sequence of over a hundred scalar instructions.
template <int BM, int BN, int GM>
__device__ __forceinline__ void group_origin(uint32_t tiles_m, uint32_t tiles_n, uint32_t L, int64_t &m0,
                                             int64_t &n0) {
    const uint32_t per_group = GM * tiles_n;
    const uint32_t g = L / per_group, in = L - g * per_group;
    const uint32_t first_m = g * GM;
    const uint32_t gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    uint32_t mi, ni;
    if (gsz == GM) {
        mi = in % GM;
        ni = in / GM;
    } else {
        ni = in / gsz;
        mi = in - ni * gsz;
    }
    m0 = static_cast<int64_t>(first_m + mi) * BM;
    n0 = static_cast<int64_t>(ni) * BN;
}

// Number of a work item after the XCD-contiguous renumbering: dispatch goes
// round robin over the 8 XCDs (each with its own L2), so items x, x + 8, ...
// run on one XCD and are given consecutive numbers.
__device__ __forceinline__ uint32_t xcd_order(uint32_t item, uint32_t count) {
    return count % 8 == 0 ? (item % 8) * (count / 8) + item / 8 : item;
}

// Origin of output tile `bid` of a BM x BN tiling of M x N.
template <int BM, int BN, int GM>
__device__ __forceinline__ void tile_origin(int64_t M, int64_t N, uint32_t bid, int64_t &m0, int64_t &n0) {
    const uint32_t tiles_m = static_cast<uint32_t>((M + BM - 1) / BM);
    const uint32_t tiles_n = static_cast<uint32_t>((N + BN - 1) / BN);
    group_origin<BM, BN, GM>(tiles_m, tiles_n, xcd_order(bid, tiles_m * tiles_n), m0, n0);
}

// A workgroup of WM x WN wave64s computes a BM x BN output tile; each wave
// owns a (BM/WM) x (BN/WN) sub-tile held as 16x16 fp32 accumulators.  LDS
// row r holds 8 chunks of 8 k; chunk c sits at position c ^ (r & 7).  Two
// LDS stages: stage k+1 is in flight while stage k is consumed.
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
    int64_t m0, n0;
    tile_origin<BM, BN, GM>(M, N, blockIdx.x, m0, n0);

    // ---- per-lane DMA source rows for this wave's share of the blocks
    // block b covers rows 8b..8b+7; lane l fills row r = 8b + l/8, position
    // l%8, which holds chunk (l%8) ^ swz128(r).
    const int drow = lane >> 3;
    const uint16_t *asrc[A_INSTR / NW];
    const uint16_t *bsrc[B_INSTR / NW];
#pragma unroll
    for (int j = 0; j < A_INSTR / NW; ++j) {
        const int r = (wave + j * NW) * 8 + drow;
        int64_t row = m0 + r;
        if (row >= M) row = M - 1;
        asrc[j] = a.X + row * K + ((lane & 7) ^ swz128(r)) * 8;
    }
#pragma unroll
    for (int j = 0; j < B_INSTR / NW; ++j) {
        const int r = (wave + j * NW) * 8 + drow;
        int64_t row = n0 + r;
        if (row >= N) row = N - 1;
        bsrc[j] = a.W + row * K + ((lane & 7) ^ swz128(r)) * 8;
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
                af[ks][i] = *reinterpret_cast<const bf16x8 *>(sa + row * ROWB + ((c ^ swz128(row)) << 4));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 16 + fr;
                bfr[ks][j] = *reinterpret_cast<const bf16x8 *>(sb + row * ROWB + ((c ^ swz128(row)) << 4));
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

// Column position of a value of tile row r in the bf16 LDS staging tile:
// 32-column blocks are swapped when bit 0 of the row differs from bit 2.
// Together with the pair exchange below, the 32-bit writes of one
// instruction then cover each 64-byte run of a 128-byte bank window once.
__device__ __forceinline__ int stage_col(int r, int c) { return c ^ ((((r >> 2) ^ r) & 1) << 5); }

// two fp32 -> bf16 (round to nearest even) in one 32-bit word, lo first
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Write a wave's 32x32-layout accumulators (FM x FN blocks at tile rows
// row0 + 32 i, columns col0 + 32 j), after bias and optional GELU, into the
// bf16 staging tile t16[BM][BN] (columns placed by stage_col).  A lane holds
// one column and pairs of adjacent rows; neighbouring lanes (columns c, c+1)
// swap one value of each pair (DPP quad permutation 1,0,3,2), so that each
// writes two adjacent columns of one row as one 32-bit word.
template <int BN, int FM, int FN, bool GELU>
__device__ __forceinline__ void stage_tile_bf16(uint16_t *t16, const f32x16 (&acc)[FM][FN], const float (&bias)[FN],
                                                int row0, int col0, int lane) {
    const int fr = lane & 31, fq = lane >> 5;
    const bool odd = lane & 1;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 32 + (fr & ~1);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                float e0 = acc[i][j][v] + bias[j], e1 = acc[i][j][v + 1] + bias[j];
                if (GELU) {
                    e0 = gelu_tanh_fast(e0);
                    e1 = gelu_tanh_fast(e1);
                }
                const float send = odd ? e0 : e1;
                const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, true));
                const float lo = odd ? recv : e0, hi = odd ? e1 : recv;
                const int row = row0 + i * 32 + 8 * (v / 4) + (v % 4) + 4 * fq + (odd ? 1 : 0);
                *reinterpret_cast<uint32_t *>(t16 + row * BN + stage_col(row, col)) = pack_bf16x2(lo, hi);
            }
    }
}

// Barrier without a memory fence (the waits are explicit): the empty asm
// statements keep the compiler from moving memory accesses across it, the
// scheduling fences keep every other instruction on its side.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Eight-wave "ping-pong" GEMM.  Waves w and w+4 of a workgroup share a SIMD
// (the dispatcher places wave w on SIMD w mod 4 in a fixed rotation), so the
// workgroup is two groups of four waves, one wave of each group per SIMD.
// Phases are separated by workgroup barriers and the groups take turns: while
// one group runs a phase of nothing but matrix ops, the other reads its
// fragments for the next k-step from LDS and issues its share of the DMA
// copies.  The matrix pipe of every SIMD is then fed by one wave while the
// other wave's memory instructions issue, instead of one wave interleaving
// both.
//   * tile 256 x BN, BK = 32 stages in a D = 5 slot LDS ring (64-byte rows,
//     16-byte chunks at position chunk ^ ((row >> 2) & 3)); wave w owns rows
//     64 (w / 2) .. +63 and columns (BN / 2) (w % 2) .. +BN/2-1: 2 x FN
//     blocks of 32 x 32;
//   * the swizzle: a 32x32 fragment read takes one chunk of 32 rows in
//     lanes 0..31 and the next chunk of the same rows in lanes 32..63.
//     Measured with SQ_LDS_BANK_CONFLICT over the candidate patterns,
//     (row >> 2) & 3 has no bank conflicts here, (row >> 1) & 3 (the
//     conflict-free one for 16-row fragments) costs 4 conflict cycles per
//     read and no swizzle 12.  The DMA writes lane i to position i, so the
//     XOR picks each lane's source;
//   * group 0 reads stage t in phase 2t and multiplies in phase 2t+1;
//   * group 1 is one phase behind: reads in 2t+1, multiplies in 2t+2;
//   * in its read phase for stage t each group issues its copies of stage
//     t+4 into the slot of stage t-1, whose last reader (group 1, phase
//     2t-1) finished before the barrier that opened the phase;
//   * stage s must be in LDS before phase 2s: group 0 waits for its own
//     copies of stage t+1 at the end of its multiply phase for stage t,
//     group 1 at the end of its read phase for stage t, both just before the
//     barrier that opens phase 2t+2.
template <int BN, int GM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pp_kernel(Args a) {
    constexpr int BM = 256, BK = 32, D = 5, LEADK = 4, NW = 8;
    constexpr int TM = 64, TN = BN / 2;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int A_BLK = BM / 16, B_BLK = BN / 16, TOTAL = A_BLK + B_BLK;
    static_assert(TOTAL % 4 == 0 && A_BLK == 2 * NW, "copy split");
    static_assert(D * STAGE <= 160 * 1024 && BM * BN * 2 <= D * STAGE, "LDS budget");
    static_assert(LEADK < D, "a slot is refilled only after its last read");
    static_assert(BN % 64 == 0, "epilogue swizzle works on 64-column halves");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    int64_t m0, n0;
    tile_origin<BM, BN, GM>(M, N, blockIdx.x, m0, n0);

    // DMA: copy j of a wave is 1 KB block wave + 8 j of the stage (blocks
    // 0..15 hold X rows, the rest W rows); lane l fills row 16b + l/4,
    // position l%4, holding chunk (l%4) ^ ((l/16)%4).
    constexpr int NCMAX = (TOTAL + NW - 1) / NW;
    const int drow = lane >> 2;
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(a.X + m0 * K, static_cast<uint32_t>(rows_a * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(a.W + n0 * K, static_cast<uint32_t>(rows_b * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_none = buffer_rsrc(a.X, 0);
    uint32_t voff[NCMAX];
#pragma unroll
    for (int j = 0; j < NCMAX; ++j) {
        const int blk = wave + NW * j;
        const int r = (j < 2 ? blk : blk - A_BLK) * 16 + drow;
        voff[j] = static_cast<uint32_t>(r * K * 2 + dchunk * 16);
    }
    const int KT = static_cast<int>(K / BK);
    auto copy = [&](int j, int t, int slot) {
        const uint32_t soff = static_cast<uint32_t>((t < KT ? t : KT - 1) * (BK * 2));
        dma16_buf(t < KT ? (j < 2 ? rsrc_a : rsrc_b) : rsrc_none, voff[j], soff,
                  lds + slot * STAGE + (wave + NW * j) * 1024);
    };
    auto slot_add = [](int slot, int d) { return slot + d >= D ? slot + d - D : slot + d; };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int fr = lane & 31, fq = lane >> 5;
    const int sw = (fr >> 2) & 3;
    auto frag = [&](const char *base, int row0, int h) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(base + (row0 + fr) * ROWB + (((2 * h + fq) ^ sw) << 4));
    };

    // bias for this lane's columns, loaded before the main loop so that its
    // latency is hidden
    float bias[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 32 + fr;
        bias[j] = ((a.epi & 1) && n < N) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
    }

    // the body for one group; NC: this group's copies per stage (every wave
    // of a group has the same count because TOTAL % 4 == 0)
    auto run = [&](auto grp_tag) {
        constexpr int GRP = decltype(grp_tag)::value;
        constexpr int NC = (TOTAL - 4 * GRP + NW - 1) / NW;
        // prologue: stages 0..LEADK-1 in flight, stage 0 landed and visible
        // (the loop waits for stage t+1 while it works on stage t)
        for (int t = 0; t < LEADK; ++t) {
#pragma unroll
            for (int j = 0; j < NC; ++j) copy(j, t, t);
        }
        wait_vm<NC *(LEADK - 1)>();
        barrier_nofence();
        if (GRP == 1) barrier_nofence();
        bf16x8 af[FM][2], bfr[FN][2];
        for (int t = 0, slot = 0; t < KT; ++t, slot = slot_add(slot, 1)) {
            // read phase: fragments of stage t, copies of stage t + LEADK
            const char *sa = lds + slot * STAGE, *sb = sa + BM * ROWB;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < FM; ++i) af[i][h] = frag(sa, wm * TM + i * 32, h);
#pragma unroll
                for (int j = 0; j < FN; ++j) bfr[j][h] = frag(sb, wn * TN + j * 32, h);
            }
            const int cslot = slot_add(slot, LEADK);
#pragma unroll
            for (int j = 0; j < NC; ++j) copy(j, t + LEADK, cslot);
            if (GRP == 1) {
                wait_vm<NC *(LEADK - 1)>();  // stage t+1 landed (this wave's part)
                // the next phase is group 0's read phase of stage t+1, which
                // refills the slot of stage t: this wave's reads of stage t,
                // the last of that slot, must have landed
                lds_wait_all();
            }
            barrier_nofence();
            // multiply phase
            lds_wait_all();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i][h], bfr[j][h], acc[i][j]);
            if (GRP == 0) wait_vm<NC *(LEADK - 1)>();  // stage t+1 landed (this wave's part)
            barrier_nofence();
        }
        if (GRP == 0) barrier_nofence();
    };
    if (KT > 0) {
        if (grp == 0)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});
    }
    // copies past the end (empty resource) still write LDS: drain them
    wait_vm<0>();
    __syncthreads();

    // ---- epilogue: the tile is staged through LDS as bf16 (stage_tile_bf16),
    // then written with 16-byte row-contiguous stores; partial tiles, fp32
    // output or an unaligned Y store element by element
    const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (N % 8 == 0) && a.out == OUT_BF16 &&
                      (reinterpret_cast<uintptr_t>(a.Y) % 16 == 0);
    if (full) {
        uint16_t *t16 = reinterpret_cast<uint16_t *>(lds);
        if (a.epi & 2)
            stage_tile_bf16<BN, FM, FN, true>(t16, acc, bias, wm * TM, wn * TN, lane);
        else
            stage_tile_bf16<BN, FM, FN, false>(t16, acc, bias, wm * TM, wn * TN, lane);
        __syncthreads();
        // read-back: all of a thread's LDS reads first, then its stores
        constexpr int CPR = BN / 8;
        constexpr int NPASS = BM * CPR / 512;
        static_assert(BM * CPR % 512 == 0, "whole passes");
        u32x4 v[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;
            v[p] = *reinterpret_cast<const u32x4 *>(t16 + row * BN + stage_col(row, ch * 8));
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;
            __builtin_nontemporal_store(v[p], reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.Y) + (m0 + row) * N + n0 + ch * 8));
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
}

// Eight-wave ping-pong GEMM with 128-byte LDS rows.  The same two groups and
// phases as gemm_pp_kernel, but each operand is copied 64 k-values at a time
// (128 bytes per row), which halves the L2 requests of the 64-byte rows and
// the address unit's stalls behind them.  A whole 256 x 256 x 64 stage would
// leave room for only two stages in LDS, so the ring holds operand halves:
// five 32 KB slots that take, in order, A(0), B(0), A(1), B(1), A(2), ...
// (half h in slot h mod 5; A(T) / B(T) are the X / W rows of k-range
// [64T, 64T + 64)).
//   * k-step s (32 k-values) reads A(s/2), B(s/2) at byte offset 64 (s % 2)
//     of each row; rows hold 16-byte chunks at position chunk ^ swz128(row);
//   * group 0 reads step s in phase 2s and multiplies in 2s+1, group 1 is one
//     phase behind; A(T), B(T) are last read in phase 4T+3;
//   * in its read phase of step 2T each group copies its half of B(T+1), in
//     that of step 2T+1 its half of A(T+2): the slots of A(T-1), B(T-1),
//     free since phase 4T;
//   * A(T+1) and B(T+1) must be in LDS before phase 4T+4: each wave waits for
//     all but its copies of A(T+2) at the end of step 2T+1 (group 0 after
//     its matrix ops, group 1 after its reads), just before the barrier that
//     opens phase 4T+4; steps 2T have nothing to wait for.
template <int BN, int GM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pp64_kernel(Args a) {
    constexpr int BM = 256, NW = 8, SLOTS = 5, SLOT = 32 * 1024;
    constexpr int TM = 64, TN = BN / 2;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ROWB = 128;
    constexpr int A_BLK = BM / 8, B_BLK = BN / 8;      // 1 KB copies (8 rows of 128 bytes)
    constexpr int NCA = A_BLK / NW, NCB = B_BLK / NW;  // copies per wave per half
    static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "copies divide over the waves");
    static_assert(BM * ROWB <= SLOT && BN * ROWB <= SLOT, "a half fits a slot");
    static_assert(SLOTS * SLOT <= 160 * 1024 && BM * BN * 2 <= SLOTS * SLOT, "LDS budget");
    static_assert(BN % 64 == 0, "epilogue swizzle works on 64-column halves");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wg = wave & 3;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    int64_t m0, n0;
    tile_origin<BM, BN, GM>(M, N, blockIdx.x, m0, n0);

    // copies: a group's half of an operand half is blocks
    // grp * (BLK/2) + wg + 4 j; lane l of a copy fills row r = 8b + l/8,
    // position l%8, which holds chunk (l%8) ^ swz128(r)
    const int drow = lane >> 3;
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(a.X + m0 * K, static_cast<uint32_t>(rows_a * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(a.W + n0 * K, static_cast<uint32_t>(rows_b * K * 2));
    const __amdgpu_buffer_rsrc_t rsrc_none = buffer_rsrc(a.X, 0);
    const int KH = static_cast<int>(K / 64);  // k-ranges of 64
    auto blk_a = [&](int j) { return grp * (A_BLK / 2) + wg + 4 * j; };
    auto blk_b = [&](int j) { return grp * (B_BLK / 2) + wg + 4 * j; };
    // this wave's copies of A(T) (into half-slot index 2T) or B(T) (2T+1)
    auto copy_a = [&](int T) {
        char *slot = lds + ((2 * T) % SLOTS) * SLOT;
        const uint32_t soff = static_cast<uint32_t>((T < KH ? T : KH - 1) * ROWB);
#pragma unroll
        for (int j = 0; j < NCA; ++j) {
            const int b = blk_a(j);
            const int r = b * 8 + drow;
            dma16_buf(T < KH ? rsrc_a : rsrc_none, static_cast<uint32_t>(r * K * 2 + ((lane & 7) ^ swz128(r)) * 16),
                      soff, slot + b * 1024);
        }
    };
    auto copy_b = [&](int T) {
        char *slot = lds + ((2 * T + 1) % SLOTS) * SLOT;
        const uint32_t soff = static_cast<uint32_t>((T < KH ? T : KH - 1) * ROWB);
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
            const int b = blk_b(j);
            const int r = b * 8 + drow;
            dma16_buf(T < KH ? rsrc_b : rsrc_none, static_cast<uint32_t>(r * K * 2 + ((lane & 7) ^ swz128(r)) * 16),
                      soff, slot + b * 1024);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int fr = lane & 31, fq = lane >> 5;
    const int sw = swz128(fr);  // row0 is a multiple of 32
    // fragment of 32 rows from row0 (a multiple of 32) of a half-slot, k-step
    // parity p, k-half h: chunk 4p + 2h + l/32 of row row0 + l%32
    auto frag = [&](const char *base, int row0, int p, int h) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(base + (row0 + fr) * ROWB + (((4 * p + 2 * h + fq) ^ sw) << 4));
    };

    float bias[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * TN + j * 32 + fr;
        bias[j] = ((a.epi & 1) && n < N) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
    }

    auto run = [&](auto grp_tag) {
        constexpr int GRP = decltype(grp_tag)::value;
        // prologue: A(0), B(0), A(1) in flight, A(0) and B(0) landed and visible
        copy_a(0);
        copy_b(0);
        copy_a(1);
        wait_vm<NCA>();
        barrier_nofence();
        if (GRP == 1) barrier_nofence();
        bf16x8 af[FM][2], bfr[FN][2];
        for (int T = 0; T < KH; ++T) {
            const char *sa = lds + ((2 * T) % SLOTS) * SLOT, *sb = lds + ((2 * T + 1) % SLOTS) * SLOT;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                // read phase of step 2T + p
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int i = 0; i < FM; ++i) af[i][h] = frag(sa, wm * TM + i * 32, p, h);
#pragma unroll
                    for (int j = 0; j < FN; ++j) bfr[j][h] = frag(sb, wn * TN + j * 32, p, h);
                }
                if (p == 0)
                    copy_b(T + 1);
                else
                    copy_a(T + 2);
                if (GRP == 1 && p == 1) {
                    wait_vm<NCA>();  // A(T+1), B(T+1) landed (this wave's part)
                    // the next phase is group 0's read phase of step 2T+2,
                    // which refills the slot of A(T): this wave's reads of
                    // step 2T+1, the last of A(T), must have landed
                    lds_wait_all();
                }
                barrier_nofence();
                // multiply phase
                lds_wait_all();
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i][h], bfr[j][h], acc[i][j]);
                if (GRP == 0 && p == 1) wait_vm<NCA>();
                barrier_nofence();
            }
        }
        if (GRP == 0) barrier_nofence();
    };
    if (KH > 0) {
        if (grp == 0)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});
    }
    // copies past the end (empty resource) still write LDS: drain them
    wait_vm<0>();
    __syncthreads();

    const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (N % 8 == 0) && a.out == OUT_BF16 &&
                      (reinterpret_cast<uintptr_t>(a.Y) % 16 == 0);
    if (full) {
        uint16_t *t16 = reinterpret_cast<uint16_t *>(lds);
        if (a.epi & 2)
            stage_tile_bf16<BN, FM, FN, true>(t16, acc, bias, wm * TM, wn * TN, lane);
        else
            stage_tile_bf16<BN, FM, FN, false>(t16, acc, bias, wm * TM, wn * TN, lane);
        __syncthreads();
        constexpr int CPR = BN / 8;
        constexpr int NPASS = BM * CPR / 512;
        static_assert(BM * CPR % 512 == 0, "whole passes");
        u32x4 v[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;
            v[p] = *reinterpret_cast<const u32x4 *>(t16 + row * BN + stage_col(row, ch * 8));
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;
            __builtin_nontemporal_store(v[p], reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.Y) + (m0 + row) * N + n0 + ch * 8));
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
}

// Write a wave's 16x16x32-layout accumulators (FM x FN blocks at tile rows
// row0 + 16 i, columns col0 + 16 j), after bias and the optional GELU, into
// the bf16 staging tile t16[rows][BN] (columns placed by stage_col).  A lane holds one column and rows 4 (l/16) + 0..3 of each
// block: each pair of adjacent rows is converted in one packed conversion
// and written as two 16-bit stores, which keeps the vector ALU work (the
// bound of a GELU epilogue) at the GELU itself.
template <int BN, int FM, int FN, bool GELU>
__device__ __forceinline__ void stage_tile16_bf16(uint16_t *t16, const f32x4 (&acc)[FM][FN], const float (&bias)[FN],
                                                  int row0, int col0, int lane) {
    const int fr = lane & 15, fg = lane >> 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 16 + fr;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
                float e0 = acc[i][j][v] + bias[j], e1 = acc[i][j][v + 1] + bias[j];
                if (GELU) {
                    e0 = gelu_tanh_fast(e0);
                    e1 = gelu_tanh_fast(e1);
                }
                const uint32_t p = pack_bf16x2(e0, e1);
                const int row = row0 + i * 16 + 4 * fg + v;
                t16[row * BN + stage_col(row, col)] = static_cast<uint16_t>(p);
                t16[(row + 1) * BN + stage_col(row + 1, col)] = static_cast<uint16_t>(p >> 16);
            }
    }
}

// Chunk position of W row r on 128-byte LDS rows for the DIRECT persistent
// kernel.  One of its fragment reads gives 16 lanes the rows
// 8 q + 4 j + t (q, t = 0..3; j fixed) of a 32-row pair: bits 0, 1, 3, 4
// vary.  Rows of each parity (bit 0) must sit at 8 distinct positions of the
// 256-byte bank window (see swz128), so the XOR takes bits 1, 3 and 4.
__device__ __forceinline__ int swz_w(int row) { return ((row >> 1) & 1) | ((row >> 2) & 6); }

// W row (within a 32-row pair) that operand row r of block j of the pair
// reads in the DIRECT persistent kernel.
__device__ __forceinline__ int pair_row(int r, int j) { return 8 * (r >> 2) + 4 * j + (r & 3); }

// bf16 number q (0..7) of eight packed in a 16-byte vector, as fp32
__device__ __forceinline__ float bf16_at(const u32x4 &v, int q) {
    const uint32_t w = v[q >> 1];
    return __uint_as_float((q & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Epilogue of the DIRECT persistent kernel, straight from registers.  Block
// (i, j) of acc holds token rows mrow0 + 16 i + (lane % 16) and, over a pair
// of blocks (2 jp, 2 jp + 1), output features ncol0 + 32 jp + 8 fg .. +7
// (fg = lane / 16): acc[i][2 jp][0..3] then acc[i][2 jp + 1][0..3].  With
// S > 1 the fp32 partial of this K split goes to the workspace; otherwise
// bias, GELU and the output rounding are applied and the 8 outputs are
// written with one 16-byte store (bf16) or two (fp32) where the row holds
// them whole and aligned, element by element at the ragged edges.
template <int FM, int FN>
__device__ __forceinline__ void direct_epilogue(const Args &a, const f32x4 (&acc)[FM][FN],
                                                const u32x4 (&biasp)[FN / 2], int S, int split, int64_t mrow0,
                                                int64_t ncol0, int fr, int fg) {
    const int64_t M = a.M, N = a.N;
    if (S > 1) {
        float *ws = a.ws + static_cast<int64_t>(split) * M * N;
        const bool vec = N % 4 == 0;  // the workspace is 256-byte aligned and n a multiple of 8
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = mrow0 + i * 16 + fr;
#pragma unroll
            for (int jp = 0; jp < FN / 2; ++jp) {
                const int64_t n = ncol0 + jp * 32 + 8 * fg;
                if (m >= M || n >= N) continue;
                float *dst = ws + m * N + n;
                // plus the bias registers, which read zero here (see the
                // caller): every path reads them
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (e < 4 ? acc[i][2 * jp][e] : acc[i][2 * jp + 1][e - 4]) + bf16_at(biasp[jp], e);
                if (vec && n + 8 <= N) {
                    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(dst));
                    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(dst + 4));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) dst[e] = v[e];
                }
            }
        }
        return;
    }
    const bool yal = reinterpret_cast<uintptr_t>(a.Y) % 16 == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = mrow0 + i * 16 + fr;
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp) {
            const int64_t n = ncol0 + jp * 32 + 8 * fg;
            if (m >= M || n >= N) continue;
            // the bias is added even when there is none (it reads zero
            // then): a sum started at +0 is never -0, so adding +0 changes
            // nothing, and the bias registers are then read on every path
            // (a loaded register left unread stays pending into the next
            // tile, whose first reuse of it would wait behind the stores)
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (e < 4 ? acc[i][2 * jp][e] : acc[i][2 * jp + 1][e - 4]) + bf16_at(biasp[jp], e);
            if (a.epi & 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = gelu_tanh_fast(v[e]);
            }
            if (a.out == OUT_BF16) {
                uint16_t *y = static_cast<uint16_t *>(a.Y) + m * N + n;
                if (yal && N % 8 == 0 && n + 8 <= N) {
                    const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                      pack_bf16x2(v[6], v[7])};
                    __builtin_nontemporal_store(pk, reinterpret_cast<u32x4 *>(y));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) y[e] = f32_to_bf16_bits(v[e]);
                }
            } else {
                float *y = static_cast<float *>(a.Y) + m * N + n;
                if (yal && N % 4 == 0 && n + 8 <= N) {
                    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(y));
                    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(y + 4));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) y[e] = v[e];
                }
            }
        }
    }
}

// Persistent form of gemm_pp64_kernel: one workgroup per CU walks tiles
// blockIdx.x, blockIdx.x + gridDim.x, ...  The LDS ring runs on across tiles
// (the copies the last k-ranges of a tile would make past K fetch the next
// tile's A(0), B(0), A(1) instead), so the next tile's first operands are in
// flight while this tile finishes and its epilogue runs, and there is no
// workgroup launch between tiles.  The epilogue stages the tile through the
// two slots the last k-range frees (the other three hold the next tile's
// first halves): group 0's rows 0..127 first, then group 1's rows 128..255,
// each 64-row wave block in one slot.  Needs K >= 128 (two k-ranges), so
// that the ring's look-ahead stays within the next tile.
// With S > 1 the work items are (tile, K split) pairs -- for token counts
// that give too few tiles to fill the CUs -- and each item writes its fp32
// partial to the workspace, which the split-K reduction kernel sums with the
// epilogue; a split covers at least two k-ranges.
// Matrix ops are 16x16x32 (each wave 4 x BN/32 blocks of 16 x 16, one
// fragment per 16 rows and k-step): with the same LDS traffic this form ran
// 6% faster than 32x32x16 blocks on the M=4096, K=N=8192 GEMM.
//
// DIRECT (family gemmpp64d): the matrix op takes the W fragment as its first
// operand and the X fragment as its second, so a 16 x 16 block holds Y
// transposed: a lane holds one token row (lane % 16) and four output
// features.  The 16 W rows of the two blocks of each 32-feature pair are
// taken in the order 8 (r / 4) + 4 j + r % 4 (r the operand row, j the block
// of the pair), so a lane holds 8 consecutive features of its row:
// features 8 (lane / 16) .. +7 of the pair.  The epilogue then adds the
// bias, applies GELU and stores those 8 outputs as one 16-byte store (bf16)
// straight from registers -- no staging through LDS and no barrier, so the
// next tile's first k-ranges (already in flight) start right after.  W rows
// are then read 16 at a time in that order, so W's chunks are placed by
// swz_w (below) instead of swz128 to stay free of bank conflicts.
template <int BN, int GM, bool DIRECT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pp64p_kernel(Args a, int S) {
    constexpr int BM = 256, NW = 8, SLOTS = 5, SLOT = 32 * 1024;
    constexpr int TM = 64, TN = BN / 2;
    constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 blocks
    constexpr int ROWB = 128;
    constexpr int A_BLK = BM / 8, B_BLK = BN / 8;
    constexpr int NCA = A_BLK / NW, NCB = B_BLK / NW;
    static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "copies divide over the waves");
    static_assert(BM * ROWB <= SLOT && BN * ROWB <= SLOT && TM * BN * 2 <= SLOT, "halves and staging fit a slot");
    static_assert(SLOTS * SLOT <= 160 * 1024, "LDS budget");
    static_assert(BN % 64 == 0, "epilogue swizzle works on 64-column halves");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wg = wave & 3;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;
    // Work items are decoded in 32-bit arithmetic (the launcher keeps
    // tiles x S below 2^31), with one division by a runtime value per item
    // for S = 1: the decoding runs at the start of every tile, on the path
    // to its first copies, and a 64-bit division by a runtime value is a
    // sequence of over a hundred scalar instructions.
    const uint32_t tiles_m = static_cast<uint32_t>((M + BM - 1) / BM);
    const uint32_t tiles_n = static_cast<uint32_t>((N + BN - 1) / BN);
    const uint32_t us = static_cast<uint32_t>(S);
    // work items: (tile, K split) pairs, item = tile * S + split; a split
    // covers k-ranges [KH * split / S, KH * (split + 1) / S), at least two
    const uint32_t GS = tiles_m * tiles_n * us;
    const uint32_t KH = static_cast<uint32_t>(K / 64);
    struct Work {
        int64_t m0, n0;
        int kb, ke, split;
    };
    // item -> tile origin and k-ranges: XCD-contiguous renumbering of the
    // items (a workgroup's items all lie on its XCD, since gridDim.x is a
    // multiple of 8), then GM-row groups of tiles
    auto decode = [&](uint32_t item) -> Work {
        const uint32_t r = xcd_order(item, GS);
        Work w;
        uint32_t L = r;
        w.split = 0;
        w.kb = 0;
        w.ke = static_cast<int>(KH);
        if (us > 1) {
            L = r / us;
            const uint32_t sp = r - L * us;
            w.split = static_cast<int>(sp);
            w.kb = static_cast<int>((KH * sp) / us);
            w.ke = static_cast<int>((KH * (sp + 1)) / us);
        }
        group_origin<BM, BN, GM>(tiles_m, tiles_n, L, w.m0, w.n0);
        return w;
    };
    // buffer resources over an item's tile's valid X and W rows, and the
    // item's first k-range (empty resources past the last item)
    auto resources = [&](uint32_t item, __amdgpu_buffer_rsrc_t &ra, __amdgpu_buffer_rsrc_t &rb, int &kb) {
        if (item >= GS) {
            ra = rb = buffer_rsrc(a.X, 0);
            kb = 0;
            return;
        }
        const Work w = decode(item);
        kb = w.kb;
        const int64_t rows_a = (M - w.m0) < BM ? (M - w.m0) : BM;
        const int64_t rows_b = (N - w.n0) < BN ? (N - w.n0) : BN;
        ra = buffer_rsrc(a.X + w.m0 * a.kx, static_cast<uint32_t>(rows_a * a.kx * 2));
        rb = buffer_rsrc(a.W + w.n0 * K, static_cast<uint32_t>(rows_b * K * 2));
    };

    const int drow = lane >> 3;
    // X rows are kx long (K, or K/2 for a hi/lo weight pair, whose second
    // half of k-ranges reads X from the start again)
    const int KHX = static_cast<int>(a.kx / 64);
    auto copy_a = [&](__amdgpu_buffer_rsrc_t r, int T, int slot) {
        const uint32_t soff = static_cast<uint32_t>((T >= KHX ? T - KHX : T) * ROWB);
#pragma unroll
        for (int j = 0; j < NCA; ++j) {
            const int b = grp * (A_BLK / 2) + wg + 4 * j;
            const int row = b * 8 + drow;
            dma16_buf(r, static_cast<uint32_t>(row * a.kx * 2 + ((lane & 7) ^ swz128(row)) * 16), soff,
                      lds + slot * SLOT + b * 1024);
        }
    };
    auto copy_b = [&](__amdgpu_buffer_rsrc_t r, int T, int slot) {
        const uint32_t soff = static_cast<uint32_t>(T * ROWB);
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
            const int b = grp * (B_BLK / 2) + wg + 4 * j;
            const int row = b * 8 + drow;
            const int sz = DIRECT ? swz_w(row) : swz128(row);
            dma16_buf(r, static_cast<uint32_t>(row * K * 2 + ((lane & 7) ^ sz) * 16), soff,
                      lds + slot * SLOT + b * 1024);
        }
    };
    auto slot_add = [](int slot, int d) { return slot + d >= SLOTS ? slot + d - SLOTS : slot + d; };

    // 16x16x32 fragments: lane l reads row row0 + l%16, chunk 4p + l/16
    const int fr = lane & 15, fg = lane >> 4;
    const int sw = swz128(fr);  // row0 is a multiple of 16
    auto frag = [&](const char *base, int row0, int p) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(base + (row0 + fr) * ROWB + (((4 * p + fg) ^ sw) << 4));
    };
    // DIRECT: block j of the wave's W rows (pair j / 2, block j % 2 of it)
    auto frag_w = [&](const char *base, int j, int p) -> bf16x8 {
        const int row = wn * TN + (j >> 1) * 32 + pair_row(fr, j & 1);
        return *reinterpret_cast<const bf16x8 *>(base + row * ROWB + (((4 * p + fg) ^ swz_w(row)) << 4));
    };
    static_assert(!DIRECT || FN % 2 == 0, "DIRECT takes W blocks in pairs");

    uint32_t item = blockIdx.x;
    __amdgpu_buffer_rsrc_t ca, cb, na, nb;
    int ckb, nkb;
    resources(item, ca, cb, ckb);
    // slot of A of the current k-range (half index 2g for the g-th k-range
    // this workgroup handles, counted across items)
    int s0 = 0;
    copy_a(ca, ckb, 0);
    copy_b(cb, ckb, 1);
    copy_a(ca, ckb + 1, 2);
    // the next item's resources while the first copies are in flight
    resources(item + gridDim.x, na, nb, nkb);
    wait_vm<NCA>();
    barrier_nofence();

    for (; item < GS; item += gridDim.x) {
        const Work cur = decode(item);
        const int64_t m0 = cur.m0, n0 = cur.n0;
        const int kb = cur.kb, ke = cur.ke, split = cur.split;
        // Bias bits of this lane's output features (column j * 16 + fr of
        // block j, or (DIRECT) features 8 fg .. +7 of pair jp as packed
        // bf16), read through a resource over the N bias values: features
        // past N, and every feature when there is no bias, read zero.  They
        // are converted only in the epilogue.  Using them here would wait
        // for these loads, and loads and stores complete in order, so that
        // wait would also take in every copy and every store of the
        // previous tile's output still in flight.  The loads are issued on
        // every path and every epilogue path adds what they read (zero
        // when there is no bias, and for a K split, S > 1, whose bias the
        // reduction adds): a loaded register left unread is still pending
        // when the next tile reuses it, and that reuse would wait the same
        // way.  A sum started at +0 is never -0, so adding +0 changes
        // nothing.
        constexpr int NB = DIRECT ? 1 : FN;
        constexpr int NBP = DIRECT ? FN / 2 : 1;
        const __amdgpu_buffer_rsrc_t rbias =
            buffer_rsrc(a.bias, ((a.epi & 1) && S == 1) ? static_cast<uint32_t>(N * 2) : 0u);
        uint32_t braw[NB];  // one 32-bit register each: packing two would wait for both loads
        u32x4 biasp[NBP];
        if constexpr (!DIRECT) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t n = n0 + wn * TN + j * 16 + fr;
                braw[j] = __builtin_amdgcn_raw_buffer_load_b16(rbias, static_cast<int>(n * 2), 0, 0);
            }
        } else if (N % 8 == 0) {
            // a lane's 8 features lie wholly inside or wholly past N
#pragma unroll
            for (int jp = 0; jp < FN / 2; ++jp) {
                const int64_t n = n0 + wn * TN + jp * 32 + 8 * fg;
                biasp[jp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, static_cast<int>(n * 2), 0, 0));
            }
        } else {
#pragma unroll
            for (int jp = 0; jp < FN / 2; ++jp) {
                const int64_t n = n0 + wn * TN + jp * 32 + 8 * fg;
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rbias, static_cast<int>((n + 2 * q) * 2), 0, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rbias, static_cast<int>((n + 2 * q + 1) * 2), 0, 0);
                    w[q] = lo | (hi << 16);
                }
                biasp[jp] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        f32x4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto run = [&](auto grp_tag) {
            constexpr int GRP = decltype(grp_tag)::value;
            if (GRP == 1) barrier_nofence();
            bf16x8 af[FM], bfr[FN];
            for (int T = kb; T < ke; ++T) {
                const char *sa = lds + s0 * SLOT, *sb = lds + slot_add(s0, 1) * SLOT;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
#pragma unroll
                    for (int i = 0; i < FM; ++i) af[i] = frag(sa, wm * TM + i * 16, p);
#pragma unroll
                    for (int j = 0; j < FN; ++j) bfr[j] = DIRECT ? frag_w(sb, j, p) : frag(sb, wn * TN + j * 16, p);
                    if (p == 0) {
                        // B(T+1): this item's, or the next item's first
                        if (T + 1 < ke)
                            copy_b(cb, T + 1, slot_add(s0, 3));
                        else
                            copy_b(nb, nkb, slot_add(s0, 3));
                    } else {
                        // A(T+2): this item's, or the next item's first two
                        if (T + 2 < ke)
                            copy_a(ca, T + 2, slot_add(s0, 4));
                        else
                            copy_a(na, nkb + T + 2 - ke, slot_add(s0, 4));
                    }
                    if (GRP == 1 && p == 1) {
                        wait_vm<NCA>();  // A(T+1), B(T+1) landed (this wave's part)
                        lds_wait_all();  // the next phase refills the slot of A(T)
                    }
                    barrier_nofence();
                    lds_wait_all();
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = DIRECT ? mfma16x16x32(bfr[j], af[i], acc[i][j])
                                               : mfma16x16x32(af[i], bfr[j], acc[i][j]);
                    if (GRP == 0 && p == 1) wait_vm<NCA>();
                    barrier_nofence();
                }
                s0 = slot_add(s0, 2);
            }
            if (GRP == 0) barrier_nofence();
        };
        if (grp == 0)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});

        if constexpr (DIRECT) {
            direct_epilogue<FM, FN>(a, acc, biasp, S, split, m0 + wm * TM, n0 + wn * TN, fr, fg);
        } else {
        float bias[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            // the empty asm keeps the conversion (and the compiler's wait for
            // the load) here rather than hoisted up to the load
            uint32_t bits = braw[j];
            asm volatile("" : "+v"(bits));
            bias[j] = bf16_bits_to_f32(bits);
        }
        // ---- epilogue.  The slots of the last k-range's A and B (s0 + 3,
        // s0 + 4) are free once every wave's reads of it have landed; the
        // next tile's A(0), B(0), A(1) are in the other three.
        const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (N % 8 == 0) && a.out == OUT_BF16 &&
                          (reinterpret_cast<uintptr_t>(a.Y) % 16 == 0);
        if (S > 1) {
            // fp32 partial of this K split, summed (with the epilogue) by
            // the split-K reduction kernel
            float *ws = a.ws + static_cast<int64_t>(split) * M * N;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t n = n0 + wn * TN + j * 16 + fr;
                if (n >= N) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int64_t m = m0 + wm * TM + i * 16 + 4 * fg + v;
                        if (m < M) __builtin_nontemporal_store(acc[i][j][v] + bias[j], ws + m * N + n);
                    }
            }
        } else if (full) {
            lds_wait_all();
            barrier_nofence();
            uint16_t *stage0 = reinterpret_cast<uint16_t *>(lds + slot_add(s0, 3) * SLOT);
            uint16_t *stage1 = reinterpret_cast<uint16_t *>(lds + slot_add(s0, 4) * SLOT);
            constexpr int CPR = BN / 8;
            constexpr int NPASS = 2 * TM * CPR / 512;
            static_assert(2 * TM * CPR % 512 == 0, "whole passes");
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                // round r: group r's two 64-row blocks (wave rows wm * 64)
                if (grp == r) {
                    uint16_t *t16 = (wm & 1) ? stage1 : stage0;
                    if (a.epi & 2)
                        stage_tile16_bf16<BN, FM, FN, true>(t16, acc, bias, 0, wn * TN, lane);
                    else
                        stage_tile16_bf16<BN, FM, FN, false>(t16, acc, bias, 0, wn * TN, lane);
                }
                lds_wait_all();
                barrier_nofence();
                u32x4 v[NPASS];
#pragma unroll
                for (int p = 0; p < NPASS; ++p) {
                    const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;  // row 0..127 of the round
                    const uint16_t *t16 = (row >= TM) ? stage1 : stage0;
                    const int rr = row & (TM - 1);
                    v[p] = *reinterpret_cast<const u32x4 *>(t16 + rr * BN + stage_col(rr, ch * 8));
                }
#pragma unroll
                for (int p = 0; p < NPASS; ++p) {
                    const int c = tid + 512 * p, row = c / CPR, ch = c % CPR;
                    __builtin_nontemporal_store(
                        v[p], reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.Y) + (m0 + r * 2 * TM + row) * N + n0 + ch * 8));
                }
                lds_wait_all();
                barrier_nofence();
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t n = n0 + wn * TN + j * 16 + fr;
                if (n >= N) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int64_t m = m0 + wm * TM + i * 16 + 4 * fg + v;
                        if (m < M) store_out(a.Y, a.out, m * N + n, apply_epilogue(acc[i][j][v], a.epi, bias[j]));
                    }
            }
        }
        }
        ca = na;
        cb = nb;
        resources(item + 2 * gridDim.x, na, nb, nkb);
    }
    // the copies issued for the tile after the last one (empty resource)
    // still write LDS: drain them before the workgroup ends
    wait_vm<0>();
}

// One list drives both compilation passes (device: kernel instantiation,
// host: launch table).
#define PROJ_GEMM_VARIANTS(X)                                                                    \
    X(128, 128, 2, 2, 4) X(256, 128, 2, 2, 4) X(128, 256, 2, 2, 4) X(256, 256, 2, 2, 4)          \
    X(256, 192, 2, 2, 4) X(192, 256, 2, 2, 4) X(256, 256, 2, 4, 4) X(256, 256, 4, 2, 4)          \
    X(256, 128, 4, 2, 4) X(256, 256, 2, 2, 8) X(256, 256, 2, 2, 2)

#define PROJ_GEMM_INST(BM, BN, WM, WN, GM) template __global__ void gemm_kernel<BM, BN, 64, WM, WN, GM>(Args);
PROJ_GEMM_VARIANTS(PROJ_GEMM_INST)


#define PROJ_GEMM_PP_VARIANTS(X) X(256, 4) X(256, 8) X(192, 4)
#define PROJ_GEMM_PP_INST(BN, GM) template __global__ void gemm_pp_kernel<BN, GM>(Args);
PROJ_GEMM_PP_VARIANTS(PROJ_GEMM_PP_INST)

#define PROJ_GEMM_PP64_VARIANTS(X) X(256, 4) X(256, 8) X(192, 4)
#define PROJ_GEMM_PP64_INST(BN, GM) template __global__ void gemm_pp64_kernel<BN, GM>(Args);
PROJ_GEMM_PP64_VARIANTS(PROJ_GEMM_PP64_INST)
#define PROJ_GEMM_PP64P_INST(BN, GM)                                          \
    template __global__ void gemm_pp64p_kernel<BN, GM, false>(Args, int); \
    template __global__ void gemm_pp64p_kernel<BN, GM, true>(Args, int);
PROJ_GEMM_PP64_VARIANTS(PROJ_GEMM_PP64P_INST)

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
static hipError_t launch_gemm(const Args &a, int S, hipStream_t st) {
    if (S != 1 || a.kx != a.K || a.wpack) return hipErrorInvalidValue;  // no K split, hi/lo pair or packed W
    const int64_t G = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = 2 * (BM + BN) * BK * 2;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, GM>), dim3(static_cast<unsigned>(G)),
                       dim3(WM * WN * 64), lds_bytes, st, a);
    return hipGetLastError();
}

// The ping-pong kernels address a 256-row tile through 32-bit buffer
// offsets.
constexpr int64_t kRingMaxK = (int64_t{1} << 31) / (256 * 2);

template <int BN, int GM>
static hipError_t prepare_gemm_pp() {
    auto fn = gemm_pp_kernel<BN, GM>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               5 * (256 + BN) * 64);
}

template <int BN, int GM>
static hipError_t launch_gemm_pp(const Args &a, int S, hipStream_t st) {
    if (S != 1 || a.kx != a.K || a.wpack) return hipErrorInvalidValue;  // no K split, hi/lo pair or packed W
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = 5 * (256 + BN) * 64;
    hipLaunchKernelGGL((gemm_pp_kernel<BN, GM>), dim3(static_cast<unsigned>(G)), dim3(512), lds_bytes, st, a);
    return hipGetLastError();
}

template <int BN, int GM>
static hipError_t prepare_gemm_pp64() {
    auto fn = gemm_pp64_kernel<BN, GM>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               5 * 32 * 1024);
}

template <int BN, int GM>
static hipError_t launch_gemm_pp64(const Args &a, int S, hipStream_t st) {
    if (S != 1 || a.kx != a.K || a.wpack) return hipErrorInvalidValue;  // no K split, hi/lo pair or packed W
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_pp64_kernel<BN, GM>), dim3(static_cast<unsigned>(G)), dim3(512), 5 * 32 * 1024, st, a);
    return hipGetLastError();
}

// compute units of the device the library was prepared on (the persistent
// kernel launches one workgroup per CU)
static int g_num_cus = 0;

template <int BN, int GM, bool DIRECT>
static hipError_t prepare_gemm_pp64p() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&g_num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    auto fn = gemm_pp64p_kernel<BN, GM, DIRECT>;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                               5 * 32 * 1024);
}

// K < 128 (one k-range) runs the non-persistent kernel; S > 1 splits K into
// S parts of at least two k-ranges each and adds the reduction pass
template <int BN, int GM, bool DIRECT>
static hipError_t launch_gemm_pp64p(const Args &a, int S, hipStream_t st) {
    if (a.wpack || (a.kx != a.K && (a.kx % 64 != 0 || a.K < 128))) return hipErrorInvalidValue;
    if (a.K < 128) return S == 1 ? launch_gemm_pp64<BN, GM>(a, 1, st) : hipErrorInvalidValue;
    if (S < 1 || a.K / 64 < 2 * static_cast<int64_t>(S)) return hipErrorInvalidValue;
    const int64_t G = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN) * S;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t cus = g_num_cus > 0 ? g_num_cus : 256;
    const int64_t grid = G < cus ? G : cus;
    hipLaunchKernelGGL((gemm_pp64p_kernel<BN, GM, DIRECT>), dim3(static_cast<unsigned>(grid)), dim3(512), 5 * 32 * 1024, st, a,
                       S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_splitk_reduce(a, S, st);
}

#define PROJ_GEMM_ENTRY(BM, BN, WM, WN, GM) \
    {"gemm", BM, BN, 64, 64, WM, WN, GM, 0, 1, &launch_gemm<BM, BN, 64, WM, WN, GM>, &prepare_gemm<BM, BN, 64, WM, WN, GM>},
#define PROJ_GEMM_PP_ENTRY(BN, GM) \
    {"gemmpp", 256, BN, 32, 32, 4, 2, GM, kRingMaxK, 1, &launch_gemm_pp<BN, GM>, &prepare_gemm_pp<BN, GM>},
#define PROJ_GEMM_PP64_ENTRY(BN, GM) \
    {"gemmpp64", 256, BN, 64, 64, 4, 2, GM, kRingMaxK, 1, &launch_gemm_pp64<BN, GM>, &prepare_gemm_pp64<BN, GM>},
#define PROJ_GEMM_PP64P_ENTRY(BN, GM) \
    {"gemmpp64p", 256, BN, 64, 64, 4, 2, GM, kRingMaxK, 16, &launch_gemm_pp64p<BN, GM, false>, &prepare_gemm_pp64p<BN, GM, false>},
#define PROJ_GEMM_PP64D_ENTRY(BN, GM) \
    {"gemmpp64d", 256, BN, 64, 64, 4, 2, GM, kRingMaxK, 16, &launch_gemm_pp64p<BN, GM, true>, &prepare_gemm_pp64p<BN, GM, true>},
const GemmVariant kGemmVariants[] = {PROJ_GEMM_VARIANTS(PROJ_GEMM_ENTRY) PROJ_GEMM_PP_VARIANTS(PROJ_GEMM_PP_ENTRY)
                                         PROJ_GEMM_PP64_VARIANTS(PROJ_GEMM_PP64_ENTRY)
                                             PROJ_GEMM_PP64_VARIANTS(PROJ_GEMM_PP64P_ENTRY)
                                                 PROJ_GEMM_PP64_VARIANTS(PROJ_GEMM_PP64D_ENTRY)};
const int kNumGemmVariants = sizeof(kGemmVariants) / sizeof(kGemmVariants[0]);
#endif

}  // namespace proj
