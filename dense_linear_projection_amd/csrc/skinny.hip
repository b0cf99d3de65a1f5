// skinny.hip -- weight-streaming projection for few token rows (M <= 64).
//
// At small M every weight is used by only M rows, so the time goes into
// reading W once (worklog "How I made Muse's GPU projections 1.32x faster
// in the Open Kernel Challenge", section "A rough way to ask how much room
// was left": M flops per weight byte).  The kernel therefore streams W with
// 128-bit loads, splits the long K sum over many waves so that every CU has
// loads in flight (same page, sections "Having lots of workers doesn't help
// if I give them nothing to do" and "My first useful win: split up the
// sum"), and combines the partial sums on chip.
//
// Work decomposition (one workgroup = WAVES wave64s):
//   * a workgroup owns NT*16 consecutive output features n (W rows) and one
//     of S contiguous K ranges; ranges split the ceil(K/32) k-steps as evenly
//     as integers allow (floor(s*T/S) .. floor((s+1)*T/S)), so every k-step
//     is summed exactly once (same page, section "How splitting changes the
//     grid" and the uneven three-way split in "Why the later TMA/WGMMA kernel
//     was a new experiment");
//   * inside the workgroup, wave w takes k-steps w, w+WAVES, w+2*WAVES, ...
//     of that range, so at any moment the waves of a workgroup read one
//     contiguous stretch of each W row;
//   * a k-step is one v_mfma_f32_16x16x32_bf16 per (m-tile, n-tile): the A
//     operand is 16 token rows x 32 k of X, the B operand 32 k x 16 features
//     of W; each lane loads 8 consecutive k (16 bytes) of one X row and one W
//     row, and the same k chunk for both, so the contraction pairs matching
//     k whatever order the hardware sums in;
//   * partial accumulators of the waves are summed through LDS; with S == 1
//     the workgroup applies the epilogue and writes Y once; with S > 1 it
//     stores its fp32 partial tile to the workspace, and the last workgroup
//     of the tile to arrive (completion counter, release/acquire fences; the
//     page's "last-block" scheme, section "Why a last-block scheme was more
//     complicated than it sounded") sums the S partials in split order --
//     so the result does not depend on arrival order -- applies the
//     epilogue, writes Y, and resets the counter to zero for the next call
//     or graph replay.
//
// Rows beyond M or N read a clamped valid row (their results are never
// stored), and the k chunks of a final partial k-step (K % 32 != 0) read the
// zero page instead of memory, so no load leaves the caller's buffers.
#include "common.hpp"
#include "kernels.hpp"

namespace proj {

template <int MT, int NT, int WAVES, int U, bool NTL, bool ROT>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(Args a, int S) {
    constexpr int E = MT * NT * 256;  // fp32 outputs per workgroup tile
    __shared__ float red[WAVES * E];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;   // operand row inside a 16-row block
    const int g = lane >> 4;   // which 8-element k chunk of the 32-k step
    const int tile = blockIdx.x / S;
    const int split = blockIdx.x % S;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t n0 = static_cast<int64_t>(tile) * (16 * NT);

    const uint16_t *wp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int64_t n = n0 + nt * 16 + r;
        if (n >= N) n = N - 1;
        wp[nt] = a.W + n * K + 8 * g;
    }
    const uint16_t *xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int64_t m = mt * 16 + r;
        if (m >= M) m = M - 1;
        xp[mt] = a.X + m * K + 8 * g;
    }

    const int64_t T = (K + 31) / 32;          // k-steps, the last may be partial
    const int64_t Tfull = K / 32;
    const int64_t tb = (T * split) / S, te = (T * (split + 1)) / S;
    const int64_t tfe = te < Tfull ? te : Tfull;  // end of full steps in range
    const int64_t nfull = tfe > tb ? tfe - tb : 0;  // full k-steps of this split
    // Position p of the split's full steps is k-step tb + (p + rot) mod nfull.
    // With ROT, workgroups start at different k so that, at any moment, the
    // machine's loads are spread over the whole K extent of W instead of all
    // hitting the same column offset of every (power-of-two strided) row.
    const int64_t rot = (ROT && nfull > 0) ? (static_cast<int64_t>(tile) * 97) % nfull : 0;
    const int64_t nj = nfull > wave ? (nfull - wave + WAVES - 1) / WAVES : 0;
    auto step = [&](int64_t j) -> int64_t {
        int64_t p = wave + j * WAVES + rot;
        if (p >= nfull) p -= nfull;
        return tb + p;
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto ldw = [&](int nt, int64_t t) -> bf16x8 {
        const uint16_t *p = wp[nt] + 32 * t;
        return NTL ? load16_nt(p) : load16(p);
    };
    auto ldx = [&](int mt, int64_t t) -> bf16x8 { return load16(xp[mt] + 32 * t); };

    // Double-buffered batches of U k-steps: the loads of batch b+1 are in
    // flight while batch b feeds the MFMAs.
    const int64_t nb = nj / U;
    bf16x8 wc[U][NT], xc[U][MT];
    if (nb > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t t = step(u);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wc[u][nt] = ldw(nt, t);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xc[u][mt] = ldx(mt, t);
        }
    }
#pragma unroll 2
    for (int64_t b = 0; b < nb; ++b) {
        bf16x8 wn[U][NT], xn[U][MT];
        if (b + 1 < nb) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int64_t t = step((b + 1) * U + u);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) wn[u][nt] = ldw(nt, t);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xn[u][mt] = ldx(mt, t);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = mfma16x16x32(xc[u][mt], wc[u][nt], acc[mt][nt]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wc[u][nt] = wn[u][nt];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xc[u][mt] = xn[u][mt];
        }
    }
    // leftover full steps
    for (int64_t j = nb * U; j < nj; ++j) {
        int64_t t = step(j);
        bf16x8 w1[NT], x1[MT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) w1[nt] = ldw(nt, t);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) x1[mt] = ldx(mt, t);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(x1[mt], w1[nt], acc[mt][nt]);
    }
    // final partial k-step (K % 32 != 0): chunks past K read zeros
    if (te > Tfull && Tfull >= tb && ((Tfull - tb) % WAVES) == wave) {
        const bool in = 32 * Tfull + 8 * g < K;
        bf16x8 w1[NT], x1[MT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) w1[nt] = load16(in ? wp[nt] + 32 * Tfull : a.zeros);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) x1[mt] = load16(in ? xp[mt] + 32 * Tfull : a.zeros);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(x1[mt], w1[nt], acc[mt][nt]);
    }

    // ---- sum the waves' partial tiles through LDS: red[wave][tile][i][lane]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[wave * E + (mt * NT + nt) * 256 + i * 64 + lane] = acc[mt][nt][i];
    __syncthreads();

    constexpr int PER = (E + WAVES * 64 - 1) / (WAVES * 64);
    float sum[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid + q * WAVES * 64;
        float s = 0.f;
        if (e < E) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s += red[w * E + e];
        }
        sum[q] = s;
    }

    // element e -> (m, n) of the MFMA output layout: lane holds column
    // lane%16 and rows 4*(lane/16) + i of each 16x16 block.
    auto coords = [&](int e, int64_t &m, int64_t &n) {
        const int tl = e >> 8, i = (e >> 6) & 3, ln = e & 63;
        const int mt = tl / NT, nt = tl % NT;
        m = mt * 16 + 4 * (ln >> 4) + i;
        n = n0 + nt * 16 + (ln & 15);
    };

    if (S > 1) {
        // publish this split's partial tile, then count arrivals
        float *part = a.ws + (static_cast<int64_t>(tile) * S + split) * E;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = tid + q * WAVES * 64;
            if (e < E) part[e] = sum[q];
        }
        __threadfence();
        __syncthreads();
        __shared__ int last;
        if (tid == 0) {
            unsigned prev = atomicAdd(&a.counters[tile], 1u);
            last = (prev == static_cast<unsigned>(S - 1));
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        const float *base = a.ws + static_cast<int64_t>(tile) * S * E;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = tid + q * WAVES * 64;
            float s = 0.f;
            if (e < E) {
                for (int sp = 0; sp < S; ++sp) s += __builtin_nontemporal_load(base + sp * E + e);
            }
            sum[q] = s;
        }
        if (tid == 0) a.counters[tile] = 0u;
    }

#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid + q * WAVES * 64;
        if (e >= E) continue;
        int64_t m, n;
        coords(e, m, n);
        if (m < M && n < N) {
            const float b = (a.epi & 1) ? bf16_bits_to_f32(a.bias[n]) : 0.f;
            store_out(a.Y, a.out, m * N + n, apply_epilogue(sum[q], a.epi, b));
        }
    }
}

// ---------------------------------------------------------------- registry
// One list drives both compilation passes: the device pass instantiates the
// kernels, the host pass builds the launch table.  Variants that would spill
// registers at their occupancy are left out.
#define PROJ_SKINNY_VARIANTS(X)                                                                            \
    X(1, 1, 4, 4, false, false) X(1, 1, 8, 4, false, false) X(1, 1, 8, 8, false, false)                     \
    X(1, 1, 16, 4, false, false) X(1, 2, 8, 4, false, false) X(1, 2, 16, 2, false, false)                   \
    X(1, 4, 8, 2, false, false) X(1, 1, 8, 4, true, false) X(1, 2, 16, 2, true, false)                      \
    X(1, 1, 8, 4, false, true) X(1, 1, 8, 8, false, true) X(1, 1, 16, 4, false, true)                        \
    X(1, 2, 8, 4, false, true) X(1, 2, 16, 2, false, true) X(1, 1, 8, 4, true, true)                         \
    X(1, 2, 16, 2, true, true) X(2, 1, 8, 4, false, false) X(2, 2, 8, 4, false, false)                       \
    X(2, 2, 16, 2, false, false) X(2, 2, 16, 2, false, true) X(4, 1, 8, 4, false, false)                    \
    X(4, 2, 8, 2, false, false) X(4, 4, 4, 2, false, false) X(4, 2, 8, 2, false, true)                      \
    X(4, 4, 4, 2, false, true)

#define PROJ_SKINNY_INST(MT, NT, WV, U, NTL, ROT) \
    template __global__ void skinny_kernel<MT, NT, WV, U, NTL, ROT>(Args, int);
PROJ_SKINNY_VARIANTS(PROJ_SKINNY_INST)

#ifndef __HIP_DEVICE_COMPILE__
template <int MT, int NT, int WAVES, int U, bool NTL, bool ROT>
static hipError_t launch_skinny(const Args &a, int S, hipStream_t st) {
    const int64_t tiles = (a.N + 16 * NT - 1) / (16 * NT);
    const int64_t grid = tiles * S;
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((skinny_kernel<MT, NT, WAVES, U, NTL, ROT>), dim3(static_cast<unsigned>(grid)),
                       dim3(WAVES * 64), 0, st, a, S);
    return hipGetLastError();
}

#define PROJ_SKINNY_ENTRY(MT, NT, WV, U, NTL, ROT) \
    {"skinny", MT, NT, WV, U, NTL, ROT, &launch_skinny<MT, NT, WV, U, NTL, ROT>},
const SkinnyVariant kSkinnyVariants[] = {PROJ_SKINNY_VARIANTS(PROJ_SKINNY_ENTRY)};
const int kNumSkinnyVariants = sizeof(kSkinnyVariants) / sizeof(kSkinnyVariants[0]);
#endif

}  // namespace proj
