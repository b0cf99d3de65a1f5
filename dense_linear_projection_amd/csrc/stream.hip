// stream.hip -- weight-streaming projection for few token rows, staged
// through an LDS ring filled by global->LDS DMA.
//
// At small M each weight is used by only M token rows, so the projection is
// bound by reading W once (worklog "How I made Muse's GPU projections 1.32x
// faster in the Open Kernel Challenge", section "A rough way to ask how much
// room was left": M flops per weight byte).  What matters is keeping enough
// W bytes in flight on every CU, reading them in long contiguous runs, and
// doing the little arithmetic on the side.
//
// Decomposition:
//   * a workgroup owns 16*MT token rows (one of ceil(M / 16*MT) row blocks;
//     the row block is the slowest-varying part of the workgroup index),
//     16*NT output features (W rows) and one of S
//     contiguous ranges of K, cut at KC-element stage boundaries as evenly
//     as integers allow (stages floor(s*T/S) .. floor((s+1)*T/S)); with S > 1
//     each range writes an fp32 partial tile and a second kernel adds the S
//     partials in split order and applies the epilogue (the worklog's
//     split-K with a partial workspace, section "My first useful win: split
//     up the sum");
//   * a stage is W[16*NT rows][KC] plus X[16*MT rows][KC], copied into one
//     slot of a D-deep LDS ring with global_load_lds_dwordx4: one wave
//     instruction moves 1 KB made of whole rows' KC-element runs, so every
//     row segment read from HBM is 2*KC contiguous bytes;
//   * the waves of the workgroup share the copies, wait for their own
//     copies with an explicit vmcnt, and meet at one barrier per stage; the
//     barrier publishes stage i and frees the slot of stage i-1, which is
//     refilled with stage i+D-1 right away, so D-1 stages stay in flight;
//   * in a stage, wave w multiplies k-steps w, w+WAVES, ... (32 k each) for
//     all of its tile with v_mfma_f32_16x16x32_bf16 (A = 16 token rows x 32 k
//     of X, B = 32 k x 16 features of W, both read from LDS), accumulating
//     fp32; the waves' partial tiles are summed through LDS at the end;
//   * LDS rows hold 16-byte chunks at position chunk ^ (row & 15), so the 16
//     rows read by one fragment load fall on distinct banks; the DMA writes
//     lane i to position i, so the XOR picks each lane's global source;
//   * optionally (WNT) the W copies carry the non-temporal cache hint: W is
//     read once, and streaming it past L2 keeps the X rows, which every
//     workgroup re-reads, resident there (it pays when X is large, M = 64);
//   * with S > 1 and fp32 output the partials may instead be added straight
//     into Y with fp32 atomics (a.atomic), Y having been zeroed by a small
//     kernel first, the bias added by split 0 only: no workspace and no
//     second pass over it (the worklog's atomic accumulation, section "Could
//     I avoid reading all those router partials back?"); the order of the
//     additions then varies from run to run, so the result is correct within
//     rounding, not bit-reproducible, unless every sum is exact;
//   * workgroups walk their stages starting at a tile-dependent rotation
//     (stage s t mod T for tile t, the stride s a planner choice:
//     Args::walk), so at any moment the machine's reads are spread over all
//     of K rather than all hitting the same column offset of every
//     power-of-two-strided row.
// Chunks past K or rows past M / N read the zero page (no load leaves the
// caller's buffers); rows past M / N are not stored.
//
// Packed weights (a.wpack == NT, FAST only): the tile's rows are stored as
// consecutive blocks of [16*NT rows][128 columns], one per 128-column step
// of K, so a stage of the tile is one contiguous run of 16*NT*KC*2 bytes
// instead of 16*NT row pieces 2K bytes apart.  Only the copy offsets change.
//
// FAST (chosen per call when K is a multiple of KC): the copies go through
// buffer resources over the tile's W rows and over X, with the per-lane
// offsets fixed for the whole loop and the stage's k offset a scalar, so a
// copy is one instruction with no vector arithmetic; rows past N or M read
// as zero from the resource bounds, and stages past the end are still
// issued through an empty resource, so every stage waits for the same vmcnt
// with no branch (the general path spends most of a stage on per-lane
// address arithmetic and on picking the wait).
#include "common.hpp"
#include "kernels.hpp"

namespace proj {

// wait until at most `ahead` stages of PERW copies are still in flight
template <int PERW, int MAXAHEAD>
__device__ __forceinline__ void wait_stages(int ahead) {
    if constexpr (MAXAHEAD <= 0) {
        wait_vm<0>();
    } else {
        if (ahead >= MAXAHEAD)
            wait_vm<PERW * MAXAHEAD>();
        else
            wait_stages<PERW, MAXAHEAD - 1>(ahead);
    }
}

template <int MT, int NT, int WAVES, int KC, int D>
struct StreamCfg {
    static constexpr int NR = 16 * NT;               // W rows per workgroup
    static constexpr int MR = 16 * MT;               // X rows (padded to 16s)
    static constexpr int ROWB = KC * 2;              // bytes per row per stage
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWB;          // rows per DMA instruction
    static constexpr int STAGE = (NR + MR) * ROWB;   // bytes per stage
    static constexpr int NINSTR = STAGE / 1024;
    static constexpr int PERW = NINSTR / WAVES;      // DMA instructions per wave per stage
    static constexpr int KS = KC / 32;               // k-steps per stage
    static constexpr int RED = WAVES * MT * NT * 1024;  // reduction scratch bytes
    static constexpr int LDS = (D * STAGE > RED) ? D * STAGE : RED;
    static_assert(ROWB <= 1024 && 1024 % ROWB == 0, "a DMA block holds whole row runs");
    static_assert(CPR >= 16, "swizzle spans 16 chunks");
    static_assert(NINSTR % WAVES == 0, "copies divide evenly over the waves");
    static_assert(KS % WAVES == 0 || WAVES % KS == 0, "k-steps divide over the waves");
    static_assert(KS >= WAVES, "every wave gets a k-step per stage");
    static_assert(PERW * (D - 2) <= 63, "vmcnt range");
    static_assert(D >= 2, "ring depth");
};

template <int MT, int NT, int WAVES, int KC, int D, int WNT, bool FAST>
__global__ __launch_bounds__(WAVES * 64) void stream_kernel(Args a, int S) {
    using C = StreamCfg<MT, NT, WAVES, KC, D>;
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t K = a.K, N = a.N;
    // Workgroup coordinates in 32-bit arithmetic, with no division at all
    // for one row block and S = 1: this runs before the first copy is
    // issued, and a 64-bit division by a runtime value is a sequence of
    // over a hundred scalar instructions.  The launcher keeps the grid
    // (row blocks x tiles x S) below 2^31 and, for S > 1, the stage count
    // times S below 2^32.
    const uint32_t us = static_cast<uint32_t>(S);
    uint32_t mbu = 0, rest = blockIdx.x;
    if (a.M > C::MR) {
        const uint32_t tS = static_cast<uint32_t>((N + C::NR - 1) / C::NR) * us;
        mbu = rest / tS;
        rest -= mbu * tS;
    }
    uint32_t tile_u = rest, split_u = 0;
    if (us > 1) {
        tile_u = rest / us;
        split_u = rest - tile_u * us;
    }
    const int tile = static_cast<int>(tile_u), split = static_cast<int>(split_u);
    const int64_t n0 = static_cast<int64_t>(tile) * C::NR;
    // this workgroup's token rows: m0 .. m0 + M - 1 (M counted from m0)
    const int64_t m0 = static_cast<int64_t>(mbu) * C::MR;
    const int64_t M = (a.M - m0) < C::MR ? (a.M - m0) : C::MR;
    const uint16_t *X = a.X + m0 * a.kx;

    // stage range of this split, and the rotated walk over it
    const int64_t T = (K + KC - 1) / KC;
    int64_t sb = 0, se = T;
    if (us > 1) {
        const uint32_t t32 = static_cast<uint32_t>(T);
        sb = (t32 * split_u) / us;
        se = (t32 * (split_u + 1)) / us;
    }
    const int nst = static_cast<int>(se - sb);
    // start of the walk: stage (walk stride x tile) mod T, the stride a
    // planner choice (Args::walk; 0 means 7).  Which stride keeps the memory
    // channels busiest depends on the shape and the W layout: on one box,
    // stride 7 ran M16 N8192 at 21.7 us against 26.9 with stride 1, and
    // stride 1 ran M64 N28672 at 78.5 us against 86.3 with stride 7.
    const uint32_t stride = a.walk > 0 ? static_cast<uint32_t>(a.walk) : 7u;
    const int rot = nst > 0 ? static_cast<int>((tile_u * stride) % static_cast<uint32_t>(nst)) : 0;
    auto stage_k0 = [&](int i) -> int64_t {
        int q = i + rot;
        if (q >= nst) q -= nst;
        return (sb + q) * KC;
    };

    // per-lane DMA sources: instruction j of this wave fills block
    // b = wave + j*WAVES of the stage, rows b*RPI + lane/CPR, position
    // lane%CPR, which holds chunk (lane%CPR) ^ (row & 15).
    const uint16_t *src[C::PERW];
    int kofs[C::PERW];
#pragma unroll
    for (int j = 0; j < C::PERW; ++j) {
        const int row = (wave + j * WAVES) * C::RPI + lane / C::CPR;
        const int chunk = (lane % C::CPR) ^ (row & 15);
        kofs[j] = chunk * 8;
        if (row < C::NR) {
            const int64_t n = n0 + row;
            src[j] = n < N ? a.W + n * K + chunk * 8 : nullptr;
        } else {
            const int64_t m = row - C::NR;
            src[j] = m < M ? X + m * K + chunk * 8 : nullptr;
        }
    }
    // FAST: resources over the tile's valid W rows and over X, and each
    // copy's byte offset within its operand
    uint32_t wbytes = 0, xbytes = 0;
    uint32_t voff[C::PERW];
    const bool packed = a.wpack != 0;
    if constexpr (FAST) {
        // a packed tile is whole: rows past N are zeros in the packed array
        const int64_t rows_w = packed ? C::NR : (N - n0) < C::NR ? (N - n0) : C::NR;
        wbytes = static_cast<uint32_t>(rows_w * K * 2);
        xbytes = static_cast<uint32_t>(M * a.kx * 2);
#pragma unroll
        for (int j = 0; j < C::PERW; ++j) {
            const int row = (wave + j * WAVES) * C::RPI + lane / C::CPR;
            const int chunk = (lane % C::CPR) ^ (row & 15);
            // W rows are K long (packed: chunk c of a row sits in 128-column
            // block c / 16 of the stage), X rows kx long
            // 32-bit: the tile's W rows and the X rows span less than 4 GiB
            // on this path
            const uint32_t wofs = packed ? (chunk / 16) * C::NR * 128 + row * 128 + (chunk % 16) * 8
                                         : static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + chunk * 8;
            voff[j] = row < C::NR ? wofs * 2
                                  : (static_cast<uint32_t>(row - C::NR) * static_cast<uint32_t>(a.kx) + chunk * 8) * 2;
        }
    }
    auto issue = [&](int i) {
        char *slot = lds + (i % D) * C::STAGE;
        if constexpr (FAST) {
            const bool live = i < nst;
            const int64_t k0 = stage_k0(live ? i : 0);
            const uint32_t soff = static_cast<uint32_t>(k0 * 2 * (packed ? C::NR : 1));
            // X column of a hi/lo pair's second half wraps to the start
            const uint32_t soffx = static_cast<uint32_t>((k0 >= a.kx ? k0 - a.kx : k0) * 2);
            const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.W + n0 * K, live ? wbytes : 0u);
            const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(X, live ? xbytes : 0u);
#pragma unroll
            for (int j = 0; j < C::PERW; ++j) {
                const bool is_w = (wave + j * WAVES) * C::RPI < C::NR;  // wave-uniform
                const __amdgpu_buffer_rsrc_t r = is_w ? rw : rx;
                char *to = slot + (wave + j * WAVES) * 1024;
                if (WNT && is_w)
                    dma16_buf_nt(r, voff[j], soff, to);
                else
                    dma16_buf(r, voff[j], is_w ? soff : soffx, to);
            }
        } else {
            const int64_t k0 = i < nst ? stage_k0(i) : 0;
#pragma unroll
            for (int j = 0; j < C::PERW; ++j) {
                const bool ok = i < nst && src[j] != nullptr && k0 + kofs[j] < K;
                const void *from = ok ? static_cast<const void *>(src[j] + k0) : static_cast<const void *>(a.zeros);
                char *to = slot + (wave + j * WAVES) * 1024;
                if (WNT && (wave + j * WAVES) * C::RPI < C::NR)
                    dma16_nt(from, to);  // a block of W rows (wave-uniform branch)
                else
                    dma16(from, to);
            }
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fg = lane >> 4;
    // Bias bits of the outputs this thread finishes in the epilogue (S = 1;
    // split 0 of an atomic split adds the bias in the epilogue as before),
    // loaded now, just ahead of the first copies, and converted only there:
    // the load latency then overlaps the stream instead of following it.
    // Issued behind the copies they would add to the first stage waits
    // (loads and stores complete in order), which measured 0.2 us later.
    // Features past N read zero through the resource bounds.  Only tiles
    // of at most 4 outputs per thread prefetch (the M = 16 decode tiles);
    // with more, the compiler's handling of the loaded values (a
    // zero-extension per value) waits for them right away.
    constexpr int E = MT * NT * 256;
    constexpr int QN = (E + WAVES * 64 - 1) / (WAVES * 64);
    constexpr bool PREFETCH = QN <= 4;
    uint32_t braw[QN];  // one 32-bit register each: packing two would wait for both loads
    if (PREFETCH && S == 1 && (a.epi & 1)) {
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(a.bias, (a.epi & 1) ? static_cast<uint32_t>(N * 2) : 0u);
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int e = tid + q * WAVES * 64;
            const int tl = e >> 8, ln = e & 63;
            const int64_t n = n0 + (tl % NT) * 16 + (ln & 15);
            braw[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, e < E ? static_cast<int>(n * 2) : -1, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(i);

    for (int i = 0; i < nst; ++i) {
        // this wave's copies of stage i are done once at most
        // min(D-2, nst-1-i) later stages are still in flight (FAST: always
        // D-2, copies past the end being issued too)
        if constexpr (FAST)
            wait_vm<C::PERW * (D - 2)>();
        else
            wait_stages<C::PERW, D - 2>(nst - 1 - i);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (FAST || i + D - 1 < nst) issue(i + D - 1);
        const char *slot = lds + (i % D) * C::STAGE;
#pragma unroll
        for (int kk = wave % C::KS; kk < C::KS; kk += WAVES) {
            const int c = kk * 4 + fg;
            bf16x8 xf[MT], wf[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = C::NR + mt * 16 + fr;
                xf[mt] = *reinterpret_cast<const bf16x8 *>(slot + row * C::ROWB + ((c ^ (row & 15)) << 4));
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = nt * 16 + fr;
                wf[nt] = *reinterpret_cast<const bf16x8 *>(slot + row * C::ROWB + ((c ^ (row & 15)) << 4));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(xf[mt], wf[nt], acc[mt][nt]);
        }
    }
    wait_vm<0>();
    __syncthreads();

    // ---- sum the waves' partial tiles: red[wave][tile][i][lane]
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave * E + (mt * NT + nt) * 256 + r * 64 + lane] = acc[mt][nt][r];
    __syncthreads();

    const uint16_t *bias = a.bias;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
        const int e = tid + q * WAVES * 64;
        if (e >= E) break;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w * E + e];
        // MFMA output layout: lane holds column lane%16, rows 4*(lane/16) + r
        const int tl = e >> 8, r = (e >> 6) & 3, ln = e & 63;
        const int64_t m = (tl / NT) * 16 + 4 * (ln >> 4) + r;
        const int64_t n = n0 + (tl % NT) * 16 + (ln & 15);
        if (m >= M || n >= N) continue;
        if (S == 1) {
            float b = 0.f;
            if (a.epi & 1) {
                if constexpr (PREFETCH) {
                    // the empty asm keeps the conversion (and the compiler's
                    // wait for the load) here rather than hoisted up to it
                    uint32_t bits = braw[q];
                    asm volatile("" : "+v"(bits));
                    b = bf16_bits_to_f32(bits);
                } else {
                    b = bf16_bits_to_f32(bias[n]);
                }
            }
            store_out(a.Y, a.out, (m0 + m) * N + n, apply_epilogue(s, a.epi, b));
        } else if (a.atomic) {
            const float b = (split == 0 && (a.epi & 1)) ? bf16_bits_to_f32(bias[n]) : 0.f;
            unsafeAtomicAdd(static_cast<float *>(a.Y) + (m0 + m) * N + n, s + b);
        } else {
            a.ws[(static_cast<int64_t>(split) * a.M + m0 + m) * N + n] = s;
        }
    }
}

// Second pass of split-K: Y[m, n] = epilogue(sum over s of ws[s, m, n]),
// summed in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(Args a, int S) {
    const int64_t MN = a.M * a.N;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= MN) return;
    float s = 0.f;
    for (int sp = 0; sp < S; ++sp) s += a.ws[sp * MN + idx];
    float b = 0.f;
    if (a.epi & 1) {
        // the bias column; a 32-bit remainder where the output allows (the
        // 64-bit one is a long instruction sequence per thread)
        const int64_t n = MN < (int64_t{1} << 32) ? static_cast<int64_t>(static_cast<uint32_t>(idx) %
                                                                          static_cast<uint32_t>(a.N))
                                                  : idx % a.N;
        b = bf16_bits_to_f32(a.bias[n]);
    }
    store_out(a.Y, a.out, idx, apply_epilogue(s, a.epi, b));
}

// Y = 0 before the atomic split-K accumulation (a kernel rather than a
// memset, so that a captured graph replays it as an ordinary kernel node).
__global__ __launch_bounds__(256) void zero_f32_kernel(float *y, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        y[i] = 0.f;
}

// ---------------------------------------------------------------- registry
#define PROJ_STREAM_VARIANTS(X)                                                                           \
    X(1, 1, 8, 256, 4, 0) X(1, 2, 8, 256, 4, 0) X(1, 2, 8, 256, 3, 0) X(1, 4, 8, 256, 3, 0)                \
    X(1, 1, 4, 128, 9, 0) X(1, 1, 4, 128, 6, 0) X(1, 2, 4, 128, 5, 0) X(1, 2, 4, 128, 7, 0)                \
    X(1, 2, 2, 128, 5, 0) X(1, 4, 4, 128, 4, 0) X(1, 4, 4, 128, 3, 0)                                      \
    X(2, 2, 8, 256, 4, 0) X(2, 2, 4, 128, 5, 0) X(2, 4, 4, 128, 4, 0)                                      \
    X(4, 2, 8, 256, 3, 0) X(4, 4, 8, 256, 2, 0) X(4, 4, 4, 128, 4, 0) X(4, 4, 4, 128, 5, 0)                \
    X(4, 2, 4, 128, 4, 0) X(4, 2, 4, 128, 6, 0) X(4, 7, 4, 128, 3, 0)                                      \
    X(1, 2, 4, 128, 5, 1) X(1, 1, 8, 256, 4, 1) X(2, 4, 4, 128, 4, 1)                                      \
    X(4, 7, 4, 128, 3, 1) X(4, 4, 4, 128, 4, 1) X(4, 2, 4, 128, 6, 1)                                      \
    X(1, 2, 4, 128, 4, 1) X(1, 2, 4, 128, 6, 1) X(1, 2, 4, 128, 7, 1) X(1, 1, 4, 128, 6, 1)                \
    X(1, 4, 4, 128, 4, 1) X(1, 2, 8, 256, 4, 1) X(1, 2, 8, 256, 3, 1) X(1, 1, 4, 128, 9, 1)                \
    X(8, 1, 4, 128, 4, 0) X(8, 2, 4, 128, 3, 0) X(8, 4, 4, 128, 3, 0)                                      \
    X(8, 1, 4, 128, 4, 1) X(8, 2, 4, 128, 3, 1) X(8, 4, 4, 128, 3, 1)

#define PROJ_STREAM_INST(MT, NT, WV, KC, D, WNT)                                  \
    template __global__ void stream_kernel<MT, NT, WV, KC, D, WNT, false>(Args, int); \
    template __global__ void stream_kernel<MT, NT, WV, KC, D, WNT, true>(Args, int);
PROJ_STREAM_VARIANTS(PROJ_STREAM_INST)

#ifndef __HIP_DEVICE_COMPILE__
template <int MT, int NT, int WV, int KC, int D, int WNT>
static hipError_t prepare_stream() {
    auto slow = stream_kernel<MT, NT, WV, KC, D, WNT, false>;
    auto fast = stream_kernel<MT, NT, WV, KC, D, WNT, true>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(slow), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       StreamCfg<MT, NT, WV, KC, D>::LDS);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fast), hipFuncAttributeMaxDynamicSharedMemorySize,
                               StreamCfg<MT, NT, WV, KC, D>::LDS);
}

template <int MT, int NT, int WV, int KC, int D, int WNT>
static hipError_t launch_stream(const Args &a, int S, hipStream_t st) {
    const int64_t tiles = (a.N + 16 * NT - 1) / (16 * NT);
    const int64_t mblocks = (a.M + 16 * MT - 1) / (16 * MT);
    const int64_t grid = mblocks * tiles * S;
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    // the kernel cuts the stage range of a split in 32-bit arithmetic
    if (S > 1 && ((a.K + KC - 1) / KC) * S >= (int64_t{1} << 32)) return hipErrorInvalidConfiguration;
    constexpr int lds_bytes = StreamCfg<MT, NT, WV, KC, D>::LDS;
    // the buffer-resource path needs whole stages and 32-bit operand offsets;
    // it is also the only one that reads a hi/lo pair's X (kx < K), whose
    // wrap must fall on a stage boundary
    const int64_t rows_x = a.M < 16 * MT ? a.M : 16 * MT;  // X rows one workgroup addresses
    // atomic accumulation: split K, fp32 output, no GELU (it is not additive)
    if (a.atomic && (S < 2 || a.out != OUT_F32 || (a.epi & 2))) return hipErrorInvalidValue;
    const bool fast = a.K % KC == 0 && a.kx % KC == 0 && rows_x * a.kx * 2 < (int64_t{1} << 32) &&
                      16 * NT * a.K * 2 < (int64_t{1} << 32);
    if (!fast && a.kx != a.K) return hipErrorInvalidValue;
    if (a.wpack && (a.wpack != NT || !fast || KC % 128 != 0)) return hipErrorInvalidValue;
    if (a.atomic) {
        const int64_t n = a.M * a.N;
        const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
        hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                           static_cast<float *>(a.Y), n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (fast)
        hipLaunchKernelGGL((stream_kernel<MT, NT, WV, KC, D, WNT, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(WV * 64), lds_bytes, st, a, S);
    else
        hipLaunchKernelGGL((stream_kernel<MT, NT, WV, KC, D, WNT, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(WV * 64), lds_bytes, st, a, S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1 || a.atomic) return e;
    return launch_splitk_reduce(a, S, st);
}

hipError_t launch_splitk_reduce(const Args &a, int S, hipStream_t st) {
    const int64_t blocks = (a.M * a.N + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a, S);
    return hipGetLastError();
}

#define PROJ_STREAM_ENTRY(MT, NT, WV, KC, D, WNT) \
    {"stream", MT, NT, WV, KC, D, WNT, &launch_stream<MT, NT, WV, KC, D, WNT>, &prepare_stream<MT, NT, WV, KC, D, WNT>},
const StreamVariant kStreamVariants[] = {PROJ_STREAM_VARIANTS(PROJ_STREAM_ENTRY)};
const int kNumStreamVariants = sizeof(kStreamVariants) / sizeof(kStreamVariants[0]);
#endif

}  // namespace proj
