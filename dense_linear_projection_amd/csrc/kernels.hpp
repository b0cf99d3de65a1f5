// kernels.hpp -- the table of compiled kernel variants the planner chooses
// from.  Each variant is one template instantiation with its launcher.
#pragma once

#include "common.hpp"

namespace proj {

// Weight-streaming kernel staged through an LDS ring (stream.hip); with
// splits > 1 a second kernel adds the partials and applies the epilogue.
struct StreamVariant {
    const char *family;
    int mt, nt, waves, kc, depth;
    int wnt;  // W copies carry the non-temporal (streaming) cache hint
    hipError_t (*launch)(const Args &, int splits, hipStream_t);
    hipError_t (*prepare)();  // one-time function attributes (LDS size)
};
extern const StreamVariant kStreamVariants[];
extern const int kNumStreamVariants;

// LDS-pipelined MFMA GEMM for large M (gemm.hip).
struct GemmVariant {
    const char *family;
    int bm, bn, bk, kmult, waves_m, waves_n, group_m;  // kmult: K must be a multiple of it
    int64_t kmax;  // largest K the kernel addresses (0: no limit)
    int max_splits;  // largest K split count (1: the kernel does not split K)
    hipError_t (*launch)(const Args &, int splits, hipStream_t);
    hipError_t (*prepare)();  // one-time function attributes (LDS size)
};
extern const GemmVariant kGemmVariants[];
extern const int kNumGemmVariants;

// Few token rows (M <= mr), W rows streamed into registers (gemv.hip).
struct GemvVariant {
    const char *family;
    int mr, rows, waves, unroll;  // token rows, W rows per workgroup, waves, chunks per row per iteration
    int wnt;                      // W loads carry the non-temporal hint
    hipError_t (*launch)(const Args &, int splits, hipStream_t);
};
extern const GemvVariant kGemvVariants[];
extern const int kNumGemvVariants;

// Second pass of split-K (stream.hip): Y = epilogue(sum over the S fp32
// partials in a.ws, in split order).
hipError_t launch_splitk_reduce(const Args &a, int S, hipStream_t st);

// Any shape, any alignment (generic.hip).
hipError_t launch_generic(const Args &a, hipStream_t st);

// bf16 weights [N][K] -> tiles of R rows stored as [K/128][R][128] blocks,
// rows past N zero (generic.hip).
hipError_t launch_pack(const uint16_t *W, int64_t N, int64_t K, int R, uint16_t *Wp, hipStream_t st);

// fp32 weights [N][K] -> bf16 hi/lo pair [N][2K] (generic.hip).
hipError_t launch_hilo_split(const float *W, int64_t N, int64_t K, uint16_t *out, hipStream_t st);

// Read `bytes` of `buf` to evict other data from the caches (generic.hip);
// `sink` needs room for 256 unsigned.
hipError_t launch_flush(const void *buf, size_t bytes, unsigned *sink, hipStream_t st);

// Plain streaming read of the first bytes/16 16-byte chunks of `buf`
// (generic.hip); `sink` needs room for 256 unsigned.
hipError_t launch_read_probe(const void *buf, size_t bytes, unsigned *sink, hipStream_t st);

}  // namespace proj
