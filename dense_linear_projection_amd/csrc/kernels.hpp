// kernels.hpp -- the table of compiled kernel variants the planner chooses
// from.  Each variant is one template instantiation with its launcher.
#pragma once

#include "common.hpp"

namespace proj {

// Weight-streaming split-K kernel for small M (skinny.hip).
struct SkinnyVariant {
    const char *family;
    int mt, nt, waves, unroll;
    bool nontemporal;
    hipError_t (*launch)(const Args &, int splits, hipStream_t);
};
extern const SkinnyVariant kSkinnyVariants[];
extern const int kNumSkinnyVariants;

// LDS-pipelined MFMA GEMM for large M (gemm.hip).
struct GemmVariant {
    const char *family;
    int bm, bn, bk, waves_m, waves_n;
    hipError_t (*launch)(const Args &, hipStream_t);
    hipError_t (*prepare)();  // one-time function attributes (LDS size)
};
extern const GemmVariant kGemmVariants[];
extern const int kNumGemmVariants;

// Any shape, any alignment (generic.hip).
hipError_t launch_generic(const Args &a, hipStream_t st);

}  // namespace proj
