// Registry of the compiled kernel instantiations (host side).
#pragma once
#include <hip/hip_runtime.h>
#include "gemm_kernel.hpp"

namespace gf {

struct GemmDesc {
    int bm, bn, bk, stages, threads, sched;
    bool core;
};

constexpr GemmDesc kGemmConfigs[] = {
#define GF_GEMM(BM, BN, BK, S, T, SCHED, CORE) {BM, BN, BK, S, T, SCHED, CORE != 0},
#include "gemm_configs.def"
#undef GF_GEMM
};
constexpr int kNumGemm = sizeof(kGemmConfigs) / sizeof(kGemmConfigs[0]);

struct GemvDesc {
    int rows, unroll, waves;
};

constexpr GemvDesc kGemvConfigs[] = {
#define GF_GEMV(R, U, W) {R, U, W},
#include "gemv_configs.def"
#undef GF_GEMV
};
constexpr int kNumGemv = sizeof(kGemvConfigs) / sizeof(kGemvConfigs[0]);

typedef hipError_t (*GemmLaunchFn)(const GemmArgs&, int slices, hipStream_t);
typedef hipError_t (*GemvLaunchFn)(const uint16_t*, const uint16_t*, uint16_t*, int, int, int,
                                   hipStream_t);

// [config][epilogue * 2 + aligned]; nullptr = not compiled.
extern GemmLaunchFn g_gemm_table[kNumGemm][6];
// fp16 GEMMs with other operand layouts: [config][a_kmajor * 2 + b_kmajor][aligned]
// (index 0, both operands K-contiguous, lives in g_gemm_table).
extern GemmLaunchFn g_gemm_layout_table[kNumGemm][4][2];

// Configs that also carry the layout variants: one wave per SIMD, 64-deep K
// tiles, M and N tiles a multiple of 128 (the K-major tile swizzle needs 16
// chunks per k-row).
constexpr bool has_layouts(const GemmDesc& d)
{
    return d.sched == 2 && d.bk == 64 && d.bm % 128 == 0 && d.bn % 128 == 0;
}
// [config][aligned]
extern GemvLaunchFn g_gemv_table[kNumGemv][2];

// Instantiation shards (one object file each, compiled in parallel).
constexpr int kGemmShards = 8;

}  // namespace gf
