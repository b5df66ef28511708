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

// Skinny GEMM launch shapes.  stages = 0: direct form (blocks = 16-row
// blocks of B per workgroup, unroll = k-steps per register batch, two batches
// in flight per wave).  stages >= 2: LDS-staged form (blocks as above, that
// many 512-k chunks in the ring, unroll unused, 0).  stages = 1: vector form
// for M <= 8 (blocks = rows of B per wave, unroll = 16-byte chunks per row
// and lane per step).  stages = -1: split form for M <= 8 and K = 512 *
// unroll * waves (blocks = workgroups at most, unroll = 16-byte chunks per
// lane and row).  waves: waves per workgroup.
struct SkinnyDesc {
    int blocks, unroll, waves, stages;
};

constexpr SkinnyDesc kSkinnyConfigs[] = {
    {1, 1, 8, 0},  {1, 2, 8, 0},  {1, 4, 8, 0},  {2, 1, 8, 0},  {2, 2, 8, 0},  {2, 4, 8, 0},
    {1, 1, 16, 0}, {1, 2, 16, 0}, {1, 4, 16, 0}, {2, 1, 16, 0}, {2, 2, 16, 0}, {4, 1, 8, 0},
    {1, 0, 8, 2},  {1, 0, 8, 3},  {1, 0, 8, 4},  {1, 0, 4, 4},  {1, 0, 16, 4}, {2, 0, 8, 2},
    {2, 0, 8, 3},  {2, 0, 4, 3},  {3, 0, 8, 2},  {1, 0, 4, 3},
    {1, 4, 8, 1},  {2, 2, 8, 1},  {2, 4, 8, 1},  {4, 2, 8, 1},  {2, 2, 16, 1}, {4, 1, 8, 1},
    {1, 8, 8, 1},  {1, 4, 16, 1}, {1, 4, 4, 1},  {1, 2, 8, 1},  {1, 8, 4, 1},
    {512, 4, 4, -1}, {512, 8, 2, -1}, {512, 8, 4, -1}, {256, 8, 4, -1}, {256, 4, 8, -1},
};
constexpr int kNumSkinny = sizeof(kSkinnyConfigs) / sizeof(kSkinnyConfigs[0]);

typedef hipError_t (*GemmLaunchFn)(const GemmArgs&, int slices, hipStream_t);
typedef hipError_t (*SkinnyLaunchFn)(const uint16_t*, const uint16_t*, uint16_t*, int, int, int,
                                     hipStream_t);
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
// [config]; fast path only (K % 8 == 0, or K % 512 == 0 for the LDS-staged
// form, and 16-byte aligned A and B)
extern SkinnyLaunchFn g_skinny_table[kNumSkinny];

// Instantiation shards (one object file each, compiled in parallel).
constexpr int kGemmShards = 8;

}  // namespace gf
